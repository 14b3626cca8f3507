// deco_internal.h - layer object, workspace layout and kernel launchers (host side).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "deco_moe.h"

// offsets (bytes from the prefill/backward workspace's base) of its buffers
struct PwsOff {
  size_t to, ec, lt, sb, yb, sr, dg, dh, ag, sl, dc, dz, dl, gb, cp, wp, dhl, agl, dcl, sbh, sbl, hp, wp2;
};

struct deco_moe_layer {
  deco_moe_config cfg;
  int device;
  int d, E, F, Fs, maxT;
  int esz;                 // bytes per element (2 bf16, 4 fp32)
  int KB;                  // k per fragment (32 bf16, 16 fp32)
  int nkb_d, nkb_F, nkb_Fs;
  int pR;                  // router panels (E padded to a multiple of 64, /16)
  int pF, pD, pFs;         // 16-column panels of F, d, Fs
  int W;                   // mask words per token = ceil(E/64)
  // decode launch plan (plan_decode_sizes, plan_decode)
  int dec_np;              // 16-column panels per up-kernel slice
  int dec_S;               // column slices per routed expert
  int dec_n_shs, dec_nsub, dec_n_sh;   // shared slices, slices per shared workgroup, shared workgroups
  int dec_grid_up;
  int dec_Fp, dec_Fsp;     // F, Fs padded to whole column-pair fragments (2 k-blocks)
  int dec_kpe, dec_kps;    // column-pair fragments per routed expert / of the shared expert, per 8 columns
  int dec_ok;              // the decode path is available for this layer
  int last_path;           // path of the most recent forward (DECO_PATH_DECODE or _PREFILL)
  int pre_grid;            // persistent grid of the prefill expert kernel
  int n_cu;                // compute units of the device
  int bwd_grid;            // persistent grid of the backward expert kernel
  hipStream_t bwd_side[2]; // backward: two more streams for branches that run beside the caller's
                           // stream (default priority), and their fork/join events
  hipEvent_t bwd_ev[6];
  int gated;               // gated routed experts: NormSiLU(x.W_gate[e]) * (x.W_up[e])

  // packed weights (one allocation)
  char* wmem;
  size_t wmem_bytes;
  char* Wr_p;              // router  [pR][nkb_d] frags
  char* Wup_p;             // per expert [pF][nkb_d] frags of the NormSiLU input projection
                           // (W_up[e]; W_gate[e] for gated experts)
  char* Wlin_p;            // gated experts: per expert [pF][nkb_d] frags of W_up[e]; else null
  char* Wupm_p;            // per expert [pF][nkb_d] frags of Wup - Wbar (the decode path's NormSiLU
                           // input with the mean term folded in); null with the mean-term ablation
  char* Wbar_p;            // [pF][nkb_d] frags of Wbar, the mean of the Wup_p matrices (layer dtype)
  char* Wdn_p;             // per expert [pD][nkb_F] frags
  char* Wdn16_p;           // bf16 layers: W_down again, in fp16 (prefill); fp32 layers: = Wdn_p
  char* Wsu_p;             // [pFs][nkb_d]
  char* Wsd_p;             // [pD][nkb_Fs]
  char* Wdn8_p;            // per expert [d/8][dec_kpe] column-pair frags of W_down[e] (down operand type)
  char* Wsd8_p;            // [d/8][dec_kps] column-pair frags of Ws_down (layer dtype)
  size_t up_stride, dn_stride;   // bytes per expert
  size_t dn8_stride;       // bytes per expert of Wdn8_p
  float* b_r;
  float* lam;
  float* wbar;             // [d][F] fp32
  // backward (cfg.backward = 1; null otherwise)
  int Fp, Ep, Fsp;         // F, E, Fs rounded up to 64: sections of the dense backward operand
  int nkb_cat;             // k-blocks of Fp + Ep + Fsp
  char* WdnT_p;            // per expert [pF][nkb_d] frags of W_down[e]^T (K = d, N = F), layer dtype
  char* WupT_p;            // per expert [pD][nkb_F] frags of W_up[e]^T (K = F, N = d), down operand type
  char* WsdT_p;            // [pFs][nkb_d] frags of Ws_down^T (K = d, N = Fs)
  char* Bcat_p;            // [pD][nkb_cat] frags of [Wbar^T; W_r^T; Ws_up^T] (K = Fp + Ep + Fsp, N = d)
  char* WbarLo_p;          // bf16 layers: [pF][nkb_d] frags of Wbar - bf16(Wbar)

  // workspace (one allocation, sized for max(maxT, 16) tokens)
  char* ws;
  size_t ws_bytes;
  float* z;                // [Tcap][E] router logits
  float* g;                // [Tcap][E] gates
  uint64_t* mask;          // [Tcap][W]
  // decode
  float* mbuf;             // [Tcap][F]    x . Wbar (NormSiLU mean term; decode: rows 0..15)
  unsigned* rflag;         // [E] routing of the last decode call (1 no token, 2 some token routed to e)
  unsigned* dec_err;       // [1] device-side error flags (bit 0: a decode hand-off wait timed out)
  unsigned char* act8;     // [16][E] routing decisions of the last decode call
  char* pws;               // prefill/backward workspace (its own, or the device's shared one)
  size_t pws_bytes;
  int pws_shared;
  PwsOff pwo;
  void* hwords;            // [n_hwords] 64-bit decode hand-off words (epoch | value)
  int n_hwords;
  unsigned* dec_ctr;       // decode call counter (the up kernel's epoch is 1 + its value)
  char* arow;              // [E][16][dec_Fp] routed activations (down operand type)
  char* srow;              // [16][dec_Fsp] shared activations (layer dtype)
  // prefill
  int* tok_off;            // [Tcap + 1]
  int* ecnt;               // [E]
  int* list_tok;           // [E][Tcap]
  char* sbuf;              // [Tcap][Fs] shared activations (dtype)
  // backward workspace
  float* dgbuf;            // [Tcap][E] dLoss/dg of the active pairs
  char* dhbuf;             // [pair slots][F] dLoss/dh~ of each pair (layer dtype; bf16: high part)
  char* agbuf;             // [pair slots][F] g * a of each pair (likewise)
  char* dhbuf_lo;          // bf16 layers: low parts (v - high part) of dhbuf, agbuf, dcat; else null
  char* agbuf_lo;
  char* dcat_lo;
  char* sb_hi;             // [Tcap][Fs] s = SiLU(x Ws_up) recomputed in fp32 (bf16 layers: high part)
  char* sb_lo;             // bf16 layers: its low part
  int* slot_list;          // [E][Tcap] pair slot of each entry of an expert's token list
  char* dcat;              // [Tcap][Fp + Ep + Fsp] rows dm | dz | du_s (layer dtype)
  float* dzbuf;            // [Tcap][E] dLoss/dz
  float* dlz;              // [Tcap][E] ReLU(z) * dLoss/dg
  float* gbuf;             // [d][F] x^T dm (gradient of Wbar)
  float* colpart;          // [2][ceil(Tcap / 64)][E] partial column sums (db_r, dlambda)
  float* wpart;            // [4][d * (Fp + Ep + Fsp)] partial weight-gradient tiles of x^T [dm | dz | du_s]
  float* wpart2;           // [4][Fs * d] those of s^T dout (the two jobs run on different streams)
  float* sraw;             // shared_rms: [Tcap][Fs] x . Ws_up before the RMS-only NormSiLU (fp32)
  float* hpart;            // [SPLIT_NKS][split_maxT * (E + 1)][F] K-part sums of x . W_up[e] per
                           // pair slot (small-batch prefill), or null
  int split_maxT;          // largest batch the small-batch prefill split is sized for (0: none)
  char* ybuf;              // [Tcap * (E + 1) + 1][d] pair buffer, token-major: per token its
                           // shared-expert output, then gate * expert output for each
                           // active expert in ascending order (fp16 for bf16 layers,
                           // fp32 for fp32 layers); the last row is scratch
};

namespace deco_host {

// Per-kernel timing: when enabled, returns a start/stop event pair that the
// launch itself records (hipExtLaunchKernel stamps the kernel's own dispatch,
// so the elapsed time matches a profiler's kernel duration); else nulls.
void timing_events(int slot, hipEvent_t* start, hipEvent_t* stop);

template <typename... KArgs, typename... Args>
inline hipError_t launch(int slot, void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t s,
                         Args... args) {
  hipEvent_t a = nullptr, b = nullptr;
  timing_events(slot, &a, &b);
  hipExtLaunchKernelGGL(kernel, grid, block, 0, s, a, b, 0, static_cast<KArgs>(args)...);
  return hipGetLastError();
}

// kernel slots for timing
enum {
  KS_PACK = 0,
  KS_DEC_UP,
  KS_DEC_DOWN,
  KS_PRE_TOPK,
  KS_PRE_ROUTER_SHARED,
  KS_PRE_DISPATCH,
  KS_PRE_EXPERT,
  KS_PRE_COMBINE,
  KS_BWD_SHARED,
  KS_BWD_EXPERT,
  KS_BWD_TOKEN,
  KS_BWD_COLSUM,
  KS_BWD_DENSE_DX,
  KS_BWD_COMBINE,
  KS_BWD_WGRAD,
  KS_PRE_DC,
  KS_PRE_UP_PART,
  KS_COUNT
};
const char* kernel_slot_name(int slot);

// launchers (return hipSuccess or the launch error)
// W_norm: the projection NormSiLU acts on (W_up, or W_gate for gated
// experts); W_lin: gated experts' W_up (null otherwise)
// bf16 layers: *ok = W_down fits fp16 (the prefill down-projection operand)
// and, with the mean term, max |W_norm| <= 32752 (the decode path's folded
// NormSiLU input W_norm - Wbar in fp16)
hipError_t check_down_range(deco_moe_layer* L, const void* W_down, const void* W_norm, hipStream_t s, bool* ok);
hipError_t launch_pack_all(deco_moe_layer* L, const void* W_r, const void* W_norm, const void* W_lin,
                           const void* W_down, const void* Ws_up, const void* Ws_down, hipStream_t s);
void plan_decode_sizes(deco_moe_layer* L, int n_cu);   // decode slices and buffer sizes (load time)
hipError_t plan_decode(deco_moe_layer* L);   // decode residency check (load time, after plan_prefill)
hipError_t plan_prefill(deco_moe_layer* L);  // prefill launch shape (load time)
hipError_t plan_backward(deco_moe_layer* L); // backward launch shape (load time, after plan_prefill)
hipError_t launch_decode(const deco_moe_layer* L, const void* x, int T, void* out, hipStream_t s);
// path: DECO_PATH_PREFILL (variant chosen here), _PAIRS or _TOKEN
hipError_t launch_prefill(const deco_moe_layer* L, const void* x, int T, void* out, hipStream_t s, int path);
bool prefill_token_ok(const deco_moe_layer* L);   // the token-major down-projection fits the layer
int split_max_tokens(const deco_moe_layer* L, long long grid);   // small-batch split: largest batch (load time)
constexpr int SPLIT_NKS_MAX = 4;                 // k parts of the small-batch split, at most
hipError_t launch_dec_mask(const deco_moe_layer* L, int T, uint64_t* mask, hipStream_t s);
// allocation-free decode (static device array as scratch)
size_t decode_scratch_bytes(const deco_moe_layer* L);
size_t decode_scratch_limit();
hipError_t launch_decode_scratch(const deco_moe_layer* L, const void* x, int T, void* out, hipStream_t s);
hipError_t launch_backward(const deco_moe_layer* L, const void* x, const void* dout, int T, float reg_coef,
                           const deco_moe_grads* gr, hipStream_t s);

}  // namespace deco_host
