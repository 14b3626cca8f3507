// prefill_kernels.h - device code of the bucketed large-batch path, shared
// by the forward launchers (prefill.hip) and the backward pass
// (backward.hip), which reuses the router, dispatch and expert-tile kernels.
// Included by exactly those two translation units; everything here has
// internal linkage.
//
//   k_pre_router_shared  one GEMM of x against the concatenated column panels
//                        [router | inter-expert mean Wbar | shared up-proj].
//                        Router epilogue: logits + b_r, gates lambda_e*ReLU(z)
//                        and active-expert bit masks (DECO paper Sec. 2
//                        "Router design"; zero or negative scores are ignored:
//                        qidianchuan.cn write-up, section 二, router).  Mean
//                        epilogue: m = x.Wbar in fp32 (the NormSiLU mean term,
//                        the same for every expert).  Shared epilogue: SiLU,
//                        stored for the shared down-projection.
//   k_pre_dispatch       per-expert token buckets ("expert batching") from a
//                        workgroup prefix scan: ascending token lists per
//                        expert, and per token the offset of its slots in a
//                        token-major pair buffer (slot 0: shared expert, then
//                        one slot per active expert in ascending order).
//   k_pre_expert         persistent grouped kernel.  Expert tiles (expert e,
//                        up to 128 of its tokens): gathered x rows . W_up[e] on
//                        MFMA, minus the mean term, NormSiLU (RMS over the F
//                        columns of a row, then SiLU), . W_down[e] in fp16,
//                        times the gate (DECO paper Sec. 2 "Router design": the
//                        router gives every expert a weight), stored in fp16
//                        to the pair slot.  Shared tiles: SiLU(x Ws_up) .
//                        Ws_down into slot 0.
//   k_pre_combine        out[t] = sum of token t's pair rows in slot order, in
//                        fp32, rounded once to the dtype.
//
// All GEMMs run on the LDS-staged tile of gemm_tile.h with swapped operands,
// so an accumulator lane holds 4 consecutive columns of one row.  Pair values
// are fp16 (11-bit significand): a bf16 pair buffer costs up to 4 % of
// RMS(out) on heavy-tailed gates.
#pragma once

#include <string.h>

#include "deco_common.h"
#include "deco_internal.h"
#include "gemm_tile.h"

using namespace deco;

namespace {

struct PreArgs {
  const void* x;
  void* out;
  unsigned* err;       // device error flags (bit 5: a value outside the fp16 range)
  int T, Tcap, d, E, F, Fs, W;
  int top_k;           // TopK routing variant (0: ReLU routing)
  int fuse_shared;     // the shared expert's down-projection runs in k_pre_shared_combine, not as
                       // shared tiles of k_pre_expert (slot 0 of the pair rows stays unused)
  int no_mean, no_rms; // NormSiLU ablations: drop the mean term / the RMS step
  float* sraw;         // RMS-only NormSiLU shared expert: [T][Fs] x . Ws_up (fp32), else null
  int nkb_d, nkb_F, nkb_Fs, pR, pF, pD, pFs;
  int pF4, pFs4;       // panel counts of the mean and shared sections, padded to 4
  int rs_nt;           // 8-panel column tiles of the router/mean/shared GEMM
  const char* Wr_p;
  const char* Wup_p;       // NormSiLU input projection (a gated expert's gate projection)
  const char* Wlin_p;      // gated experts' up-projection
  const char* Wbar_p;
  const char* Wdn_p;
  const char* Wdn16_p;     // down-projection operand of the prefill path (fp16 or fp32)
  const char* Wsu_p;
  const char* Wsd_p;
  size_t up_stride, dn_stride;
  const float* b_r;
  const float* lam;
  float eps;
  float* z;
  float* g;
  float* mbuf;
  uint64_t* mask;
  int* tok_off;
  int* ecnt;
  int* list_tok;
  void* sbuf;
  void* ybuf;
  // backward pass
  const void* dout;        // [T][d] upstream gradient of the layer output
  const char* WdnT_p;      // W_down[e]^T frags (K = d, N = F)
  const char* WupT_p;      // W_up[e]^T frags (K = F, N = d), down operand type
  float* dgbuf;            // [Tcap][E] dLoss/dg
  void* dhbuf;             // [pair slots][F] dLoss/dh~ (layer dtype; bf16 layers: the high part)
  void* agbuf;             // [pair slots][F] g * a (likewise)
  void* dhbuf_lo;          // bf16 layers: the low parts (value - high part, rounded), else null
  void* agbuf_lo;
  int* slot_list;          // [E][Tcap] pair slot of each list entry
  // small-batch split of the expert tiles (see k_pre_expert, PART)
  float* hpart;            // [nks][pcap][F] K-part sums of x . W_up[e] per pair slot
  size_t pcap;             // pair-slot rows of one K part
  int nks, ncb;            // K parts of the up-projection, column blocks of the down-projection
};

// what an expert tile computes
constexpr int XM_FWD = 0;     // NormSiLU(x.W_up[e] - m) . W_down[e], times the gate
constexpr int XM_GATED = 1;   // (NormSiLU(x.W_gate[e] - m) * x.W_up[e]) . W_down[e], times the gate
constexpr int XM_BWD = 2;     // backward of XM_FWD: dLoss/dh~ . W_up[e]^T and the pair rows

__device__ __forceinline__ float dsilu_f(float u) {
  const float sg = 1.0f / (1.0f + __expf(-u));
  return sg * (1.0f + u * (1.0f - sg));
}

#ifndef DECO_PRE_NS
#define DECO_PRE_NS 2     // pipeline stages in LDS (32 KiB each for the dense tiles)
#endif
#ifndef DECO_PRE_XNS
#define DECO_PRE_XNS DECO_PRE_NS   // stages of the expert tiles' up-projection ring
#endif
// Gated experts' tiles (64 rows, two K = d passes) with 3 up-projection stages
// (up to 128-column experts; wider ones would not fit two workgroups per CU):
// same-box A/B at T = 4096 on the d = 2048 layer, expert kernel 219 -> 208 us.
// The non-gated 64-row tiles got slower with 3 stages (169 -> 232 us), and the
// backward's were unchanged, so they keep DECO_PRE_XNS.
#ifndef DECO_PRE_GNS
#define DECO_PRE_GNS 3
#endif

constexpr int NXCD = 8;
constexpr int GM = 128;   // rows of the dense GEMM tiles
constexpr int GP = 8;     // 16-column panels of the dense GEMM tiles
template <class DT>
using DenseTile = Tile<DT, GM, GP, DECO_PRE_NS>;
#ifndef DECO_SPLIT_SGP
#define DECO_SPLIT_SGP 4   // panels per shared tile beside the split's column-block units
#endif

// Workgroups are handed to the 8 XCDs round-robin (workgroup b runs on XCD
// b % 8).  Renumber them so each XCD works on one contiguous range of tiles:
// tiles next to each other share operands, and each XCD has its own L2.
__device__ __forceinline__ int xcd_tile(int b, int n) {
  const int per = n / NXCD, rem = n % NXCD, x = b % NXCD, i = b / NXCD;
  return x * per + (x < rem ? x : rem) + i;
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, m);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), m);
  return ((uint64_t)hi << 32) | lo;
}

// 4 consecutive values of one row, stored as the dtype (8 bytes bf16, 16 fp32)
template <class DT>
__device__ __forceinline__ void store4(typename DT::elem* p, float v0, float v1, float v2, float v3) {
  if constexpr (sizeof(typename DT::elem) == 2) {
    uint2 u;
    u.x = f32_to_bf16(v0) | (f32_to_bf16(v1) << 16);
    u.y = f32_to_bf16(v2) | (f32_to_bf16(v3) << 16);
    *reinterpret_cast<uint2*>(p) = u;
  } else {
    *reinterpret_cast<float4*>(p) = make_float4(v0, v1, v2, v3);
  }
}

// v = hi + lo to about 16 significant bits, both bf16 (for fp32 layers the
// value itself, lo unused)
template <class DT>
__device__ __forceinline__ void store4_split(typename DT::elem* hi, typename DT::elem* lo, const float* v) {
  store4<DT>(hi, v[0], v[1], v[2], v[3]);
  if constexpr (sizeof(typename DT::elem) == 2) {
    float r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = v[i] - bf16_to_f32(f32_to_bf16(v[i]));
    store4<DT>(lo, r[0], r[1], r[2], r[3]);
  }
}

// fp16 pair rows: `bad` is raised for a value outside the fp16 range (the
// caller reports it), which would otherwise be stored as inf
constexpr float FP16_MAX = 65504.f;
template <class PT>
__device__ __forceinline__ void store4_pair(PT* p, const f32x4_t& v, bool& bad) {
  if constexpr (sizeof(PT) == 2) {
    bad |= !(fabsf(v[0]) <= FP16_MAX && fabsf(v[1]) <= FP16_MAX && fabsf(v[2]) <= FP16_MAX &&
             fabsf(v[3]) <= FP16_MAX);
    typedef __attribute__((__vector_size__(4 * sizeof(_Float16)))) _Float16 h4;
    h4 h = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
    *reinterpret_cast<h4*>(p) = h;
  } else {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
}

// 4 consecutive activation values at element `idx` of a row-major buffer of
// the down-projection operand type (fp16: `bad` is raised for a value
// outside the fp16 range)
template <class DN>
__device__ __forceinline__ void store4_act(void* base, size_t idx, const float* v, bool& bad) {
  if constexpr (DN::KB == 32) {
    bad |= !(fabsf(v[0]) <= FP16_MAX && fabsf(v[1]) <= FP16_MAX && fabsf(v[2]) <= FP16_MAX &&
             fabsf(v[3]) <= FP16_MAX);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(base) + idx) =
        make_uint2(DN::bits(v[0]) | (DN::bits(v[1]) << 16), DN::bits(v[2]) | (DN::bits(v[3]) << 16));
  } else {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(base) + idx) = make_float4(v[0], v[1], v[2], v[3]);
  }
}

// --------------------------------------------------------------------------
// NS pipeline stages in LDS: 2 (64 KiB, two workgroups per CU) when the grid
// exceeds the CUs, 4 (one per CU, three steps of loads in flight) when it
// does not, which is the case below a few thousand tokens; BMR rows per tile:
// 128, or 64 when even the four-stage grid of 128-row tiles leaves CUs idle.
// BNP 16-column panels per tile: 8, or 4 or 2 for small batches, where 8-panel
// tiles leave most CUs without work and each busy CU streams 1 MiB of weights
// at one CU's rate.  Narrow tiles go column-tile major (the row tiles of one
// column tile on one XCD, which then reads those weight panels once).
template <class DT, int NS, int BMR = GM, int BNP = GP>
__global__ void __launch_bounds__(256, 2) k_pre_router_shared(PreArgs a) {
  using elem = typename DT::elem;
  using TC = Tile<DT, BMR, BNP, NS>;
  static_assert(BNP == 2 || BNP == 4 || BNP == 8, "a wave's panels must lie in one 4-panel section");
  __shared__ i32x4_t lds[TC::LDS_V];
  const int tid = threadIdx.x, w = tid >> 6, wm = w >> 1, wn = w & 1, l = tid & 63, g = l >> 4, c = l & 15;
  const int t = xcd_tile(blockIdx.x, gridDim.x);
  const int n_mt = (a.T + BMR - 1) / BMR;
  const int m0 = BNP == GP ? (t / a.rs_nt) * BMR : (t % n_mt) * BMR;
  const int p0 = BNP == GP ? (t % a.rs_nt) * GP : (t / n_mt) * BNP;
  const elem* x = (const elem*)a.x;
  // rows past T and padding panels read valid memory; those outputs are dropped
  auto row = [&](int r) -> const elem* {
    const int rr = m0 + r;
    return x + (size_t)(rr < a.T ? rr : a.T - 1) * a.d;
  };
  auto panel = [&](int p) -> const char* {
    int q = p0 + p;
    if (q < a.pR) return a.Wr_p + frag_off(q, 0, a.nkb_d);
    q -= a.pR;
    if (q < a.pF4) return a.Wbar_p + frag_off(q < a.pF ? q : 0, 0, a.nkb_d);
    q -= a.pF4;
    return a.Wsu_p + frag_off(q < a.pFs ? q : 0, 0, a.nkb_d);
  };
  f32x4_t acc[TC::MB][TC::NBW];
#pragma unroll
  for (int i = 0; i < TC::MB; ++i)
#pragma unroll
    for (int j = 0; j < TC::NBW; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  tile_gemm<DT, TC, true>(lds, row, panel, a.nkb_d, acc);

  // lane: row m0 + wm*BMR/2 + 16 i + c, columns 16 (q0 + j) + 4 g + ii
  const int q0 = p0 + wn * TC::NBW;   // a multiple of NBW: one section per wave
  if (q0 < a.pR) {
    float be[TC::NBW][4], le[TC::NBW][4];
#pragma unroll
    for (int j = 0; j < TC::NBW; ++j)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int e = (q0 + j) * 16 + 4 * g + ii;
        be[j][ii] = e < a.E ? a.b_r[e] : 0.f;
        le[j][ii] = e < a.E ? a.lam[e] : 0.f;
      }
#pragma unroll
    for (int i = 0; i < TC::MB; ++i) {
      const int r = m0 + wm * (BMR / 2) + 16 * i + c;
      uint64_t bits = 0;
#pragma unroll
      for (int j = 0; j < TC::NBW; ++j)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int e = (q0 + j) * 16 + 4 * g + ii;
          const float zv = acc[i][j][ii] + be[j][ii];
          const bool act = e < a.E && zv > 0.f && le[j][ii] != 0.f;
          if (act) bits |= 1ull << (16 * j + 4 * g + ii);
          if (r < a.T && e < a.E) {
            a.z[(size_t)r * a.E + e] = zv;
            a.g[(size_t)r * a.E + e] = act ? le[j][ii] * zv : 0.f;
          }
        }
      bits |= shfl_xor_u64(bits, 16);
      bits |= shfl_xor_u64(bits, 32);
      // the wave's 16 NBW experts are bits 16 (q0 % 4) .. of mask word q0 / 4
      // (little-endian: bytes 2 (q0 % 4) ..); narrower tiles store their part
      if (g == 0 && r < a.T) {
        uint64_t* mw = a.mask + (size_t)r * a.W + q0 / 4;
        if constexpr (TC::NBW == 4) *mw = bits;
        else if constexpr (TC::NBW == 2) reinterpret_cast<uint32_t*>(mw)[(q0 & 3) >> 1] = (uint32_t)bits;
        else reinterpret_cast<uint16_t*>(mw)[q0 & 3] = (uint16_t)bits;
      }
    }
  } else if (q0 - a.pR < a.pF4) {
    const int q = q0 - a.pR;
#pragma unroll
    for (int j = 0; j < TC::NBW; ++j) {
      if (q + j < a.pF) {
        const int f0 = (q + j) * 16 + 4 * g;
#pragma unroll
        for (int i = 0; i < TC::MB; ++i) {
          const int r = m0 + wm * (BMR / 2) + 16 * i + c;
          if (r < a.T)
            *reinterpret_cast<float4*>(a.mbuf + (size_t)r * a.F + f0) =
                make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
        }
      }
    }
  } else {
    const int q = q0 - a.pR - a.pF4;
    elem* sb = (elem*)a.sbuf;
#pragma unroll
    for (int j = 0; j < TC::NBW; ++j) {
      if (q + j < a.pFs) {
        const int c0 = (q + j) * 16 + 4 * g;
#pragma unroll
        for (int i = 0; i < TC::MB; ++i) {
          const int r = m0 + wm * (BMR / 2) + 16 * i + c;
          if (r < a.T) {
            if (a.sraw)   // RMS-only NormSiLU: the row's RMS spans other workgroups' columns
              *reinterpret_cast<float4*>(a.sraw + (size_t)r * a.Fs + c0) =
                  make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
            else
              store4<DT>(sb + (size_t)r * a.Fs + c0, silu_f(acc[i][j][0]), silu_f(acc[i][j][1]),
                         silu_f(acc[i][j][2]), silu_f(acc[i][j][3]));
          }
        }
      }
    }
  }
}

// RMS-only NormSiLU of the shared expert (an ablation switch): one wave per
// token, s = SiLU(u / sqrt(mean_j u_j^2 + eps)) from the fp32 row u = x . Ws_up.
template <class DT>
__global__ void __launch_bounds__(256) k_pre_shared_rms(PreArgs a) {
  using elem = typename DT::elem;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + w;
  if (r >= a.T) return;
  const float* u = a.sraw + (size_t)r * a.Fs;
  float ss = 0.f;
  for (int j = l; j < a.Fs; j += 64) ss += u[j] * u[j];
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
  const float rinv = 1.0f / sqrtf(ss / (float)a.Fs + a.eps);
  elem* sb = (elem*)a.sbuf + (size_t)r * a.Fs;
  for (int j = l; j < a.Fs; j += 64) sb[j] = DT::from_f32(silu_f(u[j] * rinv));
}

// --------------------------------------------------------------------------
// TopK routing variant (the baseline of the DECO paper's Sec. 4 acceleration
// experiment, Table 4): one wave per token keeps the top_k largest of the
// logits the router GEMM stored (ties to the lower expert index) and
// replaces the token's gates (softmax of the kept logits) and mask words.
__global__ void __launch_bounds__(256) k_pre_topk(PreArgs a) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6), l = threadIdx.x & 63;
  if (t >= a.T) return;
  float zv[4];
  bool sel[4];
  float gate[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = 64 * j + l;
    zv[j] = e < a.E ? a.z[(size_t)t * a.E + e] : -__builtin_inff();
  }
  topk_wave<4>(zv, a.top_k, sel, gate);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = 64 * j + l;
    if (e < a.E) a.g[(size_t)t * a.E + e] = gate[j];
    const unsigned long long word = __ballot(sel[j]);
    if (l == 0 && j < a.W) a.mask[(size_t)t * a.W + j] = word;
  }
}

// --------------------------------------------------------------------------
// Exclusive scan of one int per thread over a workgroup of NW waves; *total
// receives the sum.  s_tmp holds NW ints.
template <int NW>
__device__ __forceinline__ int block_excl_scan(int v, int* s_tmp, int* total) {
  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (l >= o) incl += y;
  }
  if (l == 63) s_tmp[w] = incl;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) {
    const int t = s_tmp[ww];
    if (ww < w) base += t;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return base + incl - v;
}

// Workgroup e < E: the ascending token list of expert e and its size.
// Workgroup E: per token, the offset of its pair slots (exclusive prefix of
// 1 + the token's active-expert count): slot 0 for the shared expert, then
// one per active expert in ascending e.
constexpr int DISP_NT = 1024, DISP_TPT = 4;

__global__ void __launch_bounds__(DISP_NT) k_pre_dispatch(PreArgs a) {
  __shared__ int s_tmp[DISP_NT / 64];
  const int e = blockIdx.x, tid = threadIdx.x;
  const bool offsets = e == a.E;
  const int wi = e >> 6, bit = e & 63;
  int run = 0;
  for (int t0 = 0; t0 < a.T; t0 += DISP_NT * DISP_TPT) {
    const int tb = t0 + tid * DISP_TPT;
    int v[DISP_TPT], local = 0;
#pragma unroll
    for (int k = 0; k < DISP_TPT; ++k) {
      const int t = tb + k;
      v[k] = 0;
      if (t < a.T) {
        if (offsets) {
          v[k] = 1;   // slot 0: the shared expert
          for (int ww = 0; ww < a.W; ++ww) v[k] += __popcll(a.mask[(size_t)t * a.W + ww]);
        } else {
          v[k] = (int)((a.mask[(size_t)t * a.W + wi] >> bit) & 1ull);
        }
      }
      local += v[k];
    }
    int tot;
    int pos = run + block_excl_scan<DISP_NT / 64>(local, s_tmp, &tot);
#pragma unroll
    for (int k = 0; k < DISP_TPT; ++k) {
      const int t = tb + k;
      if (offsets) {
        if (t < a.T) a.tok_off[t] = pos;
      } else if (v[k]) {
        a.list_tok[(size_t)e * a.Tcap + pos] = t;
      }
      pos += v[k];
    }
    run += tot;
  }
  if (tid == 0) {
    if (offsets) a.tok_off[a.T] = run;
    else a.ecnt[e] = run;
  }
}

// --------------------------------------------------------------------------
#ifndef DECO_SPLIT_NS
#define DECO_SPLIT_NS 3   // up-projection ring stages of the split's k-part units
#endif
template <class DT, int BNP, int MODE, bool SMALL = false, int NSU = DECO_PRE_NS>
struct ExpertShape {
  using DN = typename DT::Down;                      // down-projection operand type
  // token rows per tile (gated experts and the backward hold a second
  // K = d accumulator, so their tiles have half the rows; SMALL: batches too
  // small to fill the persistent grid with 128-row tiles use 64)
  static constexpr int BM = (BNP >= 16 || MODE != XM_FWD || SMALL) ? 64 : 128;
  using TC = Tile<DT, BM, BNP, NSU>;                  // up-projection ring
  static constexpr int F = BNP * 16;
  static constexpr int NKF = F / DN::KB;             // k-blocks of the down-projection
  static constexpr int RB = BM / 16;                 // 16-row blocks of the tile
  static constexpr int MB = BM / 32;                 // 16-row blocks per wave
  static constexpr int ACT_V = RB * NKF * 64;        // 16-byte LDS slots of the activations
  static constexpr int DP = NKF >= 8 ? 2 : 4;        // W_down panels per ring stage
  static constexpr int DSTAGE_V = DP * NKF * 64;
  static constexpr int DNS = 3;                      // ring stages
  static constexpr int DLPW = DP * NKF / 4;          // ring loads per wave per stage
  // output staging: the gated pair values of one ring stage (BM tokens x
  // 16 DP columns) go through LDS so that global stores write whole rows.
  // 16-byte chunk q of staged row R sits at slot R*OCH + (q ^ (R % OCH)).
  using PT = typename DT::pair;
  static constexpr int OROW = DP * 16 * (int)sizeof(PT);   // bytes of one staged row
  static constexpr int OCH = OROW / 16;                    // 16-byte chunks per staged row
  static constexpr int OBUF_V = BM * OCH;
  static constexpr int FPT = BM * OCH / 256;               // staged-row stores per thread
  static_assert(BM * OCH % 256 == 0 && (OCH & (OCH - 1)) == 0, "staged rows must divide over the workgroup");
  static constexpr int OCC = sizeof(typename DT::elem) == 2 ? 2 : 1;   // workgroups per CU
  static constexpr int cmax(int x, int y) { return x > y ? x : y; }
  // shared tiles stage their 128 x 128 output the same way
  static constexpr int SPITCH_V = GP * 16 * (int)sizeof(PT) / 16 + 1;
  static constexpr int GM_SPITCH_V = GM * SPITCH_V;
  static constexpr int LDS_V = cmax(cmax(TC::LDS_V, ACT_V),
                                    cmax(DNS * DSTAGE_V + OBUF_V,
                                         cmax(DenseTile<DT>::LDS_V, GM * SPITCH_V)));
  static_assert((DP * NKF) % 4 == 0, "ring fragments must divide over the 4 waves");
};

// One persistent kernel for all grouped work after the dispatch:
//   expert tiles  (expert e, up to BM of its tokens): gathered x . W_up[e],
//                 NormSiLU, then . W_down[e], scaled by the gates and written
//                 to the tokens' pair slots;
//   shared tiles  (128 tokens x 128 columns): SiLU(x Ws_up) . Ws_down, written
//                 to slot 0 of each token's pairs.
// Expert tiles come first (they are the longer ones); each XCD works through
// its own contiguous range of both lists.
//
// XM_GATED: a routed expert's NormSiLU output is multiplied, element by
// element, by x . W_up[e] (a second pass of the tile over W_lin before the
// NormSiLU input's pass; its accumulators wait in registers).
//
// XM_BWD (backward pass; expert tiles only): with q = dout . W_down[e]^T
// (the ungated output gradient, a second pass of the tile), u = h~ / r and
// a = SiLU(u) recomputed as in the forward pass, per row
//   dg  = sum_f a_f q_f                               (gradient of the gate)
//   du  = g q SiLU'(u)
//   dh~ = du / r - h~ (sum_f du_f h~_f) / (F r^3)     (through NormSiLU step 2)
// dg goes to dgbuf, dh~ and g*a to the pair-slot rows of dhbuf and agbuf
// (operands of the weight gradients), the slot to slot_list, and
// dh~ . W_up[e]^T (this pair's part of dLoss/dx) to the pair buffer.
//
// PART (small batches, XM_FWD): the expert tiles split over more workgroups,
// in two launches.  PART = 1: unit (expert tile, k part q) computes the
// tile's x . W_up[e] over k-blocks q nkb/nks .. (q + 1) nkb/nks - 1 and stores
// it in fp32 to hpart[q][pair slot]; no shared tiles.  PART = 2: unit (expert
// tile, column block b) adds the nks parts in order, applies NormSiLU and
// multiplies by column block b (pD/ncb panels) of W_down[e]; shared tiles as
// usual.  A thin expert then costs a few hundred KiB of weights per workgroup
// instead of its whole 2 d F, spread over nks + ncb workgroups.
template <class DT, int BNP, int MODE, bool SMALL = false, bool ACT = false, int PART = 0>
__global__ void __launch_bounds__(256, (ExpertShape<DT, BNP, MODE, SMALL>::OCC)) k_pre_expert(PreArgs a) {
  static_assert(PART == 0 || (MODE == XM_FWD && SMALL && !ACT), "the split runs the forward's 64-row tiles");
  using elem = typename DT::elem;
  using S = ExpertShape<DT, BNP, MODE, SMALL,
                        PART == 1 ? DECO_SPLIT_NS : (MODE == XM_GATED && BNP <= 8 ? DECO_PRE_GNS : DECO_PRE_XNS)>;
  using TC = typename S::TC;
  using DN = typename S::DN;
  using PT = typename DT::pair;
  constexpr int BM = S::BM, MB = S::MB, NBW = TC::NBW, F = S::F, NKF = S::NKF, DP = S::DP;
  // one LDS array for everything (the operand rings, the activations, the
  // staging buffer and the per-tile tables), carved below
  constexpr int SMALL_V = (257 + 4 + 3 * BM + 2 * BM + (MODE == XM_BWD ? 4 * BM : 0) + 3) / 4;
  __shared__ i32x4_t lds_all[S::LDS_V + SMALL_V];
  i32x4_t* lds = lds_all;
  int* s_toff = reinterpret_cast<int*>(lds_all + S::LDS_V);
  int* s_tmp = s_toff + 257;
  int* s_tok = s_tmp + 4;
  int* s_slot = s_tok + BM;
  float* s_gate = reinterpret_cast<float*>(s_slot + BM);
  float (*s_ss)[BM] = reinterpret_cast<float (*)[BM]>(s_gate + BM);
  float (*s_bw)[2][BM] = reinterpret_cast<float (*)[2][BM]>(s_gate + 3 * BM);   // XM_BWD: [dg, dot][wn][row]
  const int tid = threadIdx.x, w = tid >> 6, wm = w >> 1, wn = w & 1, l = tid & 63, g = l >> 4, c = l & 15;

  // expert e owns tiles s_toff[e] .. s_toff[e + 1] - 1
  {
    const int n = tid < a.E ? (a.ecnt[tid] + BM - 1) / BM : 0;
    int tot;
    const int ex = block_excl_scan<4>(n, s_tmp, &tot);
    if (tid < a.E) s_toff[tid] = ex;
    if (tid == 0) s_toff[a.E] = tot;
  }
  __syncthreads();
  const int nsub = PART == 1 ? a.nks : PART == 2 ? a.ncb : 1;   // units per expert tile
  const int n_et = s_toff[a.E] * nsub;                       // expert units
  // shared tiles: 128 rows x SGP panels (the split's column-block units are
  // small, and 8-panel shared tiles would be the few long ones among them)
  constexpr int SGP = PART == 2 ? DECO_SPLIT_SGP : GP;
  const int nsp = (a.pD + SGP - 1) / SGP;                    // shared tiles per 128 rows
  // the backward, the activation-output mode and the K-part units have no shared tiles
  const int n_st = (MODE == XM_BWD || ACT || PART == 1 || a.fuse_shared) ? 0 : ((a.T + GM - 1) / GM) * nsp;
  const int xg = blockIdx.x % NXCD, lb = blockIdx.x / NXCD;
  const int gx = ((int)gridDim.x - xg + NXCD - 1) / NXCD;    // workgroups on this XCD
  // consecutive units (of one tile: they share its rows) stay on one XCD
  const int e_beg = (int)((long long)n_et * xg / NXCD), e_end = (int)((long long)n_et * (xg + 1) / NXCD);
  const int s_beg = (int)((long long)n_st * xg / NXCD), s_end = (int)((long long)n_st * (xg + 1) / NXCD);
  const int n_mine = (e_end - e_beg) + (s_end - s_beg);
  const float invF = 1.0f / (float)F;
  const elem* x = (const elem*)a.x;
  PT* yb = (PT*)a.ybuf;

  for (int k = lb; k < n_mine; k += gx) {
    lds_barrier();   // the previous tile no longer reads LDS
    if (k >= e_end - e_beg) {
      // ---- shared tile: rows m0.., panels p0.. of SiLU(x Ws_up) . Ws_down
      using TD = Tile<DT, GM, SGP, DECO_PRE_NS>;
      const int ts = s_beg + k - (e_end - e_beg);
      const int m0 = (ts / nsp) * GM, p0 = (ts % nsp) * SGP;
      const elem* sbuf = (const elem*)a.sbuf;
      auto row = [&](int r) -> const elem* {
        const int rr = m0 + r;
        return sbuf + (size_t)(rr < a.T ? rr : a.T - 1) * a.Fs;
      };
      auto panel = [&](int p) -> const char* {
        return a.Wsd_p + frag_off(p0 + p < a.pD ? p0 + p : 0, 0, a.nkb_Fs);
      };
      f32x4_t acc[TD::MB][TD::NBW];
#pragma unroll
      for (int i = 0; i < TD::MB; ++i)
#pragma unroll
        for (int j = 0; j < TD::NBW; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      tile_gemm<DT, TD, true>(lds, row, panel, a.nkb_Fs, acc);
      // stage the tile (pair type) in LDS, then store whole rows
      constexpr int CPR = SGP * 16 * (int)sizeof(PT) / 16;   // 16-byte chunks per row
      constexpr int SPI = CPR + 1;                            // staged row pitch (16-byte slots)
      static_assert(GM * SPI <= S::GM_SPITCH_V, "shared staging fits the LDS");
      bool bad = false;
#pragma unroll
      for (int i = 0; i < TD::MB; ++i) {
        const int R = wm * (GM / 2) + 16 * i + c;
#pragma unroll
        for (int j = 0; j < TD::NBW; ++j)
          store4_pair(reinterpret_cast<PT*>(lds + R * SPI) + (wn * TD::NBW + j) * 16 + 4 * g, acc[i][j], bad);
      }
      if (bad) atomicOr(a.err, 32u);
      lds_barrier();
      const int ncol_ch = (a.pD - p0 < SGP ? a.pD - p0 : SGP) * 16 * (int)sizeof(PT) / 16;
      for (int idx = tid; idx < GM * CPR; idx += 256) {
        const int R = idx / CPR, q = idx % CPR, r = m0 + R;
        if (r < a.T && q < ncol_ch)
          st16(reinterpret_cast<char*>(yb + (size_t)a.tok_off[r] * a.d + p0 * 16) + q * 16, lds[R * SPI + q]);
      }
      continue;
    }

    // ---- expert tile (one unit of it)
    const int unit = e_beg + k;
    const int tile = unit / nsub, sub = unit - tile * nsub;
    int lo = 0, hi = a.E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_toff[mid] <= tile) lo = mid; else hi = mid;
    }
    const int e = lo;
    const int n_e = a.ecnt[e];
    const int r0 = (tile - s_toff[e]) * BM;
    if (tid < BM) {
      const int rank = r0 + tid;
      int tok = -1, slot = -1;
      float gate = 0.f;
      if (rank < n_e) {
        tok = a.list_tok[(size_t)e * a.Tcap + rank];
        const uint64_t* mrow = a.mask + (size_t)tok * a.W;
        int below = 0;
        for (int ww = 0; ww < (e >> 6); ++ww) below += __popcll(mrow[ww]);
        below += __popcll(mrow[e >> 6] & ((1ull << (e & 63)) - 1ull));
        slot = a.tok_off[tok] + 1 + below;   // slot 0 of the token holds the shared expert
        gate = a.g[(size_t)tok * a.E + e];
        if constexpr (MODE == XM_BWD) a.slot_list[(size_t)e * a.Tcap + rank] = slot;
      }
      s_tok[tid] = tok;
      s_slot[tid] = slot;
      s_gate[tid] = gate;
    }
    lds_barrier();

    // up-projection of the gathered rows, all F columns
    const char* Wu = a.Wup_p + (size_t)e * a.up_stride;
    if constexpr (PART == 1) {
      // k part `sub`: its k-blocks of every row and panel, stored as fp32 sums
      const int nkq = a.nkb_d / a.nks, kb0 = sub * nkq;
      auto row_q = [&](int r) -> const elem* {
        const int tk = s_tok[r];
        return x + (size_t)(tk >= 0 ? tk : 0) * a.d + (size_t)kb0 * DT::KB;
      };
      auto panel_q = [&](int p) -> const char* { return Wu + frag_off(p, kb0, a.nkb_d); };
      f32x4_t accq[MB][NBW];
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NBW; ++j) accq[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      tile_gemm<DT, TC, true>(lds, row_q, panel_q, nkq, accq);
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const int R = wm * (BM / 2) + 16 * i + c;
        if (s_tok[R] >= 0) {
          float* hp = a.hpart + ((size_t)sub * a.pcap + s_slot[R]) * F + 4 * g;
#pragma unroll
          for (int j = 0; j < NBW; ++j)
            *reinterpret_cast<float4*>(hp + 16 * (wn * NBW + j)) =
                make_float4(accq[i][j][0], accq[i][j][1], accq[i][j][2], accq[i][j][3]);
        }
      }
      continue;
    }
    auto row = [&](int r) -> const elem* {
      const int tk = s_tok[r];   // padding rows read token 0; their outputs are dropped
      return x + (size_t)(tk >= 0 ? tk : 0) * a.d;
    };
    auto panel = [&](int p) -> const char* { return Wu + frag_off(p, 0, a.nkb_d); };
    f32x4_t acc[MB][NBW], accu[MB][NBW];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NBW; ++j) acc[i][j] = accu[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if constexpr (MODE == XM_GATED) {
      const char* Wl = a.Wlin_p + (size_t)e * a.up_stride;
      auto panel_lin = [&](int p) -> const char* { return Wl + frag_off(p, 0, a.nkb_d); };
      tile_gemm<DT, TC, true>(lds, row, panel_lin, a.nkb_d, accu);
    }
    if constexpr (MODE == XM_BWD) {
      // q = dout . W_down[e]^T over the gathered rows
      const char* Wt = a.WdnT_p + (size_t)e * a.up_stride;
      const elem* dout = (const elem*)a.dout;
      auto row_d = [&](int r) -> const elem* {
        const int tk = s_tok[r];
        return dout + (size_t)(tk >= 0 ? tk : 0) * a.d;
      };
      auto panel_t = [&](int p) -> const char* { return Wt + frag_off(p, 0, a.nkb_d); };
      tile_gemm<DT, TC, true>(lds, row_d, panel_t, a.nkb_d, accu);
    }
    // the mean-term values of the tile's rows, requested before the K loop so
    // that they have landed when the NormSiLU needs them
    float4 mpre[MB][NBW];
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int tk = s_tok[wm * (BM / 2) + 16 * i + c];
      const float* mrow = a.mbuf + (size_t)(tk < 0 ? 0 : tk) * F;
#pragma unroll
      for (int j = 0; j < NBW; ++j) mpre[i][j] = *reinterpret_cast<const float4*>(mrow + 16 * (wn * NBW + j) + 4 * g);
    }
    if constexpr (PART == 2) {
      // the nks k-part sums of the tile's rows, added in part order
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const int R = wm * (BM / 2) + 16 * i + c;
        if (s_tok[R] >= 0) {
          for (int q = 0; q < a.nks; ++q) {
            const float* hp = a.hpart + ((size_t)q * a.pcap + s_slot[R]) * F + 4 * g;
#pragma unroll
            for (int j = 0; j < NBW; ++j) {
              const float4 v = *reinterpret_cast<const float4*>(hp + 16 * (wn * NBW + j));
              acc[i][j][0] += v.x;
              acc[i][j][1] += v.y;
              acc[i][j][2] += v.z;
              acc[i][j][3] += v.w;
            }
          }
        }
      }
    } else {
      tile_gemm<DT, TC, true>(lds, row, panel, a.nkb_d, acc);
    }

    // NormSiLU.  Lane: local row R = wm*BM/2 + 16 i + c, columns
    // f = 16 (wn*NBW + j) + 4 g + ii.  Subtract the mean term, then the sum
    // of squares over the row's F columns: in-lane, over the 4 lane groups,
    // then over the two column halves (waves wn = 0, 1) through LDS.
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int R = wm * (BM / 2) + 16 * i + c;
      const float mk = a.no_mean ? 0.f : 1.f;   // ablation: no mean term
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < NBW; ++j) {
        const float4 m = mpre[i][j];
        acc[i][j][0] -= mk * m.x;
        acc[i][j][1] -= mk * m.y;
        acc[i][j][2] -= mk * m.z;
        acc[i][j][3] -= mk * m.w;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) ss += acc[i][j][ii] * acc[i][j][ii];
      }
      ss += __shfl_xor(ss, 16);
      ss += __shfl_xor(ss, 32);
      if (g == 0) s_ss[wn][R] = ss;
    }
    lds_barrier();
    if constexpr (MODE == XM_BWD) {
      // per-row sums of a * q and du * h~ (same reduction path as the sums of squares)
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const int R = wm * (BM / 2) + 16 * i + c;
        const bool ok = s_tok[R] >= 0;
        const float inv_r = ok ? 1.0f / sqrtf((s_ss[0][R] + s_ss[1][R]) * invF + a.eps) : 0.f;
        const float gr = s_gate[R];
        float sdg = 0.f, sdot = 0.f;
#pragma unroll
        for (int j = 0; j < NBW; ++j)
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const float u = acc[i][j][ii] * inv_r, q = accu[i][j][ii];
            sdg += silu_f(u) * q;
            sdot += gr * q * dsilu_f(u) * acc[i][j][ii];
          }
        sdg += __shfl_xor(sdg, 16);
        sdg += __shfl_xor(sdg, 32);
        sdot += __shfl_xor(sdot, 16);
        sdot += __shfl_xor(sdot, 32);
        if (g == 0) {
          s_bw[0][wn][R] = sdg;
          s_bw[1][wn][R] = sdot;
        }
      }
      lds_barrier();
    }
    // activations into LDS in the fragment order of the down-projection's
    // token operand (rounded once to the operand type); the backward puts
    // dh~ there and stores its pair rows
    bool act_bad = false;
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int R = wm * (BM / 2) + 16 * i + c;
      const bool ok = s_tok[R] >= 0;
      const float inv_r = ok ? (a.no_rms ? 1.0f : 1.0f / sqrtf((s_ss[0][R] + s_ss[1][R]) * invF + a.eps)) : 0.f;
      float gr = 0.f, dot_r = 0.f;
      size_t prow = 0;
      if constexpr (MODE == XM_BWD) {
        gr = s_gate[R];
        dot_r = (s_bw[1][0][R] + s_bw[1][1][R]) * inv_r * inv_r * inv_r * invF;
        prow = (size_t)(ok ? s_slot[R] : 0) * F;
        if (ok && wn == 0 && g == 0) a.dgbuf[(size_t)s_tok[R] * a.E + e] = s_bw[0][0][R] + s_bw[0][1][R];
      }
#pragma unroll
      for (int j = 0; j < NBW; ++j) {
        const int p = wn * NBW + j;
        float v[4];
        if constexpr (MODE == XM_BWD) {
          float ag[4];
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const float ht = acc[i][j][ii], u = ht * inv_r, q = accu[i][j][ii];
            v[ii] = ok ? gr * q * dsilu_f(u) * inv_r - ht * dot_r : 0.f;   // dh~
            ag[ii] = ok ? gr * silu_f(u) : 0.f;
          }
          if (ok) {
            const int f = 16 * p + 4 * g;
            store4_split<DT>((elem*)a.dhbuf + prow + f, (elem*)a.dhbuf_lo + prow + f, v);
            store4_split<DT>((elem*)a.agbuf + prow + f, (elem*)a.agbuf_lo + prow + f, ag);
          }
        } else {
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            v[ii] = ok ? silu_f(acc[i][j][ii] * inv_r) : 0.f;
            if constexpr (MODE == XM_GATED) v[ii] *= accu[i][j][ii];
          }
        }
        if constexpr (ACT) {
          // the pair slot's activation row, ungated, in the down-projection
          // operand type (row-major, F values)
          if (ok) store4_act<DN>(a.ybuf, (size_t)s_slot[R] * F + 16 * p + 4 * g, v, act_bad);
        } else if constexpr (DN::KB == 32) {
          // f = 16 p + 4 g + ii: k-block p / 2, lane group 2 (p % 2) + g / 2,
          // elements 4 (g % 2) + ii of the lane
          const int slot = ((R >> 4) * NKF + (p >> 1)) * 64 + (R & 15) + 16 * (2 * (p & 1) + (g >> 1));
          *reinterpret_cast<uint2*>(reinterpret_cast<char*>(lds + slot) + 8 * (g & 1)) =
              make_uint2(DN::bits(v[0]) | (DN::bits(v[1]) << 16), DN::bits(v[2]) | (DN::bits(v[3]) << 16));
        } else {
          // fp32: f = 16 p + 4 g + ii: k-block p, lane group g, elements ii
          *reinterpret_cast<float4*>(lds + ((R >> 4) * NKF + p) * 64 + (R & 15) + 16 * g) =
              make_float4(v[0], v[1], v[2], v[3]);
        }
      }
    }
    if constexpr (ACT) {
      if (act_bad) atomicOr(a.err, 32u);
      continue;   // the down-projection runs in k_pre_dc
    }
    lds_barrier();
    // each wave keeps the activations of its token blocks in registers
    i32x4_t act[MB][NKF];
#pragma unroll
    for (int jt = 0; jt < MB; ++jt)
#pragma unroll
      for (int kb = 0; kb < NKF; ++kb) act[jt][kb] = lds[((wm * MB + jt) * NKF + kb) * 64 + l];
    float gt[MB];   // the backward's pair rows are not gated
#pragma unroll
    for (int jt = 0; jt < MB; ++jt) gt[jt] = MODE == XM_BWD ? 1.0f : s_gate[wm * (BM / 2) + 16 * jt + c];
    lds_barrier();   // every wave holds its activations: the LDS becomes the W_down ring

    // down-projection through a ring of DP-panel stages of W_down[e] (all
    // NKF k-blocks of each panel); wave (wm, wn) takes its token blocks and
    // panels wn*DP/2 .. of each stage.  Operands swapped (W_down as the row
    // operand): a lane holds 4 consecutive output columns of one token.
    const char* Wd = (MODE == XM_BWD ? a.WupT_p : a.Wdn16_p) + (size_t)e * a.dn_stride;
    // stages of this unit: all pD / DP, or (PART = 2) column block `sub` of them
    const int nds = PART == 2 ? a.pD / DP / a.ncb : a.pD / DP;
    const int st0 = PART == 2 ? sub * nds : 0;
    i32x4_t* obuf = lds + S::DNS * S::DSTAGE_V;   // staging buffer after the ring
    constexpr int OCH = S::OCH;
    auto issue = [&](int st) {
      i32x4_t* ring = lds + (st % S::DNS) * S::DSTAGE_V;
#pragma unroll
      for (int i = 0; i < S::DLPW; ++i) {
        const int f = w * S::DLPW + i;   // panel f / NKF of the stage, k-block f % NKF
        load_lds16(Wd + frag_off((st0 + st) * DP + f / NKF, f % NKF, NKF) + l * 16, ring + f * 64);
      }
    };
    // copy the staged stage `st` (BM rows x OROW bytes) to the tokens' pair
    // rows.  Exactly FPT stores per thread, none skipped (padding rows go to
    // the scratch row after the pair buffer), so the vmcnt waits below can
    // leave the latest stores in flight.
    const size_t trash = (size_t)a.Tcap * (a.E + 1);
    auto flush = [&](int st) {
#pragma unroll
      for (int u = 0; u < S::FPT; ++u) {
        const int idx = tid + 256 * u, R = idx / OCH, q = idx % OCH, slot = s_slot[R];
        st16(reinterpret_cast<char*>(yb + (slot >= 0 ? (size_t)slot : trash) * a.d + (st0 + st) * DP * 16) + q * 16,
             obuf[R * OCH + (q ^ (R & (OCH - 1)))]);
      }
    };
    static_assert(S::DNS == 3, "the vmcnt counts below assume a 3-stage ring");
    // Per iteration st the memory operations are: flush(st - 1) (FPT stores),
    // then the loads of stage st + 2.  So after the loads of stage st come:
    // st = 0: stage 1's loads; st = 1: stage 2's; st >= 2: the stores of
    // flush(st - 2) and stage st + 1's loads (those that exist).
    auto wait_stage = [&](int st) {
      const bool next = st + 1 < nds;
      if (st < 2) {
        if (next) wait_vmcnt<S::DLPW>(); else wait_vmcnt<0>();
      } else {
        if (next) wait_vmcnt<S::FPT + S::DLPW>(); else wait_vmcnt<S::FPT>();
      }
    };
    if (nds > 0) issue(0);
    if (nds > 1) issue(1);
    for (int st = 0; st < nds; ++st) {
      wait_stage(st);
      lds_barrier();   // stage st landed; staged st - 1 complete; ring stage st - 1 free
      if (st > 0) flush(st - 1);
      if (st + 2 < nds) issue(st + 2);
      const i32x4_t* ring = lds + (st % S::DNS) * S::DSTAGE_V;
      f32x4_t y[MB][DP / 2];
#pragma unroll
      for (int jt = 0; jt < MB; ++jt)
#pragma unroll
        for (int q = 0; q < DP / 2; ++q) y[jt][q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NKF; ++kb) {
        i32x4_t bv[DP / 2];
#pragma unroll
        for (int q = 0; q < DP / 2; ++q) bv[q] = ring[((wn * (DP / 2) + q) * NKF + kb) * 64 + l];
#pragma unroll
        for (int jt = 0; jt < MB; ++jt)
#pragma unroll
          for (int q = 0; q < DP / 2; ++q) DN::mma(y[jt][q], bv[q], act[jt][kb]);
      }
      lds_barrier();   // flush(st - 1) has read the staging buffer
      // gate, round to the pair type, stage: token R, columns (wn*DP/2 + q)*16 + 4 g ..
      bool bad = false;
#pragma unroll
      for (int jt = 0; jt < MB; ++jt) {
        const int R = wm * (BM / 2) + 16 * jt + c;
#pragma unroll
        for (int q = 0; q < DP / 2; ++q) {
          f32x4_t v = y[jt][q];
          v[0] *= gt[jt];
          v[1] *= gt[jt];
          v[2] *= gt[jt];
          v[3] *= gt[jt];
          const int b = ((wn * (DP / 2) + q) * 16 + 4 * g) * (int)sizeof(PT);   // byte in the staged row
          store4_pair(reinterpret_cast<PT*>(reinterpret_cast<char*>(obuf + R * OCH + ((b >> 4) ^ (R & (OCH - 1)))) +
                                            (b & 15)),
                      v, bad);
        }
      }
      if (bad) atomicOr(a.err, 32u);
    }
    lds_barrier();
    if (nds > 0) flush(nds - 1);
  }
}

// --------------------------------------------------------------------------
// The gate-weighted combine fused with the shared expert (DECO paper Sec. 2:
// the shared expert is always active and its output is added to the routed
// experts' weighted sum).  One workgroup per 128 tokens x 16 SGP columns:
// s . Ws_down for its tile on the LDS-staged MFMA tile (s = SiLU(x Ws_up)
// from the router GEMM), the fp32 result staged in LDS; then per (token,
// 8 columns) the shared value plus the token's pair rows (slots 1.. of its
// pair range, ascending expert order) in fp32, rounded once to the dtype.
// The shared term never passes through the fp16 pair buffer.
template <class DT, int SGP>
__global__ void __launch_bounds__(256, 2) k_pre_shared_combine(PreArgs a) {
  using elem = typename DT::elem;
  using PT = typename DT::pair;
  using TD = Tile<DT, GM, SGP, DECO_PRE_NS>;
  constexpr int NCOL = 16 * SGP;
  constexpr int SPF = NCOL + 4;                    // staged row pitch, floats
  constexpr int STAGE_V = GM * SPF / 4;            // 16-byte LDS slots of the stage
  constexpr int LDS_V = TD::LDS_V > STAGE_V ? TD::LDS_V : STAGE_V;
  __shared__ i32x4_t lds[LDS_V];
  const int tid = threadIdx.x, w = tid >> 6, wm = w >> 1, wn = w & 1, l = tid & 63, g = l >> 4, c = l & 15;
  const int nsp = (a.pD + SGP - 1) / SGP;
  // consecutive tiles (one XCD) are the column tiles of one row tile
  const int t = xcd_tile(blockIdx.x, gridDim.x);
  const int m0 = (t / nsp) * GM, p0 = (t % nsp) * SGP;
  const elem* sbuf = (const elem*)a.sbuf;
  auto row = [&](int r) -> const elem* {
    const int rr = m0 + r;
    return sbuf + (size_t)(rr < a.T ? rr : a.T - 1) * a.Fs;
  };
  auto panel = [&](int p) -> const char* { return a.Wsd_p + frag_off(p0 + p < a.pD ? p0 + p : 0, 0, a.nkb_Fs); };
  f32x4_t acc[TD::MB][TD::NBW];
#pragma unroll
  for (int i = 0; i < TD::MB; ++i)
#pragma unroll
    for (int j = 0; j < TD::NBW; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  tile_gemm<DT, TD, true>(lds, row, panel, a.nkb_Fs, acc);   // ends with a barrier: the ring is free
  float* st = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int i = 0; i < TD::MB; ++i) {
    const int R = wm * (GM / 2) + 16 * i + c;
#pragma unroll
    for (int j = 0; j < TD::NBW; ++j)
      *reinterpret_cast<float4*>(st + R * SPF + 16 * (wn * TD::NBW + j) + 4 * g) =
          make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
  }
  lds_barrier();
  constexpr int CH = NCOL / 8;                     // 8-column chunks per row
  const int ncol = (a.pD - p0 < SGP ? a.pD - p0 : SGP) * 16;
  for (int it = tid; it < GM * CH; it += 256) {
    const int R = it / CH, col = 8 * (it % CH), r = m0 + R;
    if (r >= a.T || col >= ncol) continue;
    float v[8];
    {
      const float4 u0 = *reinterpret_cast<const float4*>(st + R * SPF + col);
      const float4 u1 = *reinterpret_cast<const float4*>(st + R * SPF + col + 4);
      v[0] = u0.x; v[1] = u0.y; v[2] = u0.z; v[3] = u0.w;
      v[4] = u1.x; v[5] = u1.y; v[6] = u1.z; v[7] = u1.w;
    }
    const int s1 = a.tok_off[r + 1];
    int s = a.tok_off[r] + 1;   // slot 0 (the unfused shared row) is not used
    const PT* yb = (const PT*)a.ybuf + p0 * 16 + col;
    auto add = [&](const PT* p) {
      if constexpr (sizeof(PT) == 2) {
        const f16x8_t y = *reinterpret_cast<const f16x8_t*>(p);
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] += (float)y[k];
      } else {
        const float4 y0 = *reinterpret_cast<const float4*>(p);
        const float4 y1 = *reinterpret_cast<const float4*>(p + 4);
        v[0] += y0.x; v[1] += y0.y; v[2] += y0.z; v[3] += y0.w;
        v[4] += y1.x; v[5] += y1.y; v[6] += y1.z; v[7] += y1.w;
      }
    };
    for (; s + 4 <= s1; s += 4) {
      // four independent loads in flight, added in slot order
      if constexpr (sizeof(PT) == 2) {
        f16x8_t y[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) y[u] = *reinterpret_cast<const f16x8_t*>(yb + (size_t)(s + u) * a.d);
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int k = 0; k < 8; ++k) v[k] += (float)y[u][k];
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) add(yb + (size_t)(s + u) * a.d);
      }
    }
    for (; s < s1; ++s) add(yb + (size_t)s * a.d);
    elem* orow = (elem*)a.out + (size_t)r * a.d + p0 * 16 + col;
    store4<DT>(orow, v[0], v[1], v[2], v[3]);
    store4<DT>(orow + 4, v[4], v[5], v[6], v[7]);
  }
}

// --------------------------------------------------------------------------
// out[t] = sum of token t's pair rows (its shared-expert output, then its
// gated expert outputs in ascending expert order), in fp32, rounded once.
// One thread per 8 output columns; loads batched four pair rows at a time.
// F32OUT: the sum is written in fp32 (the backward's dLoss/dx).
template <class DT, bool F32OUT = false>
__global__ void __launch_bounds__(256) k_pre_combine(PreArgs a) {
  using elem = typename DT::elem;
  using PT = typename DT::pair;
  const int cpr = a.d / 8;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  const int r = (int)(idx / cpr), col = (int)(idx % cpr) * 8;
  if (r >= a.T) return;
  const int s0 = a.tok_off[r], s1 = a.tok_off[r + 1];
  const PT* yb = (const PT*)a.ybuf + col;
  float v[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) v[k] = 0.f;
  auto add = [&](const PT* p) {
    if constexpr (sizeof(PT) == 2) {
      const f16x8_t y = *reinterpret_cast<const f16x8_t*>(p);
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] += (float)y[k];
    } else {
      const float4 y0 = *reinterpret_cast<const float4*>(p);
      const float4 y1 = *reinterpret_cast<const float4*>(p + 4);
      v[0] += y0.x; v[1] += y0.y; v[2] += y0.z; v[3] += y0.w;
      v[4] += y1.x; v[5] += y1.y; v[6] += y1.z; v[7] += y1.w;
    }
  };
  int s = s0;
  for (; s + 4 <= s1; s += 4) {
    // four independent loads in flight, added in slot order
    if constexpr (sizeof(PT) == 2) {
      f16x8_t y[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) y[u] = *reinterpret_cast<const f16x8_t*>(yb + (size_t)(s + u) * a.d);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] += (float)y[u][k];
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) add(yb + (size_t)(s + u) * a.d);
    }
  }
  for (; s < s1; ++s) add(yb + (size_t)s * a.d);
  if constexpr (F32OUT) {
    float* orow = (float*)a.out + (size_t)r * a.d + col;
    *reinterpret_cast<float4*>(orow) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(orow + 4) = make_float4(v[4], v[5], v[6], v[7]);
  } else {
    elem* orow = (elem*)a.out + (size_t)r * a.d + col;
    store4<DT>(orow, v[0], v[1], v[2], v[3]);
    store4<DT>(orow + 4, v[4], v[5], v[6], v[7]);
  }
}

int round4(int v) { return (v + 3) / 4 * 4; }

// launch arguments shared by the forward and backward launchers
// --------------------------------------------------------------------------
// Down-projection and combine, token-major (large batches; F <= 4 k-blocks).
//
// A workgroup of 256 NG threads owns the output block rows m0 .. m0 + 128 NG
// and panels p0 .. p0 + 7 (128 columns).  Wave w: rows (w / 2) * 64 + 0..63 of
// the block, panels (w % 2) * 4 + 0..3; its lane (c, g) accumulates rows
// 16 i + c (i < 4) of those 64 and columns 4 g .. 4 g + 3 of each panel (the
// swapped-operand layout of the tile GEMM).
//   1. acc = S[rows] . Ws_down[:, cols] with S = the shared expert's
//      activations (one tile GEMM per group of four waves, 128 rows each).
//   2. For every expert touched by the block's tokens, in ascending order:
//      W_down[e][:, cols] arrives in a ring of three LDS stages (one expert
//      per stage, two in flight, shared by all waves).  Each wave lists its
//      own rows routed to e (a ballot over its 64 rows; the pair slot of row
//      t is its token's slot base plus the number of lower experts it uses),
//      loads those rows' activation fragments from the pair-slot buffer one
//      expert ahead, multiplies them by W_down[e], scales each row by its gate
//      and adds it to the owning lanes' accumulators through a staging block
//      of its own in LDS (16 gathered rows at a time, no workgroup barrier).
//   3. out = acc, rounded once.
// Every output element gets the shared term first and then its token's
// experts in ascending order, in fp32, on every call: the result does not
// depend on scheduling, and no per-pair output rows go through memory.
// LDS stores issued as inline asm.  While LDS-DMA loads are in flight the
// compiler cannot tell an ordinary LDS store from one that may overlap their
// destination and drains every outstanding load before it; these stores go
// to LDS that no DMA targets, and a wave's LDS accesses are performed in
// order, so reads later in the same wave see them.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}
__device__ __forceinline__ void lds_store16(void* p, float x, float y, float z, float w) {
  const f32x4_t v = {x, y, z, w};
  __asm__ volatile("ds_write_b128 %0, %1" ::"v"(lds_addr(p)), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_store4(void* p, uint32_t v) {
  __asm__ volatile("ds_write_b32 %0, %1" ::"v"(lds_addr(p)), "v"(v) : "memory");
}
template <class DT, int NKF, int NG>
struct DcShape {
  using TD = Tile<DT, GM, GP, 2>;                       // shared GEMM of one row group
  static constexpr int NT = 256 * NG, NW = 4 * NG, BT = GM * NG;
  static constexpr int WSTAGE_V = GP * NKF * 64;        // W_down slots of one expert (8 panels)
  static constexpr int NWS = 3;                         // W_down ring stages
  static constexpr int WPW = GP * NKF / NW;             // ring loads per wave per stage
  static constexpr int SP = 68;                         // floats per staged row (64 + 4 pad)
  static constexpr int STG_V = 16 * SP / 4;             // one wave's staging block (16-byte slots)
  static constexpr int PF_RB = 2;                       // row blocks per wave loaded one expert ahead
  static constexpr int MAXW = 4;                        // mask words (at most 256 experts)
  static constexpr int RING1_V = NG * TD::LDS_V;
  static constexpr int P2_V = NWS * WSTAGE_V + NW * STG_V;
  static constexpr int BIG_V = RING1_V > P2_V ? RING1_V : P2_V;
  // tables after the big region (bytes): masks, touched experts and their
  // count, the any-token words, per-wave lists (slot, gate, position) x 2
  static constexpr int T_MASK = 0;
  static constexpr int T_ANY = T_MASK + BT * MAXW * 8;
  static constexpr int T_EX = T_ANY + MAXW * 8;
  static constexpr int T_WL = T_EX + 260 * 4;
  static constexpr int T_WG = T_WL + NW * 2 * 64 * 4;
  static constexpr int T_WP = T_WG + NW * 2 * 64 * 4;
  static constexpr int T_END = T_WP + NW * 2 * 64 * 4;
  static constexpr int LDS_V = BIG_V + (T_END + 15) / 16;
  static_assert(WPW * NW == GP * NKF && WPW >= 1, "ring fragments must divide over the waves");
  static_assert(PF_RB == 2, "the kernel selects the prefetched row blocks by rb == 0 / 1");
  static_assert(LDS_V * 16 <= 160 * 1024, "LDS budget");
};

template <class DT, int NKF, int NG>
__global__ void __launch_bounds__(256 * NG, 1) k_pre_dc(PreArgs a) {
  using elem = typename DT::elem;
  using DN = typename DT::Down;
  using S = DcShape<DT, NKF, NG>;
  using TD = typename S::TD;
  constexpr int NW = S::NW, BT = S::BT, MAXW = S::MAXW, SP = S::SP, PF_RB = S::PF_RB;
  __shared__ i32x4_t lds[S::LDS_V];
  char* tab = reinterpret_cast<char*>(lds + S::BIG_V);
  uint64_t* s_mask = reinterpret_cast<uint64_t*>(tab + S::T_MASK);
  unsigned long long* s_any = reinterpret_cast<unsigned long long*>(tab + S::T_ANY);
  int* s_ex = reinterpret_cast<int*>(tab + S::T_EX);             // [256] experts, [256] their count
  int (*s_wl)[2][64] = reinterpret_cast<int (*)[2][64]>(tab + S::T_WL);
  float (*s_wg)[2][64] = reinterpret_cast<float (*)[2][64]>(tab + S::T_WG);
  int (*s_wp)[2][64] = reinterpret_cast<int (*)[2][64]>(tab + S::T_WP);

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, c = l & 15, g = l >> 4;
  const int wr = w >> 1, wc = w & 1;
  const int n_tt = (a.T + BT - 1) / BT;
  const int t = xcd_tile(blockIdx.x, gridDim.x);   // column-tile major: an XCD keeps few W_down slices
  const int m0 = (t % n_tt) * BT, p0 = (t / n_tt) * GP;
  const int nw = a.W;

  // ---- routing masks of the block's rows; experts touched by any of them
  if (tid < MAXW) s_any[tid] = 0ull;
  lds_barrier();
  // row role: lane l of wave w stands for block row wr*64 + l (both waves of
  // a row pair hold the same rows)
  const int rloc = wr * 64 + l, rrow = m0 + rloc;
  const bool rvalid = rrow < a.T;
  const int rslot0 = rvalid ? a.tok_off[rrow] + 1 : 0;   // slot 0 of a token is its shared expert's
  if (wc == 0) {
    for (int ww = 0; ww < nw; ++ww) {
      const uint64_t v = rvalid ? a.mask[(size_t)rrow * nw + ww] : 0ull;
      s_mask[rloc * MAXW + ww] = v;
      if (v) atomicOr(&s_any[ww], (unsigned long long)v);
    }
  }
  lds_barrier();
  if (w == 0) {
    int base = 0;
    for (int q = 0; q < nw; ++q) {
      const int e = 64 * q + l;
      const bool bit = e < a.E && ((s_any[q] >> l) & 1ull);
      const uint64_t bal = __ballot(bit);
      const int pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
      if (bit) s_ex[base + pos] = e;
      base += __popcll(bal);
    }
    if (l == 0) s_ex[256] = base;
  }

  // ---- 1. shared expert: acc = S[rows] . Ws_down[:, cols]
  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  {
    const int grp = w >> 2;
    const elem* sb = (const elem*)a.sbuf;
    const int rg0 = m0 + grp * GM;
    auto row = [&](int r) -> const elem* {
      const int rr = rg0 + r;   // rows past T read row T - 1; their outputs are dropped
      return sb + (size_t)(rr < a.T ? rr : a.T - 1) * a.Fs;
    };
    auto panel = [&](int p) -> const char* {
      const int q = p0 + p;
      return a.Wsd_p + frag_off(q < a.pD ? q : 0, 0, a.nkb_Fs);
    };
    tile_gemm<DT, TD, true>(lds + grp * TD::LDS_V, row, panel, a.nkb_Fs, acc, tid & 255);
  }   // ends with a barrier: s_ex is visible and the LDS ring is free

  // ---- 2. routed experts
  const int n_ex = s_ex[256];
  if (n_ex > 0) {
    i32x4_t* wring = lds;
    float* stg = reinterpret_cast<float*>(lds + S::NWS * S::WSTAGE_V + w * S::STG_V);
    const __attribute__((address_space(3))) float* stg3 = (const __attribute__((address_space(3))) float*)stg;
    const size_t act_row = (size_t)NKF * 64;   // bytes of one activation row (F values)
    const char* actb = (const char*)a.ybuf;
    // the touched experts (lane l holds entries l, 64 + l, ..) and this
    // lane's row mask in registers: no LDS round trip per expert
    int exr[MAXW];
    uint64_t rmask[MAXW];
#pragma unroll
    for (int q = 0; q < MAXW; ++q) {
      exr[q] = s_ex[64 * q + l];
      rmask[q] = q < nw ? s_mask[rloc * MAXW + q] : 0ull;
    }
    // (u uniform; the lane is read straight from each register, so the
    // result does not depend on which lanes are active at the call)
    auto expert_of = [&](int u) -> int {
      const int uu = u < n_ex ? u : n_ex - 1;
      const int q = uu >> 6, ln = uu & 63;
      const int e0 = __builtin_amdgcn_readlane(exr[0], ln), e1 = __builtin_amdgcn_readlane(exr[1], ln);
      const int e2 = __builtin_amdgcn_readlane(exr[2], ln), e3 = __builtin_amdgcn_readlane(exr[3], ln);
      return q == 0 ? e0 : q == 1 ? e1 : q == 2 ? e2 : e3;
    };
    // W_down[e][:, cols] of touched expert u into ring stage u % 3 (past the
    // end: the last expert again, never read)
    auto issue_w = [&](int u) {
      const int e = expert_of(u);
      i32x4_t* st = wring + (u % S::NWS) * S::WSTAGE_V;
      const char* base = a.Wdn16_p + (size_t)e * a.dn_stride;
#pragma unroll
      for (int i = 0; i < S::WPW; ++i) {
        const int f = w * S::WPW + i;   // panel f / NKF of the block, k-block f % NKF
        const int q = p0 + f / NKF;
        load_lds16(base + frag_off(q < a.pD ? q : 0, f % NKF, NKF) + l * 16, st + f * 64);
      }
    };
    // this wave's rows routed to touched expert u: list (parity u & 1), each
    // row's position in it, and the count
    int rank = 0;
    auto build = [&](int u, bool& bit, int& pos) -> int {
      const int e = expert_of(u);
      const int q = e >> 6;
      const uint64_t mw = q == 0 ? rmask[0] : q == 1 ? rmask[1] : q == 2 ? rmask[2] : rmask[3];
      bit = u < n_ex && ((mw >> (e & 63)) & 1ull);
      const uint64_t bal = __ballot(bit);
      pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
      const int b = u & 1;
      if (bit) lds_store4(&s_wl[w][b][pos], (uint32_t)(rslot0 + rank));
      lds_store4(&s_wp[w][b][l], (uint32_t)(bit ? pos : -1));
      rank += bit ? 1 : 0;
      return (int)__popcll(bal);
    };
    // activation fragments of the first PF_RB row blocks of list u, and the
    // gate of this lane's row
    auto issue_act = [&](int u, int n, i32x4_t (&av)[PF_RB][NKF], bool bit, float& gate) {
      const int b = u & 1;
      int slot[PF_RB];
#pragma unroll
      for (int rb = 0; rb < PF_RB; ++rb) {
        const int p = 16 * rb + c;
        slot[rb] = p < n ? s_wl[w][b][p] : 0;   // rows past the list: any valid row, unused
      }
#pragma unroll
      for (int rb = 0; rb < PF_RB; ++rb) {
        if (16 * rb >= n) break;   // no rows in this block (the count is the same for the whole wave)
        const char* src = actb + (size_t)slot[rb] * act_row + g * 16;
#pragma unroll
        for (int kb = 0; kb < NKF; ++kb) av[rb][kb] = ld16(src + kb * 64);
      }
      const int e = expert_of(u);
      gate = a.g[bit ? (size_t)rrow * a.E + e : 0];
    };
    // two register sets, used alternately (a copy from one to the other
    // would wait for the loads just issued)
    struct Unit {
      i32x4_t av[PF_RB][NKF];
      bool bit;
      int pos, n;
      float gate;
    };
    Unit ua, ub;
    ua.n = build(0, ua.bit, ua.pos);
    issue_act(0, ua.n, ua.av, ua.bit, ua.gate);
    issue_w(0);
    issue_w(1);
    auto step = [&](int u, Unit& cu, Unit& nx) {
      // stage u of W_down (issued two experts ago) and this wave's activation
      // loads of expert u (issued before the ring loads of u + 1) have landed
      wait_vmcnt<S::WPW>();
      if (cu.bit) lds_store4(&s_wg[w][u & 1][cu.pos], __float_as_uint(cu.gate));
      lds_barrier();   // stage u visible to all waves; stage u - 1 no longer read
      nx.n = build(u + 1, nx.bit, nx.pos);
      issue_act(u + 1, nx.n, nx.av, nx.bit, nx.gate);
      issue_w(u + 2);
      // expert u on this wave's rows: 16 gathered rows at a time
      const i32x4_t* st = wring + (u % S::NWS) * S::WSTAGE_V;
      const int n_c = cu.n, b = u & 1;
      const int nb = (n_c + 15) >> 4;
      // positions of the owned rows 16 i + c in the list (-1: not routed)
      int pos_i[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pos_i[i] = s_wp[w][b][16 * i + c];
      for (int rb = 0; rb < nb; ++rb) {
        const int p = 16 * rb + c;
        const float gt = p < n_c ? s_wg[w][b][p] : 0.f;
        i32x4_t av[NKF];
        if (rb < PF_RB) {
#pragma unroll
          for (int kb = 0; kb < NKF; ++kb) av[kb] = rb == 0 ? cu.av[0][kb] : cu.av[PF_RB - 1][kb];
        } else {
          // more than PF_RB * 16 rows of this wave use the expert: the rest
          // are loaded here
          const int slot = p < n_c ? s_wl[w][b][p] : 0;
          const char* src = actb + (size_t)slot * act_row + g * 16;
#pragma unroll
          for (int kb = 0; kb < NKF; ++kb) av[kb] = ld16(src + kb * 64);
        }
        f32x4_t y[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) y[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NKF; ++kb)
#pragma unroll
          for (int j = 0; j < 4; ++j) DN::mma(y[j], st[((wc * 4 + j) * NKF + kb) * 64 + l], av[kb]);
        // lane: gathered row 16 rb + c, columns 16 j + 4 g .. of the wave's 64
#pragma unroll
        for (int j = 0; j < 4; ++j)
          lds_store16(stg + c * SP + 16 * j + 4 * g, y[j][0] * gt, y[j][1] * gt, y[j][2] * gt, y[j][3] * gt);
        // the staging block is this wave's alone, written before these reads
        // (a wave's LDS accesses are performed in order): every owned row
        // reads a staged row (row 0 when it has none in this block) and keeps
        // it only when it is its own
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          f32x4_t v[2][4];
          bool own[2];
#pragma unroll
          for (int ii = 0; ii < 2; ++ii) {
            const int pp = pos_i[2 * h + ii] - 16 * rb;
            own[ii] = pp >= 0 && pp < 16;
            const int r = own[ii] ? pp : 0;
#pragma unroll
            for (int j = 0; j < 4; ++j)
              v[ii][j] = *(const __attribute__((address_space(3))) f32x4_t*)(stg3 + r * SP + 16 * j + 4 * g);
          }
#pragma unroll
          for (int ii = 0; ii < 2; ++ii)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
              for (int k = 0; k < 4; ++k) acc[2 * h + ii][j][k] += own[ii] ? v[ii][j][k] : 0.f;
        }
        // the next block's staging writes come after these reads (in order)
        __asm__ volatile("" ::: "memory");
      }
    };
    for (int u = 0; u < n_ex; u += 2) {
      step(u, ua, ub);
      if (u + 1 < n_ex) step(u + 1, ub, ua);
    }
  }

  // ---- 3. out = acc
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = m0 + wr * 64 + 16 * i + c;
    if (r >= a.T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q = p0 + wc * 4 + j;
      if (q < a.pD)
        store4<DT>((elem*)a.out + (size_t)r * a.d + 16 * q + 4 * g, acc[i][j][0], acc[i][j][1], acc[i][j][2],
                   acc[i][j][3]);
    }
  }
}

PreArgs fill_pre_args(const deco_moe_layer* L, const void* x, int T, void* out) {
  PreArgs a;
  memset(&a, 0, sizeof(a));
  a.x = x;
  a.out = out;
  a.T = T;
  a.Tcap = L->maxT < 16 ? 16 : L->maxT;
  a.d = L->d;
  a.E = L->E;
  a.F = L->F;
  a.Fs = L->Fs;
  a.W = L->W;
  a.top_k = L->cfg.top_k;
  a.no_mean = (L->cfg.normsilu & DECO_NORMSILU_NO_MEAN) != 0;
  a.no_rms = (L->cfg.normsilu & DECO_NORMSILU_NO_RMS) != 0;
  a.sraw = L->cfg.shared_rms ? L->sraw : nullptr;
  a.nkb_d = L->nkb_d;
  a.nkb_F = L->nkb_F;
  a.nkb_Fs = L->nkb_Fs;
  a.pR = L->pR;
  a.pF = L->pF;
  a.pD = L->pD;
  a.pFs = L->pFs;
  a.pF4 = round4(L->pF);
  a.pFs4 = round4(L->pFs);
  a.rs_nt = (a.pR + a.pF4 + a.pFs4 + GP - 1) / GP;
  a.Wr_p = L->Wr_p;
  a.Wup_p = L->Wup_p;
  a.Wlin_p = L->Wlin_p;
  a.Wbar_p = L->Wbar_p;
  a.Wdn_p = L->Wdn_p;
  a.Wsu_p = L->Wsu_p;
  a.Wsd_p = L->Wsd_p;
  a.up_stride = L->up_stride;
  a.dn_stride = L->dn_stride;
  a.b_r = L->b_r;
  a.lam = L->lam;
  a.eps = L->cfg.rms_eps;
  a.z = L->z;
  a.g = L->g;
  a.mbuf = L->mbuf;
  a.mask = L->mask;
  a.tok_off = L->tok_off;
  a.ecnt = L->ecnt;
  a.list_tok = L->list_tok;
  a.Wdn16_p = L->Wdn16_p;
  a.sbuf = L->sbuf;
  a.ybuf = L->ybuf;
  a.err = L->dec_err;
  a.hpart = L->hpart;
  a.pcap = (size_t)L->split_maxT * (L->E + 1);
  a.nks = a.ncb = 1;
  return a;
}

// Router tile shape: 64-row tiles, with the four-stage ring while the batch
// makes at most half as many 128-row tiles as CUs, else with the two-stage
// ring (three workgroups per CU).  Twice the tiles balance better over the
// CUs than 128-row ones (same-box A/B on the d = 2048 layer: T = 2048 32.0 ->
// 29.4 us, T = 4096 40.4 -> 36.6 us; d = 4096 layer at T = 2048: 76.0 ->
// 66.7 us).  DECO_PRE_RS_LARGE_BM = 128 restores 128-row tiles for the
// larger batches.
#ifndef DECO_PRE_RS_LARGE_BM
#define DECO_PRE_RS_LARGE_BM 64
#endif
static_assert(DECO_PRE_RS_LARGE_BM == GM || DECO_PRE_RS_LARGE_BM == GM / 2, "router tile rows");
#ifndef DECO_PRE_RS_NARROW
#define DECO_PRE_RS_NARROW 1   // 0: 8-panel router tiles at every batch size (measurement builds)
#endif
#ifndef DECO_PRE_RS_NARROW_NS
#define DECO_PRE_RS_NARROW_NS 4   // ring stages of the narrow router tiles
#endif

// the routing steps shared by the forward and backward launchers: router
// (and the mean and shared up-projection), TopK selection, dispatch
template <class DT>
hipError_t launch_routing(const deco_moe_layer* L, const PreArgs& a, int T, hipStream_t s) {
  using deco_host::launch;
  const unsigned mtiles = (unsigned)((T + GM - 1) / GM);
  const unsigned rs_grid = mtiles * a.rs_nt;
  const unsigned mt64 = (unsigned)((T + GM / 2 - 1) / (GM / 2));
  const unsigned half_grid = mt64 * a.rs_nt;
  const unsigned large_grid = DECO_PRE_RS_LARGE_BM == GM ? rs_grid : half_grid;
  // small batches: the widest of 8, 4, 2-panel tiles whose grid covers the
  // CUs (2 if none does); the sections are whole multiples of 4 panels
  const unsigned n_pan = (unsigned)(a.pR + a.pF4 + a.pFs4), cus = (unsigned)L->n_cu;
  const int bnp = (!DECO_PRE_RS_NARROW || half_grid >= cus) ? 8 : mt64 * (n_pan / 4) >= cus ? 4 : 2;
  hipError_t err;
  if (2 * rs_grid > cus)
    err = launch(deco_host::KS_PRE_ROUTER_SHARED, k_pre_router_shared<DT, DECO_PRE_NS, DECO_PRE_RS_LARGE_BM>,
                 dim3(large_grid), dim3(256), s, a);
  else if (bnp == 8)
    err = launch(deco_host::KS_PRE_ROUTER_SHARED, k_pre_router_shared<DT, 4, GM / 2>, dim3(half_grid), dim3(256), s, a);
  else if (bnp == 4)
    err = launch(deco_host::KS_PRE_ROUTER_SHARED, k_pre_router_shared<DT, DECO_PRE_RS_NARROW_NS, GM / 2, 4>, dim3(mt64 * (n_pan / 4)),
                 dim3(256), s, a);
  else
    err = launch(deco_host::KS_PRE_ROUTER_SHARED, k_pre_router_shared<DT, DECO_PRE_RS_NARROW_NS, GM / 2, 2>, dim3(mt64 * (n_pan / 2)),
                 dim3(256), s, a);
  if (err == hipSuccess && a.top_k > 0)
    err = launch(deco_host::KS_PRE_TOPK, k_pre_topk, dim3((unsigned)((T + 3) / 4)), dim3(256), s, a);
  if (err == hipSuccess && a.sraw)
    err = launch(deco_host::KS_PRE_ROUTER_SHARED, k_pre_shared_rms<DT>, dim3((unsigned)((T + 3) / 4)), dim3(256), s, a);
  if (err == hipSuccess)
    err = launch(deco_host::KS_PRE_DISPATCH, k_pre_dispatch, dim3(L->E + 1), dim3(DISP_NT), s, a);
  return err;
}

}  // namespace
