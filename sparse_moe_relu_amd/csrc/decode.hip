// decode.hip - weight-streaming forward path for small batches (T <= 16).
//
// At decode sizes the layer is a handful of matrix-vector products over the
// weights, so its cost is the HBM traffic of the weights it touches.  The
// point of ReLU routing with sparse experts is that inactive routed experts
// cost nothing: the DECO paper (Sec. 1 and the Sec. 4 acceleration paragraph
// with Table 4) attributes its speedup to skipping the memory traffic of
// inactive experts.  Three kernels, no workgroup waiting on another:
//
//   k_dec_up   one workgroup per 32 columns of the shared expert, and per
//              (routed expert, 32 columns of F).  A routed workgroup computes
//              its expert's router logits for the batch (router: linear
//              projection + bias, ReLU, per-expert scale; DECO paper Sec. 2
//              "Router design") while its slice of the inter-expert mean Wbar
//              loads (one matrix shared by all experts, so it stays in L2),
//              and exits without reading any expert weight when no token
//              activated the expert.  Otherwise it streams its slice of
//              W_up[e] through v_mfma 16x16 products (tokens padded to 16 rows)
//              into the accumulator that already holds -x.Wbar: h - m, the
//              mean-subtracted pre-activation of NormSiLU (qidianchuan.cn
//              write-up, section 二: subtract the mean term, RMS inside the
//              expert, then SiLU).  It stores h - m and the per-row sums of
//              squares of its slice; the expert's first slice also stores the
//              logits, the gates and the expert's routing flag.  Shared-expert
//              workgroups store SiLU(x.Ws_up) as down-projection operands.
//   k_dec_down one workgroup per (128 output columns, 1/Q of the reduction).
//              It lists the experts at least one token activated, loads its
//              share of their down-projection weights (and of the shared
//              expert's), completes each row's RMS from the slices' sums of
//              squares, applies SiLU and the gate while building the MFMA
//              operands, multiplies, and stores its partial product.
//   k_dec_sum  adds the Q partial products of each output in split order
//              (deterministic) and writes out.
#include "deco_common.h"
#include "deco_internal.h"
#include "gemm_tile.h"

using namespace deco;

namespace {

struct DecArgs {
  const void* x;
  void* out;
  int T, d, E, F, Fs;
  int nkb_d, nkb_F, nkb_Fs, pF, pFs, pD, n_groups, Q;
  int n_shared, wg_per_e;   // up workgroups of the shared expert; per routed expert
  int top_k, pR, W;         // TopK variant (0: ReLU routing); router panels; mask words
  int gated;                // 1: gated experts (up workgroups for W_up[e] follow each expert's own)
  int no_mean, no_rms;      // NormSiLU ablations: drop the mean term / the RMS step
  float* sraw;              // RMS-only NormSiLU shared expert: [16][Fs] x . Ws_up (fp32), else null
  const char* Wr_p;
  const char* Wup_p;        // NormSiLU input projection (a gated expert's gate projection)
  const char* Wlin_p;       // gated experts' up-projection
  const char* Wbar_p;
  const char* Wdn_p;        // W_down in the operand type of the routed down-projection
  const char* Wsu_p;
  const char* Wsd_p;
  size_t up_stride, dn_stride;
  const float* b_r;
  const float* lam;
  float eps;
  float* z;
  float* g;
  float* hbuf;              // [E][16][F] h - m of each token row
  float* ubuf;              // [E][16][F] gated experts: x . W_up[e] of each token row
  float* sspart;            // [E][wg_per_e][16] sums of squares of h - m over each slice
  char* sactf;              // shared-expert activations as down-projection operand fragments
  unsigned* rflag;          // [E] 1 no token routed to e, 2 some token did
  uint64_t* mask;           // [T][W] routing masks (stored by the TopK router)
  float* part;
};

#ifndef DECO_DEC_NW
#define DECO_DEC_NW 8
#endif
#ifndef DECO_DEC_NP
#define DECO_DEC_NP 2
#endif
#ifndef DECO_DEC_CH
#define DECO_DEC_CH 8
#endif
constexpr int DEC_NW = DECO_DEC_NW;   // waves per workgroup
constexpr int DEC_NP = DECO_DEC_NP;   // 16-column panels per up workgroup
constexpr int DEC_CH = DECO_DEC_CH;   // k-blocks held in registers per wave at a time
constexpr int DEC_QMAX = 64;          // largest K-split of the down kernel (host clamps dec_q)
constexpr int DEC_WGMAX = 8;          // largest number of up slices per routed expert
constexpr int DEC_UB = 2;             // down-kernel units (k-blocks) in flight per wave
constexpr int DEC_DP = 8;             // 16-column output panels per down workgroup
constexpr int DEC_XMAX = 64;          // routed experts one down workgroup may touch (host plan)
// A buffer-load offset past the resource's range: the load returns zeros
// without touching memory (used to mask loads without branching).
constexpr unsigned OOB = 0xFFFFFF00u;

// 16 bytes through a buffer resource: `soff` is wave-uniform (an SGPR), so a
// run of such loads needs one VGPR for all its addresses
__device__ __forceinline__ i32x4_t ld16_buf(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff) {
  return __builtin_bit_cast(i32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}
__device__ __forceinline__ float ld_buf(__amdgpu_buffer_rsrc_t r, unsigned voff) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, 0, 0));
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7FFFFFFF, 0x00020000);
}

// TopK routing variant (the baseline of the DECO paper's Sec. 4 acceleration
// experiment, Table 4): one workgroup computes the logits of all experts for
// the batch (MFMA, 16 padded rows; the waves split d, then add their
// products in a fixed order), keeps each token's top_k experts (ties to the
// lower index), stores logits, gates (softmax of the kept logits) and masks,
// and publishes each expert's flag for the up and down kernels.
template <class DT, int NW>
__global__ void __launch_bounds__(NW * 64) k_dec_topk(DecArgs a) {
  using elem = typename DT::elem;
  constexpr int CH = 4, PG = 4;   // k-blocks and router panels per load batch
  constexpr int PMAX = 16;        // router panels (E <= 256)
  __shared__ f32x4_t s_red[NW][PG][64];
  __shared__ float s_z[16][PMAX * 16];
  __shared__ int s_act[PMAX * 16];
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, g = l >> 4, c = l & 15;
  const int nkb = a.nkb_d;
  const int kb_lo = (w * nkb) / NW, kb_hi = ((w + 1) * nkb) / NW;
  const elem* xrow = (const elem*)a.x + (size_t)c * a.d;
  const bool row_ok = c < a.T;
  const __amdgpu_buffer_rsrc_t rw = buf_rsrc(a.Wr_p);
  for (int e = tid; e < PMAX * 16; e += NW * 64) s_act[e] = 0;
  for (int pg = 0; pg < a.pR; pg += PG) {
    f32x4_t acc[PG];
#pragma unroll
    for (int p = 0; p < PG; ++p) acc[p] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int kb0 = kb_lo; kb0 < kb_hi; kb0 += CH) {
      i32x4_t xf[CH], wf[CH][PG];
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        const int kb = kb0 + u;
        xf[u] = (kb < kb_hi && row_ok) ? load_row_frag<DT>(xrow, kb, g) : zero16();
#pragma unroll
        for (int p = 0; p < PG; ++p)
          wf[u][p] = (kb < kb_hi && pg + p < a.pR) ? ld16_buf(rw, 16u * l, (unsigned)frag_off(pg + p, kb, nkb)) : zero16();
      }
#pragma unroll
      for (int u = 0; u < CH; ++u)
        if (kb0 + u < kb_hi) {
#pragma unroll
          for (int p = 0; p < PG; ++p) DT::mma(acc[p], xf[u], wf[u][p]);
        }
    }
#pragma unroll
    for (int p = 0; p < PG; ++p) s_red[w][p][l] = acc[p];
    __syncthreads();
    // lane (c, g) of panel p holds rows 4 g + i of expert 16 p + c
    for (int idx = tid; idx < PG * 256; idx += NW * 64) {
      const int p = idx >> 8, ll = (idx >> 2) & 63, i = idx & 3;
      float v = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) v += s_red[ww][p][ll][i];
      const int e = (pg + p) * 16 + (ll & 15);
      s_z[4 * (ll >> 4) + i][e] = v + (e < a.E ? a.b_r[e] : 0.f);
    }
    __syncthreads();
  }
  // one wave per token: keep the top_k logits
  if (w < a.T) {
    const int t = w;
    float zv[4];
    bool sel[4];
    float gate[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 64 * j + l;
      zv[j] = e < a.E ? s_z[t][e] : -__builtin_inff();
    }
    topk_wave<4>(zv, a.top_k, sel, gate);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 64 * j + l;
      if (e < a.E) {
        a.z[(size_t)t * a.E + e] = zv[j];
        a.g[(size_t)t * a.E + e] = gate[j];
        if (sel[j]) s_act[e] = 1;
      }
      const unsigned long long word = __ballot(sel[j]);
      if (l == 0 && j < a.W) a.mask[(size_t)t * a.W + j] = word;
    }
  }
  __syncthreads();
  for (int e = tid; e < a.E; e += NW * 64) a.rflag[e] = s_act[e] ? 2u : 1u;
}

// VAR: bit 0 gated experts, bit 1 no mean term, bit 2 RMS-only NormSiLU
// shared expert (the variants are separate instantiations, so the default
// one carries none of their logic)
constexpr int DV_GATED = 1, DV_NO_MEAN = 2, DV_SHARED_RMS = 4;
template <class DT, int NW, int NP, int VAR>
__global__ void __launch_bounds__(NW * 64) k_dec_up(DecArgs a) {
  constexpr bool GT = (VAR & DV_GATED) != 0, NM = (VAR & DV_NO_MEAN) != 0, SR = (VAR & DV_SHARED_RMS) != 0;
  using elem = typename DT::elem;
  constexpr int CH = DEC_CH;
  static_assert(NP * 256 <= NW * 64, "one output entry per thread");
  static_assert(NP <= 4, "s_red holds 4 panels per wave");
  __shared__ float s_zred[NW][16];
  __shared__ float s_ss[NP][16];
  __shared__ f32x4_t s_red[NW][4][64];
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, g = l >> 4, c = l & 15;
  // grid order: shared-expert slices (they need no router result, so they
  // stream from the start), then (routed expert, slice); a gated expert's
  // slices of its NormSiLU input come first, then those of its W_up
  const int bid = blockIdx.x;
  const bool routed = bid >= a.n_shared;
  const int rb = bid - a.n_shared;
  const int spe = GT ? 2 * a.wg_per_e : a.wg_per_e;
  const int e = routed ? rb / spe : 0;
  const int rs = routed ? rb % spe : 0;
  const bool lin = GT && rs >= a.wg_per_e;   // W_up slice of a gated expert: no mean term, no RMS
  const int wgi = lin ? rs - a.wg_per_e : rs;
  const int p0 = routed ? wgi * NP : bid * NP;
  // what the first stream reads: the mean term, or a gated expert's W_up, or
  // (no mean term: an ablation) the expert's own slice
  const char* w_up_e = a.Wup_p + (size_t)e * a.up_stride;
  const bool mean_pass = !lin && !NM;   // stream -Wbar, then W_up[e]
  const char* w_first = lin ? a.Wlin_p + (size_t)e * a.up_stride : (NM ? w_up_e : a.Wbar_p);
  const int nkb = a.nkb_d;
  const int kb_lo = (w * nkb) / NW, kb_hi = ((w + 1) * nkb) / NW;
  const elem* xrow = (const elem*)a.x + (size_t)c * a.d;
  const bool row_ok = c < a.T;
  const bool x_fits = kb_hi - kb_lo <= CH;   // the wave's x fragments fit in registers at once

  i32x4_t xf[CH];
  i32x4_t wf[CH][NP];
  auto load_x = [&](int kb0) {
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int kb = kb0 + u;
      xf[u] = (kb < kb_hi && row_ok) ? load_row_frag<DT>(xrow, kb, g) : zero16();
    }
  };
  auto load_w = [&](const char* wbase, int kb0) {
    const __amdgpu_buffer_rsrc_t rw = buf_rsrc(wbase);
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int kb = kb0 + u;
#pragma unroll
      for (int p = 0; p < NP; ++p)
        wf[u][p] = kb < kb_hi ? ld16_buf(rw, 16u * l, (unsigned)frag_off(p0 + p, kb, nkb)) : zero16();
    }
  };
  f32x4_t acc[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) acc[p] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto mma_chunk = [&](int kb0) {
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      if (kb0 + u < kb_hi) {
#pragma unroll
        for (int p = 0; p < NP; ++p) DT::mma(acc[p], xf[u], wf[u][p]);
      }
    }
  };
  // acc += x . (the NP panels at p0 of wbase) over this wave's k-range; xf
  // and wf may already hold the first chunk's operands
  auto stream = [&](const char* wbase, bool w0_loaded, bool x0_loaded) {
    for (int kb0 = kb_lo; kb0 < kb_hi; kb0 += CH) {
      if (!(x0_loaded && kb0 == kb_lo)) load_x(kb0);
      if (!(w0_loaded && kb0 == kb_lo)) load_w(wbase, kb0);
      mma_chunk(kb0);
    }
  };

  if (routed && a.top_k > 0) {
    // TopK variant: k_dec_topk has routed the batch; x and the first
    // weights load while the expert's flag is read
    load_x(kb_lo);
    load_w(w_first, kb_lo);
    if (a.rflag[e] != 2u) {
      wait_all_mem();
      return;  // no token keeps expert e: none of its weights are read
    }
    stream(w_first, true, true);
    if (mean_pass) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int p = 0; p < NP; ++p) acc[p] = -acc[p];
      stream(w_up_e, false, x_fits);
    }
  } else if (routed) {
    // router logits of expert e for the 16 (padded) token rows
    const float lam_e = a.lam[e];
    const float b_e = a.b_r[e];
    float zp = 0.f;
    const char* wr = a.Wr_p + frag_off(e >> 4, 0, nkb) + (size_t)((e & 15) + 16 * g) * 16;
    for (int kb0 = kb_lo; kb0 < kb_hi; kb0 += CH) {
      load_x(kb0);
      i32x4_t wv[CH];
#pragma unroll
      for (int u = 0; u < CH; ++u) wv[u] = kb0 + u < kb_hi ? ld16(wr + (size_t)(kb0 + u) * FRAG_BYTES) : zero16();
#pragma unroll
      for (int u = 0; u < CH; ++u) {
#pragma unroll
        for (int j = 0; j < DT::EPL; ++j) zp += DT::lane_elem(xf[u], j) * DT::lane_elem(wv[u], j);
      }
    }
    __builtin_amdgcn_sched_barrier(0);   // keep the router's registers apart from the weights'
    if (!x_fits) load_x(kb_lo);
    // the first weights load while the waves combine their logits
    load_w(w_first, kb_lo);
    zp += __shfl_xor(zp, 16);
    zp += __shfl_xor(zp, 32);
    if (g == 0) s_zred[w][c] = zp;
    lds_barrier();   // LDS only: the weight loads stay in flight
    // every wave forms the logits itself (lane: token row c, same order
    // everywhere), so the activity decision needs no further barrier
    float zz = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) zz += s_zred[ww][c];
    zz += b_e;
    const bool act = c < a.T && zz > 0.f && lam_e != 0.f;
    const bool any = __ballot(act) != 0ull;
    if (rs == 0 && w == 0) {
      if (l == 0) a.rflag[e] = any ? 2u : 1u;
      if (l < a.T) {
        a.z[(size_t)l * a.E + e] = zz;
        a.g[(size_t)l * a.E + e] = act ? lam_e * zz : 0.f;
      }
    }
    if (!any) {
      wait_all_mem();
      return;  // inactive expert: none of its weights are read
    }
    // acc = -(x . Wbar) + x . W_up[e]: the NormSiLU mean term and the expert
    // in one fp32 accumulator (a gated expert's W_up slice: acc = x . W_up[e])
    stream(w_first, true, true);
    if (mean_pass) {
      __builtin_amdgcn_sched_barrier(0);   // keep the two streams' registers apart
#pragma unroll
      for (int p = 0; p < NP; ++p) acc[p] = -acc[p];
      // (with a single chunk per wave xf still holds it)
      stream(w_up_e, false, x_fits);
    }
  } else {
    stream(a.Wsu_p, false, false);
  }

  // sum the waves' partial products: one (row, column) entry per thread
#pragma unroll
  for (int p = 0; p < NP; ++p) s_red[w][p][l] = acc[p];
  __syncthreads();
  const bool mine = tid < NP * 256;
  const int pp = tid >> 8, ll = (tid >> 2) & 63, i = tid & 3;
  const int row = 4 * (ll >> 4) + i, col = (p0 + pp) * 16 + (ll & 15);
  float v = 0.f;
  if (mine) {
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) v += s_red[ww][pp][ll][i];
  }
  if (!routed) {
    // shared expert: plain SiLU, stored as down-projection operand fragments
    // (RMS-only NormSiLU: the pre-activation, for k_dec_shared_rms)
    if (mine) {
      if constexpr (SR) a.sraw[(size_t)row * a.Fs + col] = v;
      else *reinterpret_cast<elem*>(a.sactf + frag_elem_off<DT>(row, col)) = DT::from_f32(silu_f(v));
    }
    return;
  }
  if (mine && row < a.T) (lin ? a.ubuf : a.hbuf)[((size_t)e * 16 + row) * a.F + col] = v;
  if (lin) return;
  // per-row sum of squares over this slice: lanes with equal l & 3 of a wave
  // hold one row (4 (w & 3) + (l & 3)) of panel w >> 2, columns l >> 2
  float sq = v * v;
  sq += __shfl_xor(sq, 4);
  sq += __shfl_xor(sq, 8);
  sq += __shfl_xor(sq, 16);
  sq += __shfl_xor(sq, 32);
  if (mine && l < 4) s_ss[pp][row] = sq;
  __syncthreads();
  if (tid < a.T) {
    float ss = 0.f;
#pragma unroll
    for (int p = 0; p < NP; ++p) ss += s_ss[p][tid];
    a.sspart[((size_t)e * a.wg_per_e + wgi) * 16 + tid] = ss;
  }
}

template <class DT, int NW, bool MULTI, bool GATED, bool NO_RMS>
__global__ void __launch_bounds__(NW * 64) k_dec_down(DecArgs a) {
  using elem = typename DT::elem;
  using DN = typename DT::Down;   // operand type of the routed down-projection
  constexpr int UB = DEC_UB;
  constexpr int DP = DEC_DP;
  constexpr int EPL = DT::EPL;
  constexpr int NCOL = DP * 16;
  __shared__ int s_ulist[256];
  __shared__ int s_wcnt[4];
  __shared__ int s_nu;
  __shared__ float s_rinv[DEC_XMAX * 16];
  __shared__ float s_gate[DEC_XMAX * 16];
  __shared__ f32x4_t s_red[NW][4][64];
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, c = l & 15, g = l >> 4;
  const int grp = blockIdx.x % a.n_groups, q = blockIdx.x / a.n_groups;

  // ascending list of the experts that at least one token activated
  const int nwE = (a.E + 63) >> 6;
  const int e_ = w * 64 + l;
  const bool act = (w < nwE) && (e_ < a.E) && (a.rflag[e_] == 2u);
  const unsigned long long bal = __ballot(act);
  if (w < nwE && l == 0) s_wcnt[w] = __popcll(bal);
  __syncthreads();
  if (act) {
    int base = 0;
    for (int ww = 0; ww < w; ++ww) base += s_wcnt[ww];
    s_ulist[base + __popcll(bal & ((1ull << l) - 1ull))] = e_;
  }
  if (tid == 0) {
    int n = 0;
    for (int ww = 0; ww < nwE; ++ww) n += s_wcnt[ww];
    s_nu = n;
  }
  __syncthreads();
  const int nu = s_nu;
  const int n_routed_units = nu * a.nkb_F;
  const int C = n_routed_units + a.nkb_Fs;
  const int lo = (int)(((long long)q * C) / a.Q), hi = (int)(((long long)(q + 1) * C) / a.Q);
  // routed experts with units in [lo, hi): list entries i0 .. i0 + nx - 1
  const int rhi = hi < n_routed_units ? hi : n_routed_units;
  const int i0 = lo < rhi ? lo / a.nkb_F : 0;
  const int nx = lo < rhi ? (rhi - 1) / a.nkb_F - i0 + 1 : 0;

  // weights of one chunk of this wave's units (k-blocks), straight to
  // registers.  Panels past the last output column (d not a multiple of
  // NCOL) read the last panel again and their results are dropped.
  i32x4_t bfr[UB][DP];
  auto load_b = [&](int u0) {
#pragma unroll
    for (int ub = 0; ub < UB; ++ub) {
      const int u = u0 + ub * NW;   // wave-uniform
      const char* B;
      int kb, nkb;
      if (u < rhi) {
        kb = u % a.nkb_F;
        nkb = a.nkb_F;
        B = a.Wdn_p + (size_t)__builtin_amdgcn_readfirstlane(s_ulist[u / a.nkb_F]) * a.dn_stride;
      } else {
        kb = u < hi ? u - n_routed_units : 0;
        nkb = a.nkb_Fs;
        B = a.Wsd_p;
      }
      const __amdgpu_buffer_rsrc_t rb = buf_rsrc(B);
#pragma unroll
      for (int p = 0; p < DP; ++p) {
        int pan = grp * DP + p;
        pan = pan < a.pD ? pan : a.pD - 1;
        bfr[ub][p] = u < hi ? ld16_buf(rb, 16u * l, (unsigned)frag_off(pan, kb, nkb)) : zero16();
      }
    }
  };
  // raw activation operands of a chunk: for a routed unit (expert e, k-block
  // kb) lane (c, g) takes h - m of token row c at the EPL columns its
  // fragment holds (rows past T read nothing: the buffer range check returns
  // zeros), and for gated experts x . W_up[e] at the same place; for a
  // shared unit, the stored fragment
  const __amdgpu_buffer_rsrc_t rh = buf_rsrc(a.hbuf), rs = buf_rsrc(a.sactf);
  const __amdgpu_buffer_rsrc_t ru = buf_rsrc(GATED ? a.ubuf : a.hbuf);
  float hv[UB][EPL];
  float uv[UB][GATED ? EPL : 1];
  auto load_a = [&](int u0) {
#pragma unroll
    for (int ub = 0; ub < UB; ++ub) {
      const int u = u0 + ub * NW;
      i32x4_t r[EPL / 4], r2[EPL / 4];
      if (u < rhi) {
        const int e = s_ulist[u / a.nkb_F], kb = u % a.nkb_F;
        const unsigned off = c < a.T ? 4u * (unsigned)((e * 16 + c) * a.F + kb * DT::KB + EPL * g) : OOB;
#pragma unroll
        for (int k = 0; k < EPL / 4; ++k) r[k] = ld16_buf(rh, off + 16u * k, 0u);
        if constexpr (GATED) {
#pragma unroll
          for (int k = 0; k < EPL / 4; ++k) r2[k] = ld16_buf(ru, off + 16u * k, 0u);
        }
      } else {   // a shared unit, or past the range (reads nothing)
        const unsigned off = u < hi ? (unsigned)((u - n_routed_units) * FRAG_BYTES) + 16u * l : OOB;
        r[0] = ld16_buf(rs, off, 0u);
#pragma unroll
        for (int k = 1; k < EPL / 4; ++k) r[k] = zero16();
        if constexpr (GATED) {
#pragma unroll
          for (int k = 0; k < EPL / 4; ++k) r2[k] = zero16();
        }
      }
#pragma unroll
      for (int k = 0; k < EPL / 4; ++k)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          hv[ub][4 * k + j] = __int_as_float(r[k][j]);
          if constexpr (GATED) uv[ub][4 * k + j] = __int_as_float(r2[k][j]);
        }
    }
  };
  load_b(lo + w);
  load_a(lo + w);
  // 1 / RMS (NormSiLU) and gate of each (expert in range, token row)
  {
    const __amdgpu_buffer_rsrc_t rsp = buf_rsrc(a.sspart), rg = buf_rsrc(a.g);
    const float invF = 1.0f / (float)a.F;
    for (int k = tid; k < nx * 16; k += NW * 64) {
      const int e = s_ulist[i0 + (k >> 4)], t = k & 15;
      float rinv = 0.f, gt = 0.f;
      if (t < a.T) {
        float part_ss[DEC_WGMAX];
#pragma unroll
        for (int wi = 0; wi < DEC_WGMAX; ++wi)   // issued together; slices past wg_per_e read 0
          part_ss[wi] = ld_buf(rsp, wi < a.wg_per_e ? 4u * (unsigned)((e * a.wg_per_e + wi) * 16 + t) : OOB);
        float ss = 0.f;
#pragma unroll
        for (int wi = 0; wi < DEC_WGMAX; ++wi) ss += part_ss[wi];
        rinv = NO_RMS ? 1.0f : 1.0f / sqrtf(ss * invF + a.eps);
        gt = ld_buf(rg, 4u * (unsigned)(t * a.E + e));   // 0 for an inactive pair
      }
      s_rinv[k] = rinv;
      s_gate[k] = gt;
    }
  }
  __syncthreads();

  f32x4_t acc[DP];
#pragma unroll
  for (int p = 0; p < DP; ++p) acc[p] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int u0) {
#pragma unroll
    for (int ub = 0; ub < UB; ++ub) {
      const int u = u0 + ub * NW;
      __builtin_amdgcn_sched_barrier(0);   // one unit's temporaries at a time
      if (u < hi) {
        if (u < n_routed_units) {
          // NormSiLU times the router gate (and, for gated experts, times
          // x . W_up[e]), rounded once to the down-projection operand type
          const int k = (u / a.nkb_F - i0) * 16 + c;
          const float rinv = s_rinv[k], gt = s_gate[k];
#pragma unroll
          for (int j = 0; j < EPL; ++j) {
            if constexpr (GATED) hv[ub][j] = gt != 0.f ? silu_f(hv[ub][j] * rinv) * gt * uv[ub][j] : 0.f;
            else hv[ub][j] = gt != 0.f ? silu_f(hv[ub][j] * rinv) * gt : 0.f;
          }
          const i32x4_t af = DN::pack(hv[ub]);
#pragma unroll
          for (int p = 0; p < DP; ++p) DN::mma(acc[p], af, bfr[ub][p]);
        } else {
          i32x4_t af;
#pragma unroll
          for (int j = 0; j < 4; ++j) af[j] = __float_as_int(hv[ub][j]);
#pragma unroll
          for (int p = 0; p < DP; ++p) DT::mma(acc[p], af, bfr[ub][p]);
        }
      }
    }
  };
  compute(lo + w);
  if constexpr (MULTI) {
    for (int u0 = lo + w + NW * UB; u0 < hi; u0 += NW * UB) {
      load_b(u0);
      load_a(u0);
      compute(u0);
    }
  }
  // sum the waves' partial products, 4 panels at a time through LDS
  float* mypart = a.part + ((size_t)q * a.n_groups + grp) * (16 * NCOL);
#pragma unroll
  for (int h = 0; h < DP / 4; ++h) {
#pragma unroll
    for (int p = 0; p < 4; ++p) s_red[w][p][l] = acc[4 * h + p];
    __syncthreads();
    for (int idx = tid; idx < 1024; idx += NW * 64) {
      const int p = idx >> 8, ll = (idx >> 2) & 63, i = idx & 3;
      const int row = 4 * (ll >> 4) + i, col = (4 * h + p) * 16 + (ll & 15);
      if (row < a.T) {
        float v = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) v += s_red[ww][p][ll][i];
        mypart[row * NCOL + col] = v;
      }
    }
    __syncthreads();
  }
}

// RMS-only NormSiLU of the shared expert (an ablation switch): one workgroup
// per padded token row; s = SiLU(u / sqrt(mean_j u_j^2 + eps)) stored as the
// down-projection operand fragments k_dec_up stores otherwise (rows past T: 0).
template <class DT>
__global__ void __launch_bounds__(256) k_dec_shared_rms(DecArgs a) {
  using elem = typename DT::elem;
  __shared__ float s_part[4];
  const int r = blockIdx.x, tid = threadIdx.x;
  const float* u = a.sraw + (size_t)r * a.Fs;
  float ss = 0.f;
  if (r < a.T)
    for (int j = tid; j < a.Fs; j += 256) ss += u[j] * u[j];
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
  if ((tid & 63) == 0) s_part[tid >> 6] = ss;
  __syncthreads();
  const float tot = s_part[0] + s_part[1] + s_part[2] + s_part[3];
  const float rinv = 1.0f / sqrtf(tot / (float)a.Fs + a.eps);
  for (int j = tid; j < a.Fs; j += 256) {
    const float v = r < a.T ? silu_f(u[j] * rinv) : 0.f;
    *reinterpret_cast<elem*>(a.sactf + frag_elem_off<DT>(r, j)) = DT::from_f32(v);
  }
}

// out[t][c] = sum over the Q reduction splits of the down kernel's partial
// products, in split order (deterministic); 4 consecutive columns per thread.
#ifndef DECO_DEC_SUM_NT
#define DECO_DEC_SUM_NT 64
#endif
// threads per k_dec_sum workgroup: one wave, so T = 8 spreads its 4096
// threads over 64 CUs (same-box A/B, c2: 0.3 us per step faster than 256)
constexpr int DEC_SUM_NT = DECO_DEC_SUM_NT;
template <class DT>
__global__ void __launch_bounds__(DEC_SUM_NT) k_dec_sum(DecArgs a) {
  constexpr int NCOL = DEC_DP * 16;
  const int idx = blockIdx.x * DEC_SUM_NT + threadIdx.x;
  if (idx * 4 >= a.T * a.d) return;
  const int row = (idx * 4) / a.d, col = (idx * 4) % a.d;
  const int grp = col / NCOL, cin = col % NCOL;
  f32x4_t v = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int q0 = 0; q0 < a.Q; q0 += 16) {
    f32x4_t pv[16];
#pragma unroll
    for (int qq = 0; qq < 16; ++qq)   // issued together
      pv[qq] = q0 + qq < a.Q
                   ? *reinterpret_cast<const f32x4_t*>(
                         a.part + ((((size_t)(q0 + qq) * a.n_groups + grp) * 16 + row) * NCOL + cin))
                   : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int qq = 0; qq < 16; ++qq) v += pv[qq];
  }
  typename DT::elem* o = (typename DT::elem*)a.out + (size_t)row * a.d + col;
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = DT::from_f32(v[j]);
}

template <class DT>
void (*up_kernel(int var))(DecArgs) {
  switch (var) {
    case 0: return k_dec_up<DT, DEC_NW, DEC_NP, 0>;
    case 1: return k_dec_up<DT, DEC_NW, DEC_NP, 1>;
    case 2: return k_dec_up<DT, DEC_NW, DEC_NP, 2>;
    case 3: return k_dec_up<DT, DEC_NW, DEC_NP, 3>;
    case 4: return k_dec_up<DT, DEC_NW, DEC_NP, 4>;
    case 5: return k_dec_up<DT, DEC_NW, DEC_NP, 5>;
    case 6: return k_dec_up<DT, DEC_NW, DEC_NP, 6>;
    default: return k_dec_up<DT, DEC_NW, DEC_NP, 7>;
  }
}

template <class DT, bool MULTI>
void (*down_kernel_m(bool gated, bool no_rms))(DecArgs) {
  return gated ? (no_rms ? k_dec_down<DT, DEC_NW, MULTI, true, true> : k_dec_down<DT, DEC_NW, MULTI, true, false>)
               : (no_rms ? k_dec_down<DT, DEC_NW, MULTI, false, true> : k_dec_down<DT, DEC_NW, MULTI, false, false>);
}
template <class DT>
void (*down_kernel(bool multi, bool gated, bool no_rms))(DecArgs) {
  return multi ? down_kernel_m<DT, true>(gated, no_rms) : down_kernel_m<DT, false>(gated, no_rms);
}

template <class DT>
hipError_t decode(const deco_moe_layer* L, const void* x, int T, void* out, hipStream_t s) {
  DecArgs a;
  a.x = x;
  a.out = out;
  a.T = T;
  a.d = L->d;
  a.E = L->E;
  a.F = L->F;
  a.Fs = L->Fs;
  a.nkb_d = L->nkb_d;
  a.nkb_F = L->nkb_F;
  a.nkb_Fs = L->nkb_Fs;
  a.pF = L->pF;
  a.pFs = L->pFs;
  a.pD = L->pD;
  a.n_groups = L->n_groups;
  a.Q = L->dec_q;
  a.n_shared = L->pFs / DEC_NP;
  a.wg_per_e = L->pF / DEC_NP;
  a.top_k = L->cfg.top_k;
  a.gated = L->gated;
  a.no_mean = (L->cfg.normsilu & DECO_NORMSILU_NO_MEAN) != 0;
  a.no_rms = (L->cfg.normsilu & DECO_NORMSILU_NO_RMS) != 0;
  a.sraw = L->cfg.shared_rms ? L->sraw : nullptr;
  a.Wlin_p = L->Wlin_p;
  a.ubuf = L->ubuf;
  a.pR = L->pR;
  a.W = L->W;
  a.mask = L->mask;
  a.Wr_p = L->Wr_p;
  a.Wup_p = L->Wup_p;
  a.Wbar_p = L->Wbar_p;
  a.Wdn_p = L->Wdn16_p;   // fp16 copy for bf16 layers, W_down itself for fp32 layers
  a.Wsu_p = L->Wsu_p;
  a.Wsd_p = L->Wsd_p;
  a.up_stride = L->up_stride;
  a.dn_stride = L->dn_stride;
  a.b_r = L->b_r;
  a.lam = L->lam;
  a.eps = L->cfg.rms_eps;
  a.z = L->z;
  a.g = L->g;
  a.hbuf = L->hbuf;
  a.sspart = L->sspart;
  a.sactf = L->sactf;
  a.rflag = L->rflag;
  a.part = L->part;
  hipError_t err = hipSuccess;
  if (a.top_k > 0) {
    err = deco_host::launch(deco_host::KS_DEC_TOPK, k_dec_topk<DT, 16>, dim3(1), dim3(16 * 64), s, a);
    if (err != hipSuccess) return err;
  }
  const unsigned grid_up = (unsigned)(a.n_shared + L->E * (a.wg_per_e << a.gated));
  const int var = (a.gated ? DV_GATED : 0) | (a.no_mean ? DV_NO_MEAN : 0) | (a.sraw ? DV_SHARED_RMS : 0);
  void (*up)(DecArgs) = up_kernel<DT>(var);
  err = deco_host::launch(deco_host::KS_DEC_UP, up, dim3(grid_up),
                                     dim3(DEC_NW * 64), s, a);
  if (err != hipSuccess) return err;
  if (a.sraw) {
    err = deco_host::launch(deco_host::KS_DEC_UP, k_dec_shared_rms<DT>, dim3(16), dim3(256), s, a);
    if (err != hipSuccess) return err;
  }
  const unsigned grid_dn = (unsigned)(L->n_groups * L->dec_q);
  void (*down)(DecArgs) = down_kernel<DT>(L->dec_multi != 0, a.gated != 0, a.no_rms != 0);
  err = deco_host::launch(deco_host::KS_DEC_DOWN, down, dim3(grid_dn), dim3(DEC_NW * 64), s, a);
  if (err != hipSuccess) return err;
  const unsigned grid_sum = (unsigned)((T * L->d / 4 + DEC_SUM_NT - 1) / DEC_SUM_NT);
  err = deco_host::launch(deco_host::KS_DEC_SUM, k_dec_sum<DT>, dim3(grid_sum), dim3(DEC_SUM_NT), s, a);
  if (err != hipSuccess) return err;
  return hipGetLastError();
}

}  // namespace

namespace deco_host {

// Decode launch shape: the down kernel splits its reduction Q ways so that
// about DECO_DEC_DOWN_WG workgroups stream the down-projection weights.
#ifndef DECO_DEC_DOWN_WG
#define DECO_DEC_DOWN_WG 256
#endif
hipError_t plan_decode(deco_moe_layer* L) {
  int q = (DECO_DEC_DOWN_WG + L->n_groups - 1) / L->n_groups;
  q = q < 1 ? 1 : (q > DEC_QMAX ? DEC_QMAX : q);
  // With every expert active the reduction has C units.  A down workgroup
  // takes ceil(C / q) of them: one chunk of DEC_UB units per wave when that
  // fits (the kernel without a reload loop, which needs fewer registers), and
  // at most DEC_XMAX experts (1/RMS and gates in LDS; a range of n units spans
  // at most n / nkb_F + 2 experts).
  const int C = L->E * L->nkb_F + L->nkb_Fs;
  auto span = [&](int qq) { return (C + qq - 1) / qq; };
  auto xmax = [&](int qq) {
    const int x = span(qq) / L->nkb_F + 2;
    return x < L->E ? x : L->E;
  };
  while (q < DEC_QMAX && (span(q) > DEC_NW * DEC_UB || xmax(q) > DEC_XMAX)) ++q;
  if (xmax(q) > DEC_XMAX || L->pF / DEC_NP > DEC_WGMAX) return hipErrorInvalidValue;
  L->dec_q = q;
  L->dec_multi = span(q) > DEC_NW * DEC_UB;
  L->dec_ok = 1;
  return hipSuccess;
}

hipError_t launch_decode(const deco_moe_layer* L, const void* x, int T, void* out, hipStream_t s) {
  if (L->cfg.dtype == DECO_DT_BF16) return decode<BF16>(L, x, T, out, s);
  return decode<F32>(L, x, T, out, s);
}

}  // namespace deco_host
