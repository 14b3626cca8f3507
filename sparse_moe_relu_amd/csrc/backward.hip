// backward.hip - backward pass of the DECO layer (the training side: DECO
// paper Sec. 2 "Router design", "Expert design" and "Auxiliary training
// objective"; qidianchuan.cn write-up, sections 二 and 三).
//
// Gradients of Loss = sum(dout * out) + reg_coef * mean_t H_t (H_t: entropy
// of token t's gates normalised over its active experts), from x and dout:
//
//   routing          the forward's router / TopK / dispatch kernels recompute
//                    z, g, the masks, m = x.Wbar, s = SiLU(x Ws_up) and the
//                    per-expert token lists.
//   k_bwd_shared     du_s = (dout Ws_down^T) * SiLU'(x Ws_up), two MFMA
//                    passes per 128 x 128 tile.
//   k_pre_expert     (backward mode) per expert tile: recompute h~, r, a;
//                    q = dout W_down[e]^T; dg, dh~; pair rows of dh~ and g*a;
//                    dh~ W_up[e]^T to the pair buffer.
//   k_bwd_token      per token: dm = -sum of its dh~ rows (the mean term),
//                    the entropy term, dz through ReLU * lambda (or the TopK
//                    softmax), ReLU(z) * dg for dlambda; the row dm | dz | du_s.
//   k_bwd_colsum     db_r and dlambda: column sums over tokens, in a fixed
//                    order (two passes).
//   k_bwd_dense_dx   [dm | dz | du_s] . [Wbar^T; W_r^T; Ws_up^T] into pair
//                    slot 0 of each token.
//   k_pre_combine    dx = sum of each token's pair rows (fp32 output).
//   k_bwd_wgrad      every weight gradient as C = sum_k A_k^T B_k over token
//                    rows: x^T [dm | dz | du_s] (the mean term's gradient G,
//                    dW_r, dWs_up), s^T dout (dWs_down), (g a)^T dout per
//                    expert (dW_down), x^T dh~ + G / E per expert (dW_up).
//
// No atomics: every output element is written once by one workgroup, so the
// result is deterministic.
//
// Precision (bf16 layers): the fp32 intermediates that feed products (dh~,
// g*a, the row dm | dz | du_s, s) are kept as two bf16 parts, hi = bf16(v)
// and lo = bf16(v - hi), and multiplied as hi and lo passes: one bf16
// rounding of such an operand costs up to 2^-9 of the largest terms, which on
// heavy-tailed gates reaches several percent of a gradient's RMS.
#include <initializer_list>

#include "prefill_kernels.h"

namespace {

struct BwdArgs {
  const void* x;
  const void* dout;
  unsigned* err;              // device error flags (bit 5: a value outside the fp16 range)
  int T, d, E, F, Fs, W, top_k;
  int Fp, Ep, Fsp, Kc;        // dcat row: dm [Fp] | dz [Ep] | du_s [Fsp]
  int nkb_d, nkb_cat, pFs, pD;
  const char* Wsu_p;
  const char* WsdT_p;
  const char* Bcat_p;
  const char* WbarLo_p;       // bf16 layers: low part of Wbar (K = d, N = F)
  float* mbuf;                // [T][F] m = x . Wbar
  int pF;
  const float* lam;
  const float* z;
  const float* g;
  const uint64_t* mask;
  const float* dgbuf;
  const void* dhbuf;
  const void* dhbuf_lo;       // bf16 layers: low parts of dhbuf
  const int* tok_off;
  void* dcat;
  void* dcat_lo;              // bf16 layers: low parts of dcat
  void* sb_hi;                // [T][Fs] s = SiLU(x Ws_up), high and low parts
  void* sb_lo;
  float* dzbuf;
  float* dlz;
  float* colpart;             // [2][n_chunks][E] partial column sums
  float reg_coef, invT;
  void* ybuf;
  float* db_r;
  float* dlam;
  int32_t* n_active;
};

// du_s = (dout . Ws_down^T) * SiLU'(x . Ws_up) for a 128-row x 128-column tile
// of the shared expert's width, stored into the Fs section of dcat.
template <class DT>
__global__ void __launch_bounds__(256) k_bwd_shared(BwdArgs a) {
  using elem = typename DT::elem;
  using TD = DenseTile<DT>;
  __shared__ i32x4_t lds[TD::LDS_V];
  const int tid = threadIdx.x, w = tid >> 6, wm = w >> 1, wn = w & 1, l = tid & 63, g = l >> 4, c = l & 15;
  const int nct = (a.pFs + GP - 1) / GP;
  const int m0 = (blockIdx.x / nct) * GM, p0 = (blockIdx.x % nct) * GP;
  const elem* x = (const elem*)a.x;
  const elem* dout = (const elem*)a.dout;
  auto clamp_row = [&](int r) { const int rr = m0 + r; return (size_t)(rr < a.T ? rr : a.T - 1); };
  auto row_x = [&](int r) -> const elem* { return x + clamp_row(r) * a.d; };
  auto row_d = [&](int r) -> const elem* { return dout + clamp_row(r) * a.d; };
  auto pan = [&](int p) { return p0 + p < a.pFs ? p0 + p : a.pFs - 1; };
  auto panel_u = [&](int p) -> const char* { return a.Wsu_p + frag_off(pan(p), 0, a.nkb_d); };
  auto panel_d = [&](int p) -> const char* { return a.WsdT_p + frag_off(pan(p), 0, a.nkb_d); };
  f32x4_t us[TD::MB][TD::NBW], ds[TD::MB][TD::NBW];
#pragma unroll
  for (int i = 0; i < TD::MB; ++i)
#pragma unroll
    for (int j = 0; j < TD::NBW; ++j) us[i][j] = ds[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  tile_gemm<DT, TD, true>(lds, row_x, panel_u, a.nkb_d, us);
  tile_gemm<DT, TD, true>(lds, row_d, panel_d, a.nkb_d, ds);
  elem* dcat = (elem*)a.dcat;
  elem* dcat_lo = (elem*)a.dcat_lo;
#pragma unroll
  for (int i = 0; i < TD::MB; ++i) {
    const int r = m0 + wm * (GM / 2) + 16 * i + c;
#pragma unroll
    for (int j = 0; j < TD::NBW; ++j) {
      const int col = (p0 + wn * TD::NBW + j) * 16 + 4 * g;
      if (r < a.T && col < a.Fs) {
        float v[4], sv[4];
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          v[ii] = ds[i][j][ii] * dsilu_f(us[i][j][ii]);
          sv[ii] = silu_f(us[i][j][ii]);
        }
        const size_t o = (size_t)r * a.Kc + a.Fp + a.Ep + col, os = (size_t)r * a.Fs + col;
        store4_split<DT>(dcat + o, dcat_lo + o, v);
        store4_split<DT>((elem*)a.sb_hi + os, (elem*)a.sb_lo + os, sv);
      }
    }
  }
}

template <class DT>
__device__ __forceinline__ void put_split(typename DT::elem* hi, typename DT::elem* lo, size_t i, float v) {
  hi[i] = DT::from_f32(v);
  if constexpr (sizeof(typename DT::elem) == 2) lo[i] = DT::from_f32(v - DT::to_f32(hi[i]));
}

// m += x . Wbar_lo (bf16 layers): the recomputed mean term then carries
// Wbar to about 16 significant bits.  A bf16 Wbar alone costs dW_up over 2 %
// of its RMS when few tokens average the error (T = 1).
// the x . (Wbar - bf16(Wbar)) pass has only F columns: 32-row by 64-column
// tiles with a four-stage ring, so T = 4096 still spreads over 256 workgroups
template <class DT>
using MeanLoTile = Tile<DT, 32, 4, 4>;

template <class DT>
__global__ void __launch_bounds__(256) k_bwd_mean_lo(BwdArgs a) {
  using elem = typename DT::elem;
  using TD = MeanLoTile<DT>;
  __shared__ i32x4_t lds[TD::LDS_V];
  const int tid = threadIdx.x, w = tid >> 6, wm = w >> 1, wn = w & 1, l = tid & 63, g = l >> 4, c = l & 15;
  const int nct = (a.pF + TD::BNP - 1) / TD::BNP;
  const int m0 = (blockIdx.x / nct) * TD::BM, p0 = (blockIdx.x % nct) * TD::BNP;
  const elem* x = (const elem*)a.x;
  auto row = [&](int r) -> const elem* {
    const int rr = m0 + r;
    return x + (size_t)(rr < a.T ? rr : a.T - 1) * a.d;
  };
  auto panel = [&](int p) -> const char* {
    return a.WbarLo_p + frag_off(p0 + p < a.pF ? p0 + p : a.pF - 1, 0, a.nkb_d);
  };
  f32x4_t acc[TD::MB][TD::NBW];
#pragma unroll
  for (int i = 0; i < TD::MB; ++i)
#pragma unroll
    for (int j = 0; j < TD::NBW; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  tile_gemm<DT, TD, true>(lds, row, panel, a.nkb_d, acc);
#pragma unroll
  for (int i = 0; i < TD::MB; ++i) {
    const int r = m0 + wm * (TD::BM / 2) + 16 * i + c;
    if (r >= a.T) continue;
#pragma unroll
    for (int j = 0; j < TD::NBW; ++j) {
      const int p = p0 + wn * TD::NBW + j;
      if (p < a.pF) {
        float4* mp = reinterpret_cast<float4*>(a.mbuf + (size_t)r * a.F + p * 16 + 4 * g);
        float4 v = *mp;
        v.x += acc[i][j][0];
        v.y += acc[i][j][1];
        v.z += acc[i][j][2];
        v.w += acc[i][j][3];
        *mp = v;
      }
    }
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

// One wave per token: dm, the entropy term, dz, ReLU(z) * dg, and the token's
// dcat row (padding columns zeroed: the dense dx product runs over them).
template <class DT>
__global__ void __launch_bounds__(256) k_bwd_token(BwdArgs a) {
  using elem = typename DT::elem;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + w;
  if (t >= a.T) return;
  elem* drow = (elem*)a.dcat + (size_t)t * a.Kc;
  elem* drow_lo = (elem*)a.dcat_lo + (size_t)t * a.Kc;
  const elem* dh = (const elem*)a.dhbuf;
  const elem* dh_lo = (const elem*)a.dhbuf_lo;
  // the mean term: m = x . Wbar feeds every active expert's h~ with sign -1
  const int s0 = a.tok_off[t] + 1, s1 = a.tok_off[t + 1];
  for (int f = l; f < a.Fp; f += 64) {
    float v = 0.f;
    if (f < a.F)
      for (int sl = s0; sl < s1; ++sl) {
        v += DT::to_f32(dh[(size_t)sl * a.F + f]);
        if constexpr (sizeof(elem) == 2) v += DT::to_f32(dh_lo[(size_t)sl * a.F + f]);
      }
    put_split<DT>(drow, drow_lo, f, f < a.F ? -v : 0.f);
  }
  // router
  const uint64_t* mrow = a.mask + (size_t)t * a.W;
  bool act[4];
  float gv[4], dg[4];
  float S = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int e = l + 64 * k;
    act[k] = e < a.E && ((mrow[e >> 6] >> (e & 63)) & 1ull);
    gv[k] = act[k] ? a.g[(size_t)t * a.E + e] : 0.f;
    dg[k] = act[k] ? a.dgbuf[(size_t)t * a.E + e] : 0.f;
    S += gv[k];
  }
  S = wave_sum(S);
  if (a.top_k == 0 && a.reg_coef != 0.f && S > 0.f) {
    // d/dg of reg_coef/T * H_t, H_t = -sum p log p with p = g / S
    float H = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (act[k]) {
        const float p = gv[k] / S;
        H -= p * logf(p);
      }
    H = wave_sum(H);
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (act[k]) dg[k] += a.reg_coef * a.invT * (-(logf(gv[k] / S) + H) / S);
  }
  float pdg = 0.f;
  if (a.top_k > 0) {
#pragma unroll
    for (int k = 0; k < 4; ++k) pdg += gv[k] * dg[k];
    pdg = wave_sum(pdg);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int e = l + 64 * k;
    if (e >= a.Ep) continue;
    float dz = 0.f, dl = 0.f;
    if (act[k]) {
      if (a.top_k > 0) {
        dz = gv[k] * (dg[k] - pdg);   // softmax over the kept logits
      } else {
        dz = a.lam[e] * dg[k];        // g = lambda * ReLU(z)
        dl = fmaxf(a.z[(size_t)t * a.E + e], 0.f) * dg[k];
      }
    }
    if (e < a.E) {
      a.dzbuf[(size_t)t * a.E + e] = dz;
      a.dlz[(size_t)t * a.E + e] = dl;
    }
    put_split<DT>(drow, drow_lo, a.Fp + e, dz);
  }
  for (int j = a.Fs + l; j < a.Fsp; j += 64) put_split<DT>(drow, drow_lo, a.Fp + a.Ep + j, 0.f);
}

// Column sums over tokens of dzbuf (db_r) and dlz (dlambda).  Pass 1: chunk b
// of 64 tokens, one thread per expert, into colpart; pass 2: the chunks in
// order.  blockIdx.y selects the quantity.
constexpr int CS_ROWS = 64;
__global__ void __launch_bounds__(256) k_bwd_colsum1(BwdArgs a) {
  const int e = threadIdx.x, q = blockIdx.y, b = blockIdx.x;
  const int nch = (a.T + CS_ROWS - 1) / CS_ROWS;
  if (e >= a.E) return;
  const float* src = q ? a.dlz : a.dzbuf;
  const int t0 = b * CS_ROWS, t1 = t0 + CS_ROWS < a.T ? t0 + CS_ROWS : a.T;
  float v = 0.f;
#pragma unroll 16
  for (int t = t0; t < t1; ++t) v += src[(size_t)t * a.E + e];
  a.colpart[((size_t)q * nch + b) * a.E + e] = v;
}

__global__ void __launch_bounds__(256) k_bwd_colsum2(BwdArgs a) {
  const int e = threadIdx.x, q = blockIdx.y;
  const int nch = (a.T + CS_ROWS - 1) / CS_ROWS;
  if (q == 0 && e == 0 && a.n_active) a.n_active[0] = a.tok_off[a.T] - a.T;   // slots minus the shared ones
  if (e >= a.E) return;
  // chunks in order; sixteen loads in flight at a time, added in order
  float v = 0.f;
  int b = 0;
  for (; b + 16 <= nch; b += 16) {
    float p[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) p[u] = a.colpart[((size_t)q * nch + b + u) * a.E + e];
#pragma unroll
    for (int u = 0; u < 16; ++u) v += p[u];
  }
  for (; b < nch; ++b) v += a.colpart[((size_t)q * nch + b) * a.E + e];
  (q ? a.dlam : a.db_r)[e] = v;
}

// dx_dense = [dm | dz | du_s] . [Wbar^T; W_r^T; Ws_up^T] into pair slot 0.
template <class DT>
__global__ void __launch_bounds__(256) k_bwd_dense_dx(BwdArgs a) {
  using elem = typename DT::elem;
  using PT = typename DT::pair;
  using TD = DenseTile<DT>;
  __shared__ i32x4_t lds[TD::LDS_V];
  const int tid = threadIdx.x, w = tid >> 6, wm = w >> 1, wn = w & 1, l = tid & 63, g = l >> 4, c = l & 15;
  const int nct = (a.pD + GP - 1) / GP;
  const int m0 = (blockIdx.x / nct) * GM, p0 = (blockIdx.x % nct) * GP;
  const elem* dcat = (const elem*)a.dcat;
  auto row = [&](int r) -> const elem* {
    const int rr = m0 + r;
    return dcat + (size_t)(rr < a.T ? rr : a.T - 1) * a.Kc;
  };
  auto panel = [&](int p) -> const char* {
    return a.Bcat_p + frag_off(p0 + p < a.pD ? p0 + p : a.pD - 1, 0, a.nkb_cat);
  };
  f32x4_t acc[TD::MB][TD::NBW];
#pragma unroll
  for (int i = 0; i < TD::MB; ++i)
#pragma unroll
    for (int j = 0; j < TD::NBW; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  tile_gemm<DT, TD, true>(lds, row, panel, a.nkb_cat, acc);
  if constexpr (sizeof(elem) == 2) {   // the low parts of the rows
    const elem* dcat_lo = (const elem*)a.dcat_lo;
    auto row_lo = [&](int r) -> const elem* {
      const int rr = m0 + r;
      return dcat_lo + (size_t)(rr < a.T ? rr : a.T - 1) * a.Kc;
    };
    tile_gemm<DT, TD, true>(lds, row_lo, panel, a.nkb_cat, acc);
  }
  PT* yb = (PT*)a.ybuf;
  bool bad = false;
#pragma unroll
  for (int i = 0; i < TD::MB; ++i) {
    const int r = m0 + wm * (GM / 2) + 16 * i + c;
    if (r >= a.T) continue;
    const size_t base = (size_t)a.tok_off[r] * a.d;
#pragma unroll
    for (int j = 0; j < TD::NBW; ++j) {
      const int p = p0 + wn * TD::NBW + j;
      if (p < a.pD) store4_pair(yb + base + p * 16 + 4 * g, acc[i][j], bad);
    }
  }
  if (bad) atomicOr(a.err, 32u);
}

// ---------------------------------------------------------------------------
// Weight gradients: C[M][N] = sum over K rows of A_k^T B_k, A_k and B_k rows
// of row-major layer-dtype matrices (a token's row, or a pair slot's row).
// A workgroup owns one 128 x 128 tile of C (of one expert, for per-expert
// jobs) over its K range; dense jobs split K into `ksplit` ranges whose
// partial tiles k_bwd_wsum adds in order, so every element is written once.
// Each step stages 32 rows of A and of B in LDS transposed (column-major: a
// lane's MFMA fragment, EPL consecutive k of one column, is then one 16-byte
// read).  A lane loads two rows' 16-byte chunks and stores each column's
// pair of values with one LDS write.  One LDS buffer (30 KiB: four
// workgroups per CU hide each other's load latency); loads run two steps
// ahead in two register sets, row indices three (two index sets, each fetched
// before the data loads that precede its use: vector loads retire in issue
// order, so a wait for an index never waits for data requested after it).
struct WArgs {
  int M, N, K;                // C shape; K = rows of a dense job (per expert: the expert's count)
  int per_expert;             // 1: one C per expert over its token list
  int a_slot, b_slot;         // per-expert jobs: row index of A (B) = pair slot (1) or token (0)
  const void* A;
  const void* B;
  const void* A2;             // optional low parts of A (B), same layout: C = (A + A2)^T (B + B2)
  const void* B2;             // without the A2^T B2 term
  int lda, ldb;               // row pitches, elements
  int tm, tn;                 // 128 x 128 tiles of one C
  int nsec;                   // column sections of C, each stored to its own matrix
  int sc0[3], scnt[3], sld[3];
  float* sptr[3];
  size_t c_estride;           // per-expert stride of the outputs (elements)
  const float* add;           // optional: C += add_scale * add[m][n] (ld N)
  float add_scale;
  int ksplit;                 // dense jobs: K ranges (1: none); > 1 writes partial tiles to `part`
  float* part;                // [ksplit][M][N] partial sums
  const int* ecnt;
  const int* list_tok;
  const int* slot_list;
  int Tcap;
};

#ifndef DECO_WG_KS
#define DECO_WG_KS 32
#endif
constexpr int WG_KS = DECO_WG_KS;   // rows per step (32 or 64)
#ifndef DECO_WG_OCC
#define DECO_WG_OCC (WG_KS == 32 ? 3 : 2)
#endif
constexpr int WG_OCC = DECO_WG_OCC;   // workgroups per CU (registers, LDS)

template <class DT>
struct WShape {
  using elem = typename DT::elem;
  static constexpr int ES = (int)sizeof(elem);
  static constexpr int PITCH = WG_KS + 16 / ES;   // LDS elements per column (a 16-byte pad)
  static constexpr int PLANE = 128 * PITCH;       // elements per plane
  static constexpr int MAX_PLANES = ES == 2 ? 3 : 2;   // operand planes (value, low part) per buffer
  static constexpr int LDS_BYTES = MAX_PLANES * PLANE * ES;
};

template <class DT, bool SA, bool SB>
__device__ __forceinline__ void wgrad_tile(const WArgs& a, int bid, char* lds_raw) {
  using elem = typename DT::elem;
  using WS = WShape<DT>;
  constexpr int ES = WS::ES, EPL = DT::EPL, KB = DT::KB, KS = WG_KS;
  constexpr int PITCH = WS::PITCH, PLANE = WS::PLANE;
  constexpr int EPC = 16 / ES;                // elements per 16-byte chunk
  constexpr int CPR = 128 / EPC;              // chunks per 128-column row segment
  constexpr int TPL = KS / 16;                // rows per lane task (one LDS store per column)
  constexpr int NKP = KS / TPL;               // row pairs per step
  constexpr int NLD = NKP * CPR / 256;        // lane tasks per plane and step
  static_assert((NKP * CPR) % 256 == 0 && KS % KB == 0, "step shape");
  constexpr int NA = SA ? 2 : 1, NB = SB ? 2 : 1;
  static_assert(NA + NB <= WS::MAX_PLANES, "LDS planes");
  elem* sA = reinterpret_cast<elem*>(lds_raw);   // [NA][PLANE]
  elem* sB = sA + NA * PLANE;                    // [NB][PLANE]
  const int tid = threadIdx.x, w = tid >> 6, wm = w >> 1, wn = w & 1, l = tid & 63, g = l >> 4, c = l & 15;
  const int per = a.tm * a.tn;
  const int e = a.per_expert ? bid / per : 0;   // expert, or K range of a split dense job
  const int tile = bid % per;
  const int m0 = (tile / a.tn) * 128, n0 = (tile % a.tn) * 128;
  // rows k0 .. k0 + K - 1 of the job
  int k0 = 0, K = a.per_expert ? a.ecnt[e] : a.K;
  if (!a.per_expert && a.ksplit > 1) {
    const int len = ((a.K + a.ksplit - 1) / a.ksplit + KS - 1) / KS * KS;
    const int kb = bid / per;
    k0 = kb * len;
    K = a.K - k0 < len ? a.K - k0 : len;
    if (K < 0) K = 0;
  }
  const int nsteps = (K + KS - 1) / KS;
  const elem* Ap[2] = {(const elem*)a.A, (const elem*)a.A2};
  const elem* Bp[2] = {(const elem*)a.B, (const elem*)a.B2};
  // this thread's rows of a step: 2 kp and 2 kp + 1; its chunks tid / NKP + (256 / NKP) u
  const int kp = tid % NKP;
  // Row of step s.  Ranks past K read the last real row (finite data at a
  // valid address): their B values are zeroed when staged, and nothing else
  // is masked, since out-of-range columns only reach outputs that are
  // dropped.  No load sits under a branch and no loaded value is touched
  // before it is staged (either would make the compiler wait for the
  // prefetch right after issuing it).
  const int* lst_a = a.a_slot ? a.slot_list : a.list_tok;
  const int* lst_b = a.b_slot ? a.slot_list : a.list_tok;
  const int eoff = a.per_expert ? e : 0;
  auto idx = [&](int s, int t, const int* lst) -> int {
    const int k = s * KS + TPL * kp + t;
    const int kc = k < K ? k : K - 1;
    const int r = lst[(size_t)eoff * a.Tcap + kc];   // read by dense jobs too (kc < T <= Tcap): no branch
    return a.per_expert ? r : k0 + kc;
  };
  struct Regs {
    i32x4_t va[NA][NLD][TPL];
    i32x4_t vb[NB][NLD][TPL];
  };
  static_assert(TPL == 2 || TPL == 4, "rows per lane task");
  Regs R0, R1;
  struct Idx {
    int ia[TPL], ib[TPL];
  };
  Idx X0, X1;
  auto fetch_idx = [&](Idx& X, int s) {
#pragma unroll
    for (int t = 0; t < TPL; ++t) {
      X.ia[t] = idx(s, t, lst_a);
      X.ib[t] = idx(s, t, lst_b);
    }
  };
  auto load = [&](Regs& R, const Idx& X) {
    const int* ia = X.ia;
    const int* ib = X.ib;
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int ch = tid / NKP + (256 / NKP) * u;
      const int ca = m0 + ch * EPC, cb = n0 + ch * EPC;
#pragma unroll
      for (int t = 0; t < TPL; ++t) {
        const size_t oa = (size_t)ia[t] * a.lda + (ca < a.M ? ca : 0);
        const size_t ob = (size_t)ib[t] * a.ldb + (cb < a.N ? cb : 0);
#pragma unroll
        for (int h = 0; h < NA; ++h) R.va[h][u][t] = ld16(Ap[h] + oa);
#pragma unroll
        for (int h = 0; h < NB; ++h) R.vb[h][u][t] = ld16(Bp[h] + ob);
      }
    }
  };
  // column col of a plane gets the TPL rows' values at k = TPL kp .. in one store
  auto put = [&](elem* plane, int col, const i32x4_t (&r)[TPL], int j) {
    elem* dst = plane + col * PITCH + TPL * kp;
    auto el = [&](int t) { return reinterpret_cast<const elem*>(&r[t])[j]; };
    if constexpr (ES == 2 && TPL == 2) {
      *reinterpret_cast<uint32_t*>(dst) = (uint32_t)el(0) | ((uint32_t)el(1) << 16);
    } else if constexpr (ES == 2) {
      *reinterpret_cast<uint2*>(dst) = make_uint2((uint32_t)el(0) | ((uint32_t)el(1) << 16),
                                                  (uint32_t)el(2) | ((uint32_t)el(3) << 16));
    } else if constexpr (TPL == 2) {
      *reinterpret_cast<float2*>(dst) = make_float2(el(0), el(1));
    } else {
      *reinterpret_cast<float4*>(dst) = make_float4(el(0), el(1), el(2), el(3));
    }
  };
  auto stage = [&](Regs& R, int s) {
    // B rows past K contribute nothing
#pragma unroll
    for (int t = 0; t < TPL; ++t) {
      const int mk = s * KS + TPL * kp + t < K ? -1 : 0;
#pragma unroll
      for (int h = 0; h < NB; ++h)
#pragma unroll
        for (int u = 0; u < NLD; ++u)
#pragma unroll
          for (int q = 0; q < 4; ++q) R.vb[h][u][t][q] &= mk;
    }
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int ch = tid / NKP + (256 / NKP) * u;
#pragma unroll
      for (int j = 0; j < EPC; ++j) {
#pragma unroll
        for (int h = 0; h < NA; ++h) put(sA + h * PLANE, ch * EPC + j, R.va[h][u], j);
#pragma unroll
        for (int h = 0; h < NB; ++h) put(sB + h * PLANE, ch * EPC + j, R.vb[h][u], j);
      }
    }
  };
  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto frag = [&](const elem* plane, int col, int kb) {
    return *reinterpret_cast<const i32x4_t*>(plane + col * PITCH + kb * KB + EPL * g);
  };
  auto compute = [&]() {
#pragma unroll
    for (int kb = 0; kb < KS / KB; ++kb) {
      i32x4_t af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = frag(sA, wm * 64 + 16 * i + c, kb);
#pragma unroll
      for (int j = 0; j < 4; ++j) bf[j] = frag(sB, wn * 64 + 16 * j + c, kb);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) DT::mma(acc[i][j], af[i], bf[j]);
      if constexpr (SA) {   // + A_lo^T B
#pragma unroll
        for (int i = 0; i < 4; ++i) af[i] = frag(sA + PLANE, wm * 64 + 16 * i + c, kb);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) DT::mma(acc[i][j], af[i], bf[j]);
      }
      if constexpr (SB) {   // + A^T B_lo
#pragma unroll
        for (int j = 0; j < 4; ++j) bf[j] = frag(sB + PLANE, wn * 64 + 16 * j + c, kb);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) DT::mma(acc[i][j], af[i], bf[j]);
      }
    }
  };
  // steps s, s+1 alternate register sets R0 / R1 and index sets X0 / X1.
  // Loads and stages run unconditionally (past the last step they read
  // clamped rows): with no load under a branch the compiler's waits cover
  // exactly the rows being staged.
  if (nsteps > 0) {
    fetch_idx(X0, 0);
    fetch_idx(X1, 1);
    load(R0, X0);
    fetch_idx(X0, 2);
    load(R1, X1);
  }
  for (int s = 0; s < nsteps; s += 2) {
    // R0 holds step s, R1 step s + 1; X0 holds step s + 2
    stage(R0, s);
    lds_barrier();   // LDS only: the prefetched rows stay in flight
    fetch_idx(X1, s + 3);
    load(R0, X0);
    compute();
    lds_barrier();   // the buffer is read by every wave before the next stage
    if (s + 1 >= nsteps) break;
    // R1 holds step s + 1, R0 step s + 2; X1 holds step s + 3
    stage(R1, s + 1);
    lds_barrier();
    fetch_idx(X0, s + 4);
    load(R1, X1);
    compute();
    lds_barrier();
  }
  // lane (c, g) of acc[i][j]: rows m0 + wm*64 + 16 i + 4 g + ii, column n0 + wn*64 + 16 j + c
  if (!a.per_expert && a.ksplit > 1) {
    float* pt = a.part + (size_t)(bid / per) * a.M * a.N;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + wn * 64 + 16 * j + c;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int m = m0 + wm * 64 + 16 * i + 4 * g + ii;
          if (m < a.M && n < a.N) pt[(size_t)m * a.N + n] = acc[i][j][ii];
        }
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + wn * 64 + 16 * j + c;
    if (n >= a.N) continue;
    int sec = -1;
    for (int q = 0; q < a.nsec; ++q)
      if (n >= a.sc0[q] && n < a.sc0[q] + a.scnt[q]) sec = q;
    if (sec < 0) continue;   // a padding column
    float* out = a.sptr[sec] + (size_t)e * a.c_estride + (n - a.sc0[sec]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int m = m0 + wm * 64 + 16 * i + 4 * g + ii;
        if (m < a.M) {
          float v = acc[i][j][ii];
          if (a.add) v += a.add_scale * a.add[(size_t)m * a.N + n];
          out[(size_t)m * a.sld[sec]] = v;
        }
      }
  }
}

template <class DT, bool SA, bool SB>
__global__ void __launch_bounds__(256, WG_OCC) k_bwd_wgrad(WArgs a) {
  __shared__ __attribute__((aligned(16))) char lds_raw[WShape<DT>::LDS_BYTES];
  wgrad_tile<DT, SA, SB>(a, blockIdx.x, lds_raw);
}

// C = sum of a split dense job's partial tiles in K order, stored through the
// job's column sections (4 consecutive columns per thread)
__global__ void __launch_bounds__(256) k_bwd_wsum(WArgs a) {
  const long long idx = ((long long)blockIdx.x * 256 + threadIdx.x) * 4;
  if (idx >= (long long)a.M * a.N) return;
  const int m = (int)(idx / a.N), n = (int)(idx % a.N);
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int q = 0; q < a.ksplit; ++q) {
    const float4 p = *reinterpret_cast<const float4*>(a.part + (size_t)q * a.M * a.N + idx);
    v.x += p.x;
    v.y += p.y;
    v.z += p.z;
    v.w += p.w;
  }
  const float vv[4] = {v.x, v.y, v.z, v.w};
  for (int u = 0; u < 4; ++u) {
    const int nn = n + u;
    for (int q = 0; q < a.nsec; ++q)
      if (nn >= a.sc0[q] && nn < a.sc0[q] + a.scnt[q]) a.sptr[q][(size_t)m * a.sld[q] + (nn - a.sc0[q])] = vv[u];
  }
}

template <class DT>
void (*expert_kernel_bwd(int pF))(PreArgs) {
  return pF == 2 ? k_pre_expert<DT, 2, XM_BWD>
       : pF == 4 ? k_pre_expert<DT, 4, XM_BWD>
       : pF == 8 ? k_pre_expert<DT, 8, XM_BWD> : k_pre_expert<DT, 16, XM_BWD>;
}

WArgs wjob(int M, int N, const void* A, int lda, const void* B, int ldb) {
  WArgs w;
  memset(&w, 0, sizeof(w));
  w.M = M;
  w.N = N;
  w.A = A;
  w.B = B;
  w.lda = lda;
  w.ldb = ldb;
  w.tm = (M + 127) / 128;
  w.tn = (N + 127) / 128;
  return w;
}

template <class DT>
hipError_t backward(const deco_moe_layer* L, const void* x, const void* dout, int T, float reg_coef,
                    const deco_moe_grads* gr, hipStream_t s) {
  using deco_host::launch;
  PreArgs a = fill_pre_args(L, x, T, gr->dx);
  a.dout = dout;
  a.WdnT_p = L->WdnT_p;
  a.WupT_p = L->WupT_p;
  a.dgbuf = L->dgbuf;
  a.dhbuf = L->dhbuf;
  a.agbuf = L->agbuf;
  a.dhbuf_lo = L->dhbuf_lo;
  a.agbuf_lo = L->agbuf_lo;
  a.slot_list = L->slot_list;
  BwdArgs b;
  memset(&b, 0, sizeof(b));
  b.x = x;
  b.dout = dout;
  b.err = L->dec_err;
  b.T = T;
  b.d = L->d;
  b.E = L->E;
  b.F = L->F;
  b.Fs = L->Fs;
  b.W = L->W;
  b.top_k = L->cfg.top_k;
  b.Fp = L->Fp;
  b.Ep = L->Ep;
  b.Fsp = L->Fsp;
  b.Kc = L->Fp + L->Ep + L->Fsp;
  b.nkb_d = L->nkb_d;
  b.nkb_cat = L->nkb_cat;
  b.pFs = L->pFs;
  b.pD = L->pD;
  b.Wsu_p = L->Wsu_p;
  b.WsdT_p = L->WsdT_p;
  b.Bcat_p = L->Bcat_p;
  b.WbarLo_p = L->WbarLo_p;
  b.mbuf = L->mbuf;
  b.pF = L->pF;
  b.lam = L->lam;
  b.z = L->z;
  b.g = L->g;
  b.mask = L->mask;
  b.dgbuf = L->dgbuf;
  b.dhbuf = L->dhbuf;
  b.dhbuf_lo = L->dhbuf_lo;
  b.tok_off = L->tok_off;
  b.dcat = L->dcat;
  b.dcat_lo = L->dcat_lo;
  b.sb_hi = L->sb_hi;
  b.sb_lo = L->sb_lo;
  b.dzbuf = L->dzbuf;
  b.dlz = L->dlz;
  b.colpart = L->colpart;
  b.reg_coef = reg_coef;
  b.invT = 1.0f / (float)T;
  b.ybuf = L->ybuf;
  b.db_r = gr->db_r;
  b.dlam = gr->dlambda;
  b.n_active = gr->n_active_pairs;

  const unsigned mtiles = (unsigned)((T + GM - 1) / GM);
  // weight gradients
  const int d = L->d, E = L->E, F = L->F, Fs = L->Fs, Kc = b.Kc;
  const int Tcap = L->maxT < 16 ? 16 : L->maxT;
  // x^T [dm | dz | du_s]: G (Wbar's gradient), dW_r, dWs_up
  WArgs w1 = wjob(d, Kc, x, d, L->dcat, Kc);
  w1.B2 = L->dcat_lo;
  w1.K = T;
  w1.nsec = 3;
  w1.sc0[0] = 0;
  w1.scnt[0] = F;
  w1.sld[0] = F;
  w1.sptr[0] = L->gbuf;
  w1.sc0[1] = L->Fp;
  w1.scnt[1] = E;
  w1.sld[1] = E;
  w1.sptr[1] = gr->dW_r;
  w1.sc0[2] = L->Fp + L->Ep;
  w1.scnt[2] = Fs;
  w1.sld[2] = Fs;
  w1.sptr[2] = gr->dWs_up;
  // s^T dout: dWs_down
  WArgs w2 = wjob(Fs, d, L->sb_hi, Fs, dout, d);
  w2.A2 = L->sb_lo;
  w2.K = T;
  w2.nsec = 1;
  w2.scnt[0] = d;
  w2.sld[0] = d;
  w2.sptr[0] = gr->dWs_down;
  // per expert (g a)^T dout: dW_down
  WArgs w3 = wjob(F, d, L->agbuf, F, dout, d);
  w3.A2 = L->agbuf_lo;
  w3.per_expert = 1;
  w3.a_slot = 1;
  w3.nsec = 1;
  w3.scnt[0] = d;
  w3.sld[0] = d;
  w3.sptr[0] = gr->dW_down;
  w3.c_estride = (size_t)F * d;
  // per expert x^T dh~ + G / E: dW_up
  WArgs w4 = wjob(d, F, x, d, L->dhbuf, F);
  w4.B2 = L->dhbuf_lo;
  w4.per_expert = 1;
  w4.b_slot = 1;
  w4.nsec = 1;
  w4.scnt[0] = F;
  w4.sld[0] = F;
  w4.sptr[0] = gr->dW_up;
  w4.c_estride = (size_t)d * F;
  w4.add = L->gbuf;
  w4.add_scale = 1.0f / (float)E;
  for (WArgs* wp : {&w1, &w2, &w3, &w4}) {   // dense jobs read the lists too (branch-free index loads)
    wp->ecnt = L->ecnt;
    wp->list_tok = L->list_tok;
    wp->slot_list = L->slot_list;
    wp->Tcap = Tcap;
  }
  // the dense jobs (K = T) in K ranges of at least 512 rows, four at most,
  // reduced in order afterwards
  const int ks = T >= 2048 ? 4 : (T >= 1024 ? 2 : 1);
  w1.ksplit = w2.ksplit = ks;
  w1.part = L->wpart;
  w2.part = L->wpart2;   // w1 and w2 run on different streams
  auto run_job = [&](WArgs& wj, hipStream_t st) -> hipError_t {
    const unsigned grid = (unsigned)(wj.tm * wj.tn * (wj.per_expert ? E : wj.ksplit > 1 ? wj.ksplit : 1));
    void (*kw)(WArgs) = k_bwd_wgrad<DT, false, false>;
    if constexpr (sizeof(typename DT::elem) == 2) {   // the low-part passes exist for bf16 layers only
      if (wj.A2) kw = k_bwd_wgrad<DT, true, false>;
      else if (wj.B2) kw = k_bwd_wgrad<DT, false, true>;
    } else {
      wj.A2 = wj.B2 = nullptr;
    }
    hipError_t e = launch(deco_host::KS_BWD_WGRAD, kw, dim3(grid), dim3(256), st, wj);
    if (e == hipSuccess && !wj.per_expert && wj.ksplit > 1)
      e = launch(deco_host::KS_BWD_WGRAD, k_bwd_wsum, dim3((unsigned)(((long long)wj.M * wj.N / 4 + 255) / 256)),
                 dim3(256), st, wj);
    return e;
  };

  // Three streams, forked from the caller's stream and joined back into it
  // through events, so the call stays ordered on the caller's stream as a
  // whole.  The caller's stream runs routing, the shared rows, the expert
  // kernel, the token kernel, G and dW_up; once the expert kernel is done a
  // side stream runs dW_down and dWs_down, and once the token kernel is done
  // another runs the column sums, dense dx and the dx combine.
  hipStream_t s2 = L->bwd_side[0], s3 = L->bwd_side[1];
  hipEvent_t ev_expert = L->bwd_ev[0], ev_join2 = L->bwd_ev[1], ev_token = L->bwd_ev[2], ev_join3 = L->bwd_ev[3];
  hipError_t err = launch_routing<DT>(L, a, T, s);
  if (err == hipSuccess && L->WbarLo_p)
    err = launch(deco_host::KS_BWD_SHARED, k_bwd_mean_lo<DT>,
                 dim3((unsigned)((T + MeanLoTile<DT>::BM - 1) / MeanLoTile<DT>::BM) *
                      ((L->pF + MeanLoTile<DT>::BNP - 1) / MeanLoTile<DT>::BNP)),
                 dim3(256), s, b);
  if (err == hipSuccess)
    err = launch(deco_host::KS_BWD_SHARED, k_bwd_shared<DT>, dim3(mtiles * ((L->pFs + GP - 1) / GP)), dim3(256), s, b);
  if (err == hipSuccess)
    err = launch(deco_host::KS_BWD_EXPERT, expert_kernel_bwd<DT>(L->pF), dim3(L->bwd_grid), dim3(256), s, a);
  if (err == hipSuccess) err = hipEventRecord(ev_expert, s);
  if (err == hipSuccess) err = hipStreamWaitEvent(s2, ev_expert, 0);
  if (err == hipSuccess) err = run_job(w3, s2);
  if (err == hipSuccess) err = run_job(w2, s2);
  if (err == hipSuccess) err = hipEventRecord(ev_join2, s2);
  if (err == hipSuccess)
    err = launch(deco_host::KS_BWD_TOKEN, k_bwd_token<DT>, dim3((unsigned)((T + 3) / 4)), dim3(256), s, b);
  if (err == hipSuccess) err = hipEventRecord(ev_token, s);
  if (err == hipSuccess) err = hipStreamWaitEvent(s3, ev_token, 0);
  const unsigned nch = (unsigned)((T + CS_ROWS - 1) / CS_ROWS);
  if (err == hipSuccess) err = launch(deco_host::KS_BWD_COLSUM, k_bwd_colsum1, dim3(nch, 2), dim3(256), s3, b);
  if (err == hipSuccess) err = launch(deco_host::KS_BWD_COLSUM, k_bwd_colsum2, dim3(1, 2), dim3(256), s3, b);
  if (err == hipSuccess)
    err = launch(deco_host::KS_BWD_DENSE_DX, k_bwd_dense_dx<DT>, dim3(mtiles * ((L->pD + GP - 1) / GP)), dim3(256),
                 s3, b);
  if (err == hipSuccess)
    err = launch(deco_host::KS_BWD_COMBINE, k_pre_combine<DT, true>,
                 dim3((unsigned)(((long long)T * (L->d / 8) + 255) / 256)), dim3(256), s3, a);
  if (err == hipSuccess) err = hipEventRecord(ev_join3, s3);
  // dW_up (w4) after w1: its epilogue adds G / E from w1
  if (err == hipSuccess) err = run_job(w1, s);
  if (err == hipSuccess) err = run_job(w4, s);
  if (err == hipSuccess) err = hipStreamWaitEvent(s, ev_join3, 0);
  if (err == hipSuccess) err = hipStreamWaitEvent(s, ev_join2, 0);
  if (err != hipSuccess) return err;
  return hipGetLastError();
}

}  // namespace

namespace deco_host {

hipError_t launch_backward(const deco_moe_layer* L, const void* x, const void* dout, int T, float reg_coef,
                           const deco_moe_grads* gr, hipStream_t s) {
  if (L->cfg.dtype == DECO_DT_BF16) return backward<BF16>(L, x, dout, T, reg_coef, gr, s);
  return backward<F32>(L, x, dout, T, reg_coef, gr, s);
}

// persistent grid of the backward expert kernel (as for the forward one)
hipError_t plan_backward(deco_moe_layer* L) {
  void (*kx)(PreArgs) = L->cfg.dtype == DECO_DT_BF16 ? expert_kernel_bwd<BF16>(L->pF) : expert_kernel_bwd<F32>(L->pF);
  int occ = 0;
  hipError_t err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kx, 256, 0);
  if (err != hipSuccess) return err;
  int grid = (occ < 1 ? 1 : occ) * (L->n_cu < 1 ? 1 : L->n_cu);
  L->bwd_grid = (grid + NXCD - 1) / NXCD * NXCD;
  // the side stream (default priority) and its fork/join events
  for (int i = 0; i < 2 && err == hipSuccess; ++i) err = hipStreamCreateWithFlags(&L->bwd_side[i], hipStreamNonBlocking);
  for (int i = 0; i < 6 && err == hipSuccess; ++i) err = hipEventCreateWithFlags(&L->bwd_ev[i], hipEventDisableTiming);
  return err;
}

}  // namespace deco_host
