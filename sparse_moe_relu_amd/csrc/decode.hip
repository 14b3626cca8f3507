// decode.hip - weight-streaming forward path for small batches (T <= 16).
//
// At decode sizes the layer is a handful of matrix-vector products over the
// weights, so its cost is the HBM traffic of the weights it touches.  The
// point of ReLU routing with sparse experts is that inactive routed experts
// cost nothing: the DECO paper (Sec. 1 and the Sec. 4 acceleration paragraph
// with Table 4) attributes its speedup to skipping the memory traffic of
// inactive experts.  Two kernels:
//
//   k_dec_up   one workgroup per (routed expert, 32 columns of F), per 32
//              columns of the inter-expert mean Wbar, and per 32 columns of
//              the shared expert.  A routed workgroup first computes its
//              expert's router logits for the batch (router: linear
//              projection + bias, ReLU, per-expert scale; DECO paper Sec. 2
//              "Router design") and exits before touching any expert weight
//              when no token activates the expert.  Otherwise it streams its
//              slice of W_up[e] through v_mfma 16x16 products (tokens padded
//              to 16 rows).  The Wbar workgroups compute the mean term
//              m = x.Wbar once for all experts.  The last workgroup to finish
//              the rows of an expert (counted per expert, the Wbar workgroups
//              included) applies NormSiLU to the full F-wide rows
//              (qidianchuan.cn write-up, section 二: subtract the mean term,
//              RMS inside the expert, then SiLU), multiplies by the gate and
//              stores the result as down-projection operand fragments, as a
//              hi + lo pair of bf16 values.
//   k_dec_down one workgroup per (64 output columns, 1/Q of the reduction).
//              The reduction runs over the k-blocks of the experts that at
//              least one token activated, then the shared expert; the last
//              workgroup of a column group sums the Q partials in a fixed
//              order (deterministic) and writes out.
#include "deco_common.h"
#include "deco_internal.h"

using namespace deco;

namespace {

struct DecArgs {
  const void* x;
  void* out;
  int T, d, E, F, Fs;
  int nkb_d, nkb_F, nkb_Fs, pF, pFs, n_groups, Q;
  const char* Wr_p;
  const char* Wup_p;
  const char* Wbar_p;
  const char* Wdn_p;
  const char* Wsu_p;
  const char* Wsd_p;
  size_t up_stride, dn_stride;
  const float* b_r;
  const float* lam;
  float eps;
  float* z;
  float* g;
  float* mbuf;
  float* hbuf;
  char* actf;
  char* sactf;
  unsigned* eact;
  unsigned* cnt_up;
  unsigned* cnt_dn;
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
constexpr int DEC_NP = DECO_DEC_NP;   // 16-column panels per up-projection workgroup
constexpr int DEC_CH = DECO_DEC_CH;   // k-blocks held in registers per wave at a time
constexpr int DEC_QMAX = 32;          // largest K-split of the down kernel (host clamps dec_q)

// NormSiLU of the 16 (padded) token rows of each expert in `list`, times the
// gate, stored as down-projection operand fragments (hi, then lo for bf16).
// Called by the workgroup that saw the experts' arrival counts reach their
// target.  Rows are processed RB at a time per wave so their loads overlap.
template <class DT, int NW>
__device__ void dec_finalize(const DecArgs& a, const int* list, int n) {
  using elem = typename DT::elem;
  constexpr int RB = 4;
  constexpr int NPART = DT::SPLIT ? 2 : 1;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const float invF = 1.0f / (float)a.F;
  const int nrows = n * 16;
  const __amdgpu_buffer_rsrc_t rg = dev_rsrc(a.g), rh = dev_rsrc(a.hbuf), rm = dev_rsrc(a.mbuf);
  for (int r0 = w * RB; r0 < nrows; r0 += NW * RB) {
    float hv[RB][4], mv[RB][4], gate[RB];
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      const int r = r0 + rr;
      const int e = r < nrows ? list[r >> 4] : 0, t = r & 15;
      const bool ok = r < nrows;
      // inactive pairs have g == 0; rows past T are padding
      gate[rr] = (ok && t < a.T) ? ld_dev_buf(rg, 4u * (unsigned)(t * a.E + e)) : 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int f = l + 64 * q;
        const bool okf = ok && f < a.F;
        hv[rr][q] = okf ? ld_dev_buf(rh, 4u * (unsigned)((e * 16 + t) * a.F + f)) : 0.f;
        mv[rr][q] = okf ? ld_dev_buf(rm, 4u * (unsigned)(t * a.F + f)) : 0.f;
      }
    }
#pragma unroll
    for (int rr = 0; rr < RB; ++rr)
#pragma unroll
      for (int q = 0; q < 4; ++q) hv[rr][q] -= mv[rr][q];
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      const int r = r0 + rr;
      if (r >= nrows) break;
      const int e = list[r >> 4], t = r & 15;
      float ss = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) ss += hv[rr][q] * hv[rr][q];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
      const float inv_r = 1.0f / sqrtf(ss * invF + a.eps);
      char* act_e = a.actf + (size_t)e * a.nkb_F * NPART * FRAG_BYTES;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int f = l + 64 * q;
        if (f < a.F) {
          const float v = gate[rr] != 0.f ? silu_f(hv[rr][q] * inv_r) * gate[rr] : 0.f;
          char* frag = act_e + (size_t)(f / DT::KB) * NPART * FRAG_BYTES + frag_elem_off<DT>(t, f % DT::KB);
          elem hi, lo;
          split_hi_lo<DT>(v, hi, lo);
          *reinterpret_cast<elem*>(frag) = hi;
          if (DT::SPLIT) *reinterpret_cast<elem*>(frag + FRAG_BYTES) = lo;
        }
      }
    }
  }
  for (int k = tid; k < n; k += NW * 64) a.eact[list[k]] = 1u;
}

template <class DT, int NW, int NP>
__global__ void __launch_bounds__(NW * 64) k_dec_up(DecArgs a) {
  using elem = typename DT::elem;
  constexpr int CH = DEC_CH;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, c = l & 15;
  const int wg_per_e = a.pF / NP;        // workgroups per routed expert
  const int n_wbar = a.pF / NP;          // workgroups of the mean term
  const unsigned target = (unsigned)(wg_per_e + n_wbar);
  // grid order: mean-term slices, shared-expert slices, then routed slices
  // (the first two need no router result, so they stream from the start)
  const int n_shared = a.pFs / NP;
  const int bid = blockIdx.x;
  const int kind = bid < n_wbar ? 1 : (bid < n_wbar + n_shared ? 2 : 0);   // routed / mean / shared
  const int rb = bid - n_wbar - n_shared;
  const int e = kind == 0 ? rb / wg_per_e : 0;
  const int p0 = kind == 0 ? (rb % wg_per_e) * NP : (kind == 1 ? bid * NP : (bid - n_wbar) * NP);
  const int nkb = a.nkb_d;
  const int kb_lo = (w * nkb) / NW, kb_hi = ((w + 1) * nkb) / NW;
  const elem* xrow = (const elem*)a.x + (size_t)c * a.d;
  const bool row_ok = c < a.T;

  __shared__ float s_zred[NW][16];
  __shared__ int s_last;
  __shared__ int s_nfin;
  __shared__ int s_fin[256];
  __shared__ f32x4_t s_red[NW][NP][64];

  i32x4_t xf[CH];
  if (kind == 0) {
    // router logits of expert e for the 16 (padded) token rows
    const float lam_e = a.lam[e];
    const float b_e = a.b_r[e];
    float zp = 0.f;
    const char* wr = a.Wr_p + frag_off(e >> 4, 0, nkb) + (size_t)((e & 15) + 16 * g) * 16;
    for (int kb0 = kb_lo; kb0 < kb_hi; kb0 += CH) {
      i32x4_t wv[CH];
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        const int kb = kb0 + u;
        xf[u] = (kb < kb_hi && row_ok) ? load_row_frag<DT>(xrow, kb, g) : zero16();
        wv[u] = kb < kb_hi ? ld16(wr + (size_t)kb * FRAG_BYTES) : zero16();
      }
#pragma unroll
      for (int u = 0; u < CH; ++u) {
#pragma unroll
        for (int j = 0; j < DT::EPL; ++j) zp += DT::lane_elem(xf[u], j) * DT::lane_elem(wv[u], j);
      }
    }
    zp += __shfl_xor(zp, 16);
    zp += __shfl_xor(zp, 32);
    if (g == 0) s_zred[w][c] = zp;
    __syncthreads();
    // every thread forms the T logits itself (same order everywhere), so the
    // activity decision needs no further barrier
    bool any = false;
    float z_mine = 0.f;
    for (int t = 0; t < a.T; ++t) {
      float zz = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) zz += s_zred[ww][t];
      zz += b_e;
      any |= zz > 0.f && lam_e != 0.f;
      if (t == tid) z_mine = zz;
    }
    if (p0 == 0 && tid < a.T) {
      const bool act = z_mine > 0.f && lam_e != 0.f;
      a.z[(size_t)tid * a.E + e] = z_mine;
      st_dev(&a.g[(size_t)tid * a.E + e], act ? lam_e * z_mine : 0.f);
    }
    if (!any) {
      if (p0 == 0 && tid == 0) a.eact[e] = 0u;
      return;  // inactive expert: none of its weights are read
    }
  }

  // h[16 x (NP*16)] = x[16 x d] . Wslice[d x (NP*16)]
  const char* wbase = kind == 0 ? a.Wup_p + (size_t)e * a.up_stride : (kind == 1 ? a.Wbar_p : a.Wsu_p);
  const bool xf_valid = kind == 0 && (kb_hi - kb_lo <= CH);
  f32x4_t acc[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) acc[p] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int kb0 = kb_lo; kb0 < kb_hi; kb0 += CH) {
    if (!xf_valid) {
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        const int kb = kb0 + u;
        xf[u] = (kb < kb_hi && row_ok) ? load_row_frag<DT>(xrow, kb, g) : zero16();
      }
    }
    i32x4_t wf[CH][NP];
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int kb = kb0 + u;
#pragma unroll
      for (int p = 0; p < NP; ++p)
        wf[u][p] = kb < kb_hi ? ld16(wbase + frag_off(p0 + p, kb, nkb) + (size_t)l * 16) : zero16();
    }
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      if (kb0 + u < kb_hi) {
#pragma unroll
        for (int p = 0; p < NP; ++p) DT::mma(acc[p], xf[u], wf[u][p]);
      }
    }
  }
#pragma unroll
  for (int p = 0; p < NP; ++p) s_red[w][p][l] = acc[p];
  __syncthreads();
  for (int idx = tid; idx < NP * 64 * 4; idx += NW * 64) {
    const int p = idx >> 8, ll = (idx >> 2) & 63, i = idx & 3;
    float v = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) v += s_red[ww][p][ll][i];
    const int row = 4 * (ll >> 4) + i, col = (p0 + p) * 16 + (ll & 15);
    if (kind == 0) {
      st_dev(&a.hbuf[((size_t)e * 16 + row) * a.F + col], v);
    } else if (kind == 1) {
      st_dev(&a.mbuf[(size_t)row * a.F + col], v);
    } else {
      // shared expert: plain SiLU, stored as down-projection operand fragments
      *reinterpret_cast<elem*>(a.sactf + frag_elem_off<DT>(row, col)) = DT::from_f32(silu_f(v));
    }
  }
  if (kind == 2) return;

  // arrival counting: each expert finishes once its own slices and all the
  // mean-term slices are written; that last workgroup applies NormSiLU
  wait_all_mem();
  __syncthreads();
  if (kind == 0) {
    if (tid == 0) {
      s_last = (arrive(&a.cnt_up[e]) == target - 1u) ? 1 : 0;
      s_fin[0] = e;
    }
    __syncthreads();
    if (!s_last) return;
    dec_finalize<DT, NW>(a, s_fin, 1);
  } else {
    if (tid == 0) s_nfin = 0;
    __syncthreads();
    for (int ee = tid; ee < a.E; ee += NW * 64) {
      if (arrive(&a.cnt_up[ee]) == target - 1u) s_fin[atomicAdd(&s_nfin, 1)] = ee;
    }
    __syncthreads();
    const int nfin = s_nfin;
    if (nfin > 0) dec_finalize<DT, NW>(a, s_fin, nfin);
  }
}

template <class DT, int NW>
__global__ void __launch_bounds__(NW * 64) k_dec_down(DecArgs a) {
  using elem = typename DT::elem;
  constexpr int UB = 4;  // units (k-blocks) in flight per wave
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int grp = blockIdx.x % a.n_groups, q = blockIdx.x / a.n_groups;
  constexpr int NPART = DT::SPLIT ? 2 : 1;
  // the up kernel has completed: clear its per-expert arrival counters
  if (blockIdx.x == 0)
    for (int e = tid; e < a.E; e += NW * 64) st_dev_u32(&a.cnt_up[e], 0u);

  __shared__ int s_ulist[256];
  __shared__ int s_wcnt[4];
  __shared__ int s_nu;
  __shared__ int s_last;
  __shared__ f32x4_t s_red[NW][4][64];

  // ascending list of the experts that at least one token activated
  const int nwE = (a.E + 63) >> 6;
  const int e_ = w * 64 + l;
  const bool act = (w < nwE) && (e_ < a.E) && (a.eact[e_] != 0u);
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

  f32x4_t acc[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) acc[p] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int u0 = lo + w; u0 < hi; u0 += NW * UB) {
    i32x4_t af[UB], al[UB], bfr[UB][4];
#pragma unroll
    for (int ub = 0; ub < UB; ++ub) {
      const int u = u0 + ub * NW;
      if (u < hi) {
        const char* A;
        const char* B;
        int kb, nkb;
        if (u < n_routed_units) {
          const int e = s_ulist[u / a.nkb_F];
          kb = u % a.nkb_F;
          nkb = a.nkb_F;
          A = a.actf + ((size_t)e * a.nkb_F + kb) * NPART * FRAG_BYTES;
          B = a.Wdn_p + (size_t)e * a.dn_stride;
        } else {
          kb = u - n_routed_units;
          nkb = a.nkb_Fs;
          A = a.sactf + (size_t)kb * FRAG_BYTES;
          B = a.Wsd_p;
        }
        af[ub] = ld16(A + (size_t)l * 16);
        al[ub] = (DT::SPLIT && u < n_routed_units) ? ld16(A + FRAG_BYTES + (size_t)l * 16) : zero16();
#pragma unroll
        for (int p = 0; p < 4; ++p) bfr[ub][p] = ld16(B + frag_off(grp * 4 + p, kb, nkb) + (size_t)l * 16);
      } else {
        af[ub] = zero16();
        al[ub] = zero16();
#pragma unroll
        for (int p = 0; p < 4; ++p) bfr[ub][p] = zero16();
      }
    }
#pragma unroll
    for (int ub = 0; ub < UB; ++ub) {
      const int u = u0 + ub * NW;
      if (u < hi) {
#pragma unroll
        for (int p = 0; p < 4; ++p) DT::mma(acc[p], af[ub], bfr[ub][p]);
        if (DT::SPLIT && u < n_routed_units) {
#pragma unroll
          for (int p = 0; p < 4; ++p) DT::mma(acc[p], al[ub], bfr[ub][p]);
        }
      }
    }
  }
#pragma unroll
  for (int p = 0; p < 4; ++p) s_red[w][p][l] = acc[p];
  __syncthreads();
  float* mypart = a.part + ((size_t)q * a.n_groups + grp) * 1024;
  for (int idx = tid; idx < 1024; idx += NW * 64) {
    const int p = idx >> 8, ll = (idx >> 2) & 63, i = idx & 3;
    float v = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) v += s_red[ww][p][ll][i];
    const int row = 4 * (ll >> 4) + i, col = p * 16 + (ll & 15);
    st_dev(&mypart[row * 64 + col], v);
  }
  wait_all_mem();
  __syncthreads();
  if (tid == 0) s_last = (arrive(&a.cnt_dn[grp]) == (unsigned)(a.Q - 1)) ? 1 : 0;
  __syncthreads();
  if (!s_last) return;
  elem* out = (elem*)a.out;
  const __amdgpu_buffer_rsrc_t rp = dev_rsrc(a.part);
  for (int idx = tid; idx < a.T * 64; idx += NW * 64) {
    const int row = idx >> 6, col = idx & 63;
    float pv[DEC_QMAX];
#pragma unroll
    for (int qq = 0; qq < DEC_QMAX; ++qq)
      pv[qq] = qq < a.Q ? ld_dev_buf(rp, 4u * (unsigned)(((qq * a.n_groups + grp) << 10) + row * 64 + col)) : 0.f;
    float v = 0.f;
#pragma unroll
    for (int qq = 0; qq < DEC_QMAX; ++qq) v += pv[qq];   // fixed order: deterministic
    out[(size_t)row * a.d + grp * 64 + col] = DT::from_f32(v);
  }
  if (tid == 0) st_dev_u32(&a.cnt_dn[grp], 0u);
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
  a.n_groups = L->n_groups;
  a.Q = L->dec_q;
  a.Wr_p = L->Wr_p;
  a.Wup_p = L->Wup_p;
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
  a.hbuf = L->hbuf;
  a.actf = L->actf;
  a.sactf = L->sactf;
  a.eact = L->eact;
  a.cnt_up = L->cnt_up;
  a.cnt_dn = L->cnt_dn;
  a.part = L->part;
  const unsigned grid_up = (unsigned)((L->E + 1) * (L->pF / DEC_NP) + L->pFs / DEC_NP);
  hipError_t err = deco_host::launch(deco_host::KS_DEC_UP, k_dec_up<DT, DEC_NW, DEC_NP>, dim3(grid_up),
                                     dim3(DEC_NW * 64), s, a);
  if (err != hipSuccess) return err;
  const unsigned grid_dn = (unsigned)(L->n_groups * L->dec_q);
  err = deco_host::launch(deco_host::KS_DEC_DOWN, k_dec_down<DT, DEC_NW>, dim3(grid_dn), dim3(DEC_NW * 64), s, a);
  if (err != hipSuccess) return err;
  return hipGetLastError();
}

}  // namespace

namespace deco_host {

// Decode launch shape: the down kernel splits its reduction Q ways so that
// about DECO_DEC_DOWN_WG workgroups stream the down-projection weights (256
// measured best on the d = 2048 layer among 128 .. 1024: fewer partials to
// sum at the end, still one workgroup per CU streaming).
#ifndef DECO_DEC_DOWN_WG
#define DECO_DEC_DOWN_WG 256
#endif
hipError_t plan_decode(deco_moe_layer* L) {
  int q = (DECO_DEC_DOWN_WG + L->n_groups - 1) / L->n_groups;
  L->dec_q = q < 1 ? 1 : (q > DEC_QMAX ? DEC_QMAX : q);
  L->dec_ok = 1;
  return hipSuccess;
}

hipError_t launch_decode(const deco_moe_layer* L, const void* x, int T, void* out, hipStream_t s) {
  if (L->cfg.dtype == DECO_DT_BF16) return decode<BF16>(L, x, T, out, s);
  return decode<F32>(L, x, T, out, s);
}

}  // namespace deco_host
