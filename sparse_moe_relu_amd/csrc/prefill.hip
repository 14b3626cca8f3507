// prefill.hip - bucketed forward path for large batches.
//
//   k_pre_router_shared  one GEMM over x for the router columns, the columns
//                        of the inter-expert mean Wbar and the shared expert's
//                        up-projection.  Router epilogue: logits + b_r, gates
//                        lambda_e * ReLU(z), active-expert bit masks (DECO
//                        paper Sec. 2 "Router design"; zero or negative scores
//                        are ignored: qidianchuan.cn write-up, section 二,
//                        router).  Mean epilogue: m = x.Wbar in fp32 (the
//                        NormSiLU mean term, same for every expert).  Shared
//                        epilogue: SiLU, stored for the shared down-projection.
//   k_pre_dispatch       per-expert token buckets ("expert batching"), built
//                        with wave ballots and a workgroup prefix scan:
//                        ascending token lists, and for every (token, expert)
//                        pair its slot in a token-major pair buffer.
//   k_pre_expert         persistent grouped kernel over (expert, 64-token
//                        tile): gathered x rows . W_up[e] on MFMA, minus the
//                        mean term, NormSiLU on the F-wide rows in registers,
//                        then the down-projection (activations as a hi + lo
//                        bf16 pair), written ungated to the token's pair slot
//                        in fp16 (11-bit significand; a bf16 pair buffer
//                        costs up to 4 % of RMS(out) on heavy-tailed gates).
//   k_pre_shared_down    shared down-projection GEMM whose epilogue adds each
//                        token's expert outputs times their gates in fp32
//                        (the weighted combine; DECO paper Sec. 2 "Router
//                        design": the router assigns each expert a weight), in
//                        ascending expert order, then rounds to the dtype.
#include "deco_common.h"
#include "deco_internal.h"

using namespace deco;

namespace {

struct PreArgs {
  const void* x;
  void* out;
  int T, Tcap, d, E, F, Fs, W;
  int nkb_d, nkb_F, nkb_Fs, pR, pF, pD, pFs;
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
  uint64_t* mask;
  int* tok_off;
  int* ecnt;
  int* list_tok;
  int* list_slot;
  void* sbuf;
  void* ybuf;
};

constexpr int BM = 64;   // token rows per tile (4 waves x 16)

// --------------------------------------------------------------------------
template <class DT>
__global__ void __launch_bounds__(256) k_pre_router_shared(PreArgs a) {
  using elem = typename DT::elem;
  constexpr int CH = 4;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, c = l & 15;
  const int mt = blockIdx.x, nt = blockIdx.y;
  const int nRt = a.pR / 4, nMt = (a.pF + 3) / 4;
  const int kind = nt < nRt ? 0 : (nt < nRt + nMt ? 1 : 2);    // router / mean / shared
  const bool is_router = kind == 0;
  const int pbase = kind == 0 ? nt * 4 : (kind == 1 ? (nt - nRt) * 4 : (nt - nRt - nMt) * 4);
  const int np = kind == 0 ? 4 : min(4, (kind == 1 ? a.pF : a.pFs) - pbase);
  const char* Wb = kind == 0 ? a.Wr_p : (kind == 1 ? a.Wbar_p : a.Wsu_p);
  const int row = mt * BM + w * 16 + c;
  const bool row_ok = row < a.T;
  const elem* xrow = (const elem*)a.x + (size_t)row * a.d;

  f32x4_t acc[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) acc[p] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int kb0 = 0; kb0 < a.nkb_d; kb0 += CH) {
    i32x4_t xf[CH], wf[CH][4];
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int kb = kb0 + u;
      xf[u] = (kb < a.nkb_d && row_ok) ? load_row_frag<DT>(xrow, kb, g) : zero16();
#pragma unroll
      for (int p = 0; p < 4; ++p)
        wf[u][p] = (kb < a.nkb_d && p < np) ? ld16(Wb + frag_off(pbase + p, kb, a.nkb_d) + (size_t)l * 16)
                                            : zero16();
    }
#pragma unroll
    for (int u = 0; u < CH; ++u)
#pragma unroll
      for (int p = 0; p < 4; ++p) DT::mma(acc[p], xf[u], wf[u][p]);
  }

  const int rbase = mt * BM + w * 16 + 4 * g;
  if (is_router) {
    uint32_t bits[4][4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int e = nt * 64 + p * 16 + c;
      const bool e_ok = e < a.E;
      const float be = e_ok ? a.b_r[e] : 0.f;
      const float le = e_ok ? a.lam[e] : 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = rbase + i;
        const bool ok = e_ok && r < a.T;
        const float zv = acc[p][i] + be;
        const bool act = ok && zv > 0.f && le != 0.f;
        if (ok) {
          a.z[(size_t)r * a.E + e] = zv;
          a.g[(size_t)r * a.E + e] = act ? le * zv : 0.f;
        }
        const unsigned long long bal = __ballot(act);
        bits[p][i] = (uint32_t)((bal >> (16 * g)) & 0xFFFFull);
      }
    }
    if (c == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = rbase + i;
        if (r < a.T) {
          uint64_t word = 0;
#pragma unroll
          for (int p = 0; p < 4; ++p) word |= (uint64_t)bits[p][i] << (16 * p);
          a.mask[(size_t)r * a.W + nt] = word;
        }
      }
    }
  } else if (kind == 1) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      if (p < np) {
        const int col = (pbase + p) * 16 + c;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = rbase + i;
          if (r < a.T) a.mbuf[(size_t)r * a.F + col] = acc[p][i];
        }
      }
    }
  } else {
    elem* sb = (elem*)a.sbuf;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      if (p < np) {
        const int col = (pbase + p) * 16 + c;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = rbase + i;
          if (r < a.T) sb[(size_t)r * a.Fs + col] = DT::from_f32(silu_f(acc[p][i]));
        }
      }
    }
  }
}

// --------------------------------------------------------------------------
// Exclusive scan of one int per thread over a 256-thread workgroup.
__device__ int block_excl_scan(int v, int* s_tmp, int* total) {
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
  for (int ww = 0; ww < 4; ++ww) {
    const int t = s_tmp[ww];
    if (ww < w) base += t;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return base + incl - v;
}

__global__ void __launch_bounds__(256) k_pre_dispatch(PreArgs a) {
  __shared__ int s_tmp1[4], s_tmp2[4];
  const int e = blockIdx.x, tid = threadIdx.x;
  const int wi = e >> 6, bit = e & 63;
  int run_tok = 0, run_e = 0;
  for (int t0 = 0; t0 < a.T; t0 += 256) {
    const int t = t0 + tid;
    const bool valid = t < a.T;
    int cnt = 0, below = 0;
    bool act = false;
    if (valid) {
      for (int ww = 0; ww < a.W; ++ww) {
        const uint64_t m = a.mask[(size_t)t * a.W + ww];
        cnt += __popcll(m);
        if (ww < wi) below += __popcll(m);
        if (ww == wi) {
          below += __popcll(m & ((1ull << bit) - 1ull));
          act = (m >> bit) & 1ull;
        }
      }
    }
    int tot_tok, tot_e;
    const int off_t = run_tok + block_excl_scan(cnt, s_tmp1, &tot_tok);
    const int rank = run_e + block_excl_scan(act ? 1 : 0, s_tmp2, &tot_e);
    if (valid && e == 0) a.tok_off[t] = off_t;
    if (act) {
      a.list_tok[(size_t)e * a.Tcap + rank] = t;
      a.list_slot[(size_t)e * a.Tcap + rank] = off_t + below;
    }
    run_tok += tot_tok;
    run_e += tot_e;
  }
  if (tid == 0) {
    a.ecnt[e] = run_e;
    if (e == 0) a.tok_off[a.T] = run_tok;
  }
}

// --------------------------------------------------------------------------
template <class DT, int NPF>
__global__ void __launch_bounds__(256) k_pre_expert(PreArgs a) {
  using elem = typename DT::elem;
  constexpr int F = NPF * 16;
  constexpr int CH = 4;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, c = l & 15;
  constexpr int NPART = DT::SPLIT ? 2 : 1;
  __shared__ int s_toff[257];
  __shared__ elem s_a[NPART][4][16][F];

  if (tid == 0) {
    int acc = 0;
    for (int e = 0; e < a.E; ++e) {
      s_toff[e] = acc;
      acc += (a.ecnt[e] + BM - 1) / BM;
    }
    s_toff[a.E] = acc;
  }
  __syncthreads();
  const int NT = s_toff[a.E];
  const float invF = 1.0f / (float)F;
  for (int tile = blockIdx.x; tile < NT; tile += gridDim.x) {
    int lo = 0, hi = a.E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_toff[mid] <= tile) lo = mid; else hi = mid;
    }
    const int e = lo;
    const int n_e = a.ecnt[e];
    const int r0 = (tile - s_toff[e]) * BM + w * 16;
    const int* ltok = a.list_tok + (size_t)e * a.Tcap;
    const int* lslot = a.list_slot + (size_t)e * a.Tcap;

    // up-projection of the gathered rows, all F columns
    const int myrow = r0 + c;
    const int tok = myrow < n_e ? ltok[myrow] : -1;
    const elem* xrow = (const elem*)a.x + (size_t)(tok < 0 ? 0 : tok) * a.d;
    const char* Wu = a.Wup_p + (size_t)e * a.up_stride;
    f32x4_t acc[NPF];
#pragma unroll
    for (int p = 0; p < NPF; ++p) acc[p] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int kb0 = 0; kb0 < a.nkb_d; kb0 += CH) {
      i32x4_t xf[CH];
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        const int kb = kb0 + u;
        xf[u] = (kb < a.nkb_d && tok >= 0) ? load_row_frag<DT>(xrow, kb, g) : zero16();
      }
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        const int kb = kb0 + u;
        if (kb < a.nkb_d) {
#pragma unroll
          for (int p = 0; p < NPF; ++p) {
            const i32x4_t wv = ld16(Wu + frag_off(p, kb, a.nkb_d) + (size_t)l * 16);
            DT::mma(acc[p], xf[u], wv);
          }
        }
      }
    }

    // NormSiLU: subtract the mean term, RMS over the F columns of the row
    // (spread over the 16 lanes of a lane group and the NPF panels), SiLU,
    // times the gate; stored to LDS as hi (+ lo) parts
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = r0 + 4 * g + i;
      const int tk = rr < n_e ? ltok[rr] : -1;
      const float* mrow = a.mbuf + (size_t)(tk < 0 ? 0 : tk) * F;
      float ss = 0.f;
#pragma unroll
      for (int p = 0; p < NPF; ++p) {
        const float hv = tk >= 0 ? acc[p][i] - mrow[p * 16 + c] : 0.f;
        acc[p][i] = hv;
        ss += hv * hv;
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) ss += __shfl_xor(ss, o);
      const float inv_r = 1.0f / sqrtf(ss * invF + a.eps);
#pragma unroll
      for (int p = 0; p < NPF; ++p) {
        const float v = tk >= 0 ? silu_f(acc[p][i] * inv_r) : 0.f;
        elem hi, lo;
        split_hi_lo<DT>(v, hi, lo);
        s_a[0][w][4 * g + i][p * 16 + c] = hi;
        if (DT::SPLIT) s_a[NPART - 1][w][4 * g + i][p * 16 + c] = lo;
      }
    }
    __syncthreads();

    // down-projection, 64 output columns at a time, into the pair slots
    i32x4_t af[F / DT::KB], alo[F / DT::KB];
#pragma unroll
    for (int kb = 0; kb < F / DT::KB; ++kb) {
      af[kb] = load_row_frag<DT>(&s_a[0][w][c][0], kb, g);
      alo[kb] = DT::SPLIT ? load_row_frag<DT>(&s_a[NPART - 1][w][c][0], kb, g) : zero16();
    }
    const char* Wd = a.Wdn_p + (size_t)e * a.dn_stride;
    typename DT::pair* yb = (typename DT::pair*)a.ybuf;
    int slot[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = r0 + 4 * g + i;
      slot[i] = rr < n_e ? lslot[rr] : -1;
    }
    for (int n4 = 0; n4 < a.pD / 4; ++n4) {
      f32x4_t y[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) y[p] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < F / DT::KB; ++kb) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const i32x4_t wv = ld16(Wd + frag_off(n4 * 4 + p, kb, a.nkb_F) + (size_t)l * 16);
          DT::mma(y[p], af[kb], wv);
          if (DT::SPLIT) DT::mma(y[p], alo[kb], wv);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (slot[i] >= 0) {
#pragma unroll
          for (int p = 0; p < 4; ++p)
            yb[(size_t)slot[i] * a.d + (n4 * 4 + p) * 16 + c] = (typename DT::pair)y[p][i];
        }
      }
    }
    __syncthreads();
  }
}

// --------------------------------------------------------------------------
template <class DT>
__global__ void __launch_bounds__(256) k_pre_shared_down(PreArgs a) {
  using elem = typename DT::elem;
  constexpr int CH = 4;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, c = l & 15;
  const int mt = blockIdx.x, nt = blockIdx.y;
  const int row = mt * BM + w * 16 + c;
  const bool row_ok = row < a.T;
  const elem* srow = (const elem*)a.sbuf + (size_t)row * a.Fs;
  f32x4_t acc[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) acc[p] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int kb0 = 0; kb0 < a.nkb_Fs; kb0 += CH) {
    i32x4_t sf[CH], wf[CH][4];
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int kb = kb0 + u;
      sf[u] = (kb < a.nkb_Fs && row_ok) ? load_row_frag<DT>(srow, kb, g) : zero16();
#pragma unroll
      for (int p = 0; p < 4; ++p)
        wf[u][p] = kb < a.nkb_Fs ? ld16(a.Wsd_p + frag_off(nt * 4 + p, kb, a.nkb_Fs) + (size_t)l * 16) : zero16();
    }
#pragma unroll
    for (int u = 0; u < CH; ++u)
#pragma unroll
      for (int p = 0; p < 4; ++p) DT::mma(acc[p], sf[u], wf[u][p]);
  }
  const typename DT::pair* yb = (const typename DT::pair*)a.ybuf;
  elem* out = (elem*)a.out;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = mt * BM + w * 16 + 4 * g + i;
    if (r < a.T) {
      float v[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) v[p] = acc[p][i];
      // the token's pair slots hold its active experts in ascending order
      int sl = a.tok_off[r];
      for (int wi = 0; wi < a.W; ++wi) {
        uint64_t m = a.mask[(size_t)r * a.W + wi];
        while (m) {
          const int e = wi * 64 + __ffsll((unsigned long long)m) - 1;
          m &= m - 1;
          const float gate = a.g[(size_t)r * a.E + e];
          const typename DT::pair* yrow = yb + (size_t)sl * a.d + nt * 64 + c;
#pragma unroll
          for (int p = 0; p < 4; ++p) v[p] += gate * (float)yrow[p * 16];
          ++sl;
        }
      }
#pragma unroll
      for (int p = 0; p < 4; ++p) out[(size_t)r * a.d + (nt * 4 + p) * 16 + c] = DT::from_f32(v[p]);
    }
  }
}

// --------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_copy_mask(const float* __restrict__ z, const float* __restrict__ lam,
                                                   int T, int E, int W, uint64_t* __restrict__ mask) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= T * W) return;
  const int t = idx / W, wi = idx % W;
  uint64_t word = 0;
  for (int b = 0; b < 64; ++b) {
    const int e = wi * 64 + b;
    if (e < E && z[(size_t)t * E + e] > 0.f && lam[e] != 0.f) word |= 1ull << b;
  }
  mask[idx] = word;
}

template <class DT>
hipError_t prefill(const deco_moe_layer* L, const void* x, int T, void* out, hipStream_t s) {
  PreArgs a;
  a.x = x;
  a.out = out;
  a.T = T;
  a.Tcap = L->maxT < 16 ? 16 : L->maxT;
  a.d = L->d;
  a.E = L->E;
  a.F = L->F;
  a.Fs = L->Fs;
  a.W = L->W;
  a.nkb_d = L->nkb_d;
  a.nkb_F = L->nkb_F;
  a.nkb_Fs = L->nkb_Fs;
  a.pR = L->pR;
  a.pF = L->pF;
  a.pD = L->pD;
  a.pFs = L->pFs;
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
  a.mask = L->mask;
  a.tok_off = L->tok_off;
  a.ecnt = L->ecnt;
  a.list_tok = L->list_tok;
  a.list_slot = L->list_slot;
  a.sbuf = L->sbuf;
  a.ybuf = L->ybuf;
  const unsigned mtiles = (unsigned)((T + BM - 1) / BM);
  const unsigned ntiles = (unsigned)(L->pR / 4 + (L->pF + 3) / 4 + (L->pFs + 3) / 4);
  using deco_host::launch;
  hipError_t err = launch(deco_host::KS_PRE_ROUTER_SHARED, k_pre_router_shared<DT>, dim3(mtiles, ntiles),
                          dim3(256), s, a);
  if (err == hipSuccess) err = launch(deco_host::KS_PRE_DISPATCH, k_pre_dispatch, dim3(L->E), dim3(256), s, a);
  if (err == hipSuccess) {
    void (*kx)(PreArgs) = L->pF == 2 ? k_pre_expert<DT, 2>
                        : L->pF == 4 ? k_pre_expert<DT, 4>
                        : L->pF == 8 ? k_pre_expert<DT, 8> : k_pre_expert<DT, 16>;
    err = launch(deco_host::KS_PRE_EXPERT, kx, dim3(L->pre_grid), dim3(256), s, a);
  }
  if (err == hipSuccess)
    err = launch(deco_host::KS_PRE_SHARED_DOWN, k_pre_shared_down<DT>, dim3(mtiles, (unsigned)(L->pD / 4)),
                 dim3(256), s, a);
  if (err != hipSuccess) return err;
  return hipGetLastError();
}

}  // namespace

namespace deco_host {

hipError_t launch_prefill(const deco_moe_layer* L, const void* x, int T, void* out, hipStream_t s) {
  if (L->cfg.dtype == DECO_DT_BF16) return prefill<BF16>(L, x, T, out, s);
  return prefill<F32>(L, x, T, out, s);
}

hipError_t launch_copy_mask(const deco_moe_layer* L, int T, uint64_t* mask, hipStream_t s) {
  const int n = T * L->W;
  k_copy_mask<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(L->z, L->lam, T, L->E, L->W, mask);
  return hipGetLastError();
}

}  // namespace deco_host
