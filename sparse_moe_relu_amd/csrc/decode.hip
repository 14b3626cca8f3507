// decode.hip - weight-streaming forward path for small batches (T <= 16).
//
// At decode sizes the layer is a handful of matrix-vector products over the
// weights, so its cost is the HBM traffic of the weights it touches.  The
// point of ReLU routing with sparse experts is that inactive routed experts
// cost nothing: the DECO paper (Sec. 1 and the Sec. 4 acceleration paragraph
// with Table 4) attributes its speedup to skipping the memory traffic of
// inactive experts.  Two kernels:
//
//   k_dec_up    one workgroup per group of column slices of the shared
//               expert's up-projection, and per (routed expert, column
//               slice).  A routed workgroup computes its expert's router
//               logits for the batch (router: linear projection + bias, ReLU,
//               per-expert scale; DECO paper Sec. 2 "Router design") and
//               exits without reading any expert weight when no token
//               activated the expert.  Otherwise it streams its slice of
//               W_up[e] - Wbar through
//               v_mfma 16x16 products (tokens padded to 16 rows): the mean
//               term is folded into the matrix packed at load, x.(W_up[e] -
//               Wbar) = x.W_up[e] - x.Wbar.  It takes the row's RMS over all
//               F columns (the per-row sums of squares of the other slices of
//               the same expert are exchanged through device memory), applies
//               SiLU and the gate, and stores the activations as the
//               down-projection operand (NormSiLU: qidianchuan.cn write-up,
//               section 二: subtract the mean term, RMS inside the expert,
//               then SiLU).
//   k_dec_down  one workgroup per 8 output columns.  It lists the experts
//               the batch touched and multiplies their down-projection rows
//               for its 8 columns (and the shared expert's) with the
//               activations: the whole reduction over the shared expert and
//               every touched expert happens inside the workgroup, so each
//               output is written once, with no partial sums.
//
// Hand-offs inside k_dec_up (sums of squares, TopK logits) are
// 64-bit words written and read with agent-scope relaxed atomics: the high
// half is the call's epoch and the low half the value, so a reader needs no
// separate flag and no fence, and a word left from an earlier call is never
// taken for this call's.  The epoch is 1 + a call counter that the down
// kernel advances once per call, read by every up workgroup with a plain
// load (the kernel boundary orders the increment before the next call's
// reads).  Waiting workgroups only
// depend on the other slices of their own expert (consecutive workgroups) and,
// with TopK routing, on every routed workgroup; every wait is bounded (a
// timeout sets the layer's error flag).
#include <string.h>

#include <algorithm>
#include <map>
#include <mutex>

#include "deco_common.h"
#include "deco_internal.h"

using namespace deco;

namespace {

constexpr int DNW = 8;            // waves per workgroup (both kernels)
constexpr int DNT = DNW * 64;
constexpr int SPIN_LIMIT = 1 << 20;
constexpr int NSUB_MAX = 4;       // shared-expert slices per workgroup
typedef unsigned long long u64;

struct DecArgs {
  const void* x;
  void* out;
  int T, d, E, F, Fs, W;
  int nkb_d;                // k-blocks of d
  int S;                    // column slices per routed expert
  int n_sh, nsub;           // shared workgroups, shared slices per workgroup
  int n_shs;                // shared slices
  int pF, pFs;              // 16-column panels of F and Fs
  int top_k;                // TopK routing variant (0: ReLU routing)
  int no_rms;               // NormSiLU ablation: no RMS step
  float eps;
  const char* Wr_p;
  const char* Wup_p;        // NormSiLU input projection (a gated expert's gate projection)
  const char* Wlin_p;       // gated experts' up-projection
  const char* Wbar_p;
  const char* Wsu_p;
  const char* Wdn8_p;       // W_down[e] in column-pair fragments, down operand type
  const char* Wsd8_p;       // Ws_down in column-pair fragments, layer dtype
  size_t up_stride, dn8_stride;
  const float* b_r;
  const float* lam;
  float* z;                 // [T][E] logits
  float* g;                 // [T][E] gates
  unsigned char* act8;      // [16][E] routing decisions
  unsigned* rflag;          // [E] 1: no token routed to e, 2: some token was
  u64* hw;                  // hand-off words: [E * S][16] sums of squares |
                            // [E][16] logits (TopK) | [n_sh][16] shared sums of squares
  unsigned* ctr;            // call counter: the up kernel's epoch is 1 + its value
  void* arow;               // [E][16][Fp] routed activations, down operand type
  void* srow;               // [16][Fsp] shared activations, layer dtype
  int Fp, Fsp;              // F, Fs padded to whole column-pair fragments
  int kpe, kps;             // column-pair fragments per routed expert / of the shared expert
  unsigned* err;
};

__device__ __forceinline__ u64* hw_ss(const DecArgs& a) { return a.hw; }
__device__ __forceinline__ u64* hw_z(const DecArgs& a) { return hw_ss(a) + (size_t)a.E * a.S * 16; }
__device__ __forceinline__ u64* hw_sh(const DecArgs& a) { return hw_z(a) + (size_t)a.E * 16; }

__device__ __forceinline__ void put_word(u64* p, unsigned ep, float v) {
  __hip_atomic_store(p, ((u64)ep << 32) | __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u64 get_word(const u64* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool word_ok(u64 v, unsigned ep) { return (unsigned)(v >> 32) == ep; }
__device__ __forceinline__ float word_val(u64 v) { return __uint_as_float((unsigned)v); }

// Block-wide wait: every thread holds N words (already loaded from p[i];
// need marks those that matter); returns once all carry epoch ep, reloading the
// invalid ones.  Bounded: a timeout sets bit 0 of *err and the bit `which`
// naming the hand-off (4 sums of squares, 8 TopK logits, 16 shared sums of
// squares).
template <int N>
__device__ __forceinline__ void wait_words(u64 (&v)[N], const u64* const (&p)[N], const bool (&need)[N],
                                           unsigned ep, unsigned* err, unsigned which) {
  for (int it = 0;; ++it) {
    bool ok = true;
#pragma unroll
    for (int k = 0; k < N; ++k) ok = ok && (!need[k] || word_ok(v[k], ep));
    if (__syncthreads_and(ok)) return;
    if (it > SPIN_LIMIT) {
      if (threadIdx.x == 0) atomicOr(err, 1u | which);
      return;
    }
    __builtin_amdgcn_s_sleep(2);
#pragma unroll
    for (int k = 0; k < N; ++k)
      if (need[k] && !word_ok(v[k], ep)) v[k] = get_word(p[k]);
  }
}

// 16 bytes through a buffer resource; loads whose vector offset is past
// num_records return zeros without touching memory
__device__ __forceinline__ i32x4_t ld16_buf(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff) {
  return __builtin_bit_cast(i32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, unsigned bytes = 0x7FFFFFFFu) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
// one 32-bit word p[i] as a vector-memory load: a uniform load written as
// p[i] becomes a scalar load, and the scalar loads' wait (shared with the
// kernel-argument loads) would come before the router's first vector load
__device__ __forceinline__ unsigned ld_word(const void* p, int i) {
  return (unsigned)__builtin_amdgcn_raw_buffer_load_b32(buf_rsrc(p), 4 * i, 0, 0);
}

// acc[p] += x[16 rows][k-blocks kb_lo .. kb_hi) . W[..][panels p0 + p] for p < NP
// (panels at or past pmax read panel pmax - 1; their results are dropped by
// the caller).  Loads go in batches of 8 k-blocks x NP panels (up to 32
// fragments) issued together.  x rows past T read zeros (buffer range).
// 8 bf16 values -> 8 fp16 values (exact inside fp16's range); `bad` is
// raised for a value outside it
__device__ __forceinline__ i32x4_t bf16x8_to_f16x8(const i32x4_t& v, bool& bad) {
  i32x4_t r;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t u = (uint32_t)v[q];
    const float f0 = bf16_to_f32(u & 0xFFFFu), f1 = bf16_to_f32(u >> 16);
    bad |= !(fabsf(f0) <= 65504.f && fabsf(f1) <= 65504.f);
    r[q] = (int)(FP16::bits(f0) | (FP16::bits(f1) << 16));
  }
  return r;
}

// XH: the W fragments are fp16 (bf16 layers' folded NormSiLU input) and the
// x fragments are converted to fp16 for the product.  XPRE: x0 holds the
// first batch's x fragments (loaded by the router).  WPRE: w0 holds the first
// batch's W fragments (requested before the routing decision).  The first
// batch is straight-line code (no wait inherited from a loop's back edge).
template <class DT, int NP, bool XH = false, bool XPRE = false, bool WPRE = false>
__device__ __forceinline__ void up_stream(__amdgpu_buffer_rsrc_t rx, __amdgpu_buffer_rsrc_t rw, int p0, int pmax,
                                          int nkb, int kb_lo, int kb_hi, int d, f32x4_t (&acc)[NP],
                                          const i32x4_t* x0, bool* xbad = nullptr,
                                          const i32x4_t (*w0)[NP] = nullptr) {
  using elem = typename DT::elem;
  constexpr int U = 8;
  const int l = threadIdx.x & 63, c = l & 15, g = l >> 4;
  const unsigned xoff = (unsigned)(((size_t)c * d + (size_t)DT::EPL * g) * sizeof(elem));
  // past the wave's range: a valid block (k-block 0 for a wave with none),
  // whose products are skipped
  auto blk = [&](int kb) {
    kb = kb < kb_hi ? kb : kb_hi - 1;
    return kb < 0 ? 0 : kb;
  };
  auto products = [&](int kb0, const i32x4_t (&xf)[U], const i32x4_t (&wf)[U][NP]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (kb0 + u < kb_hi) {
        if constexpr (XH) {
          const i32x4_t xh = bf16x8_to_f16x8(xf[u], *xbad);
#pragma unroll
          for (int p = 0; p < NP; ++p) FP16::mma(acc[p], xh, wf[u][p]);
        } else {
#pragma unroll
          for (int p = 0; p < NP; ++p) DT::mma(acc[p], xf[u], wf[u][p]);
        }
      }
  };
  {
    i32x4_t xf[U], wf[U][NP];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kb = blk(kb_lo + u);
      if constexpr (XPRE) xf[u] = x0[u];
      else xf[u] = ld16_buf(rx, xoff, (unsigned)(kb * DT::KB * sizeof(elem)));
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int pp = p0 + p < pmax ? p0 + p : pmax - 1;
        if constexpr (WPRE) wf[u][p] = w0[u][p];
        else wf[u][p] = ld16_buf(rw, 16u * l, (unsigned)frag_off(pp, kb, nkb));
      }
    }
    __builtin_amdgcn_sched_barrier(0);   // the whole batch in flight before its first product
    products(kb_lo, xf, wf);
  }
  for (int kb0 = kb_lo + U; kb0 < kb_hi; kb0 += U) {
    i32x4_t xf[U], wf[U][NP];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kb = blk(kb0 + u);
      xf[u] = ld16_buf(rx, xoff, (unsigned)(kb * DT::KB * sizeof(elem)));
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int pp = p0 + p < pmax ? p0 + p : pmax - 1;
        wf[u][p] = ld16_buf(rw, 16u * l, (unsigned)frag_off(pp, kb, nkb));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    products(kb0, xf, wf);
  }
}

// sum the waves' accumulators into dst[row][col] (16 rows x 16 NP columns)
template <int NP, int LD>
__device__ __forceinline__ void reduce_waves(f32x4_t (&s_red)[DNW][NP][64], const f32x4_t (&acc)[NP],
                                             float (*dst)[LD]) {
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
#pragma unroll
  for (int p = 0; p < NP; ++p) s_red[w][p][l] = acc[p];
  __syncthreads();
  for (int o = tid; o < 256 * NP; o += DNT) {
    const int p = o >> 8, ll = (o >> 2) & 63, i = o & 3;
    float v = 0.f;
#pragma unroll
    for (int ww = 0; ww < DNW; ++ww) v += s_red[ww][p][ll][i];
    dst[4 * (ll >> 4) + i][16 * p + (ll & 15)] = v;
  }
  __syncthreads();
}

// VAR bits of the up kernel (separate instantiations, so the default one
// carries none of the variants' logic)
constexpr int DV_GATED = 1, DV_NO_MEAN = 2, DV_SHARED_RMS = 4;

// SPEC: the routed slice's first batch of W_up requested with the router's
// loads, before the routing decision (for batches that touch most experts)
template <class DT, int NP, int VAR, bool SPEC = false>
__global__ void __launch_bounds__(DNT) k_dec_up(DecArgs a) {
  constexpr bool GT = (VAR & DV_GATED) != 0, NM = (VAR & DV_NO_MEAN) != 0, SR = (VAR & DV_SHARED_RMS) != 0;
  using elem = typename DT::elem;
  // bf16 layers with the mean term: the NormSiLU input matrix is the folded
  // W - Wbar in fp16, multiplied by x converted to fp16
  constexpr bool XH = sizeof(elem) == 2 && !NM;
  using DN = typename DT::Down;
  constexpr int U = 8;             // k-blocks per load batch
  constexpr int NCOL = 16 * NP;    // columns of a slice
  constexpr int CPT = NCOL / 32;   // columns per thread in the row phase (32 threads per row)
  __shared__ f32x4_t s_red[DNW][NP][64];
  __shared__ float s_h[SR ? NSUB_MAX : 1][16][NCOL + 1];
  __shared__ float s_u[GT ? 16 : 1][GT ? NCOL + 1 : 1];
  __shared__ float s_zr[DNW][16];
  __shared__ float s_gate[16], s_ssx[16][33];
  __shared__ int s_act[16];
  __shared__ float s_zall[16][257];   // TopK: every expert's logits
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, c = l & 15, g = l >> 4;
  const int b = blockIdx.x;
  // this call's epoch (ep below): 1 + the number of earlier calls.  The down
  // kernel of each call advances the counter once; the kernel boundary
  // between that launch and this one makes the new value visible, so a plain
  // load issued behind the first loads reads it (no atomic round trip in
  // front of them)
  const int kind = b < a.n_sh ? 1 : 2;   // shared, routed
  const int rb = b - a.n_sh;
  const int e = kind == 2 ? rb / a.S : 0;
  const int slice = kind == 1 ? b : rb % a.S;
  const int nkb = a.nkb_d;
  const int kb_lo = (w * nkb) / DNW, kb_hi = ((w + 1) * nkb) / DNW;
  const __amdgpu_buffer_rsrc_t rx = buf_rsrc(a.x, (unsigned)((size_t)a.T * a.d * sizeof(elem)));
  // row phase: 32 threads per token row, CPT consecutive columns each
  const int row = tid >> 5, cq = tid & 31;
  const int col0 = CPT * cq;

  f32x4_t acc[NP], accu[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) acc[p] = accu[p] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  i32x4_t x0[U];   // the router's first batch of x fragments

  if (kind == 1) {
    // ---- shared expert: slices slice * nsub .. (+ nsub), SiLU(x . Ws_up) as
    // the down-projection operand (RMS-only variant: the row's RMS spans all
    // slices, exchanged between the shared workgroups)
    float ss = 0.f;
    for (int j = 0; j < a.nsub; ++j) {
      const int q = slice * a.nsub + j;
      if (q >= a.n_shs) break;
#pragma unroll
      for (int p = 0; p < NP; ++p) acc[p] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      up_stream<DT, NP>(rx, buf_rsrc(a.Wsu_p), q * NP, a.pFs, nkb, kb_lo, kb_hi, a.d, acc, x0);
      reduce_waves<NP, NCOL + 1>(s_red, acc, s_h[SR ? j : 0]);
      const int gcol0 = q * NCOL + col0;
      const bool col_ok = gcol0 < a.Fs;   // a partial last slice: CPT divides 32, so all or none
      if constexpr (SR) {
#pragma unroll
        for (int k = 0; k < CPT; ++k) ss += col_ok ? s_h[j][row][col0 + k] * s_h[j][row][col0 + k] : 0.f;
      } else if (row < a.T && col_ok) {
        elem* srow = (elem*)a.srow + (size_t)row * a.Fsp + gcol0;
#pragma unroll
        for (int k = 0; k < CPT; ++k) srow[k] = DT::from_f32(silu_f(s_h[0][row][col0 + k]));
      }
    }
    if constexpr (SR) {
#pragma unroll
      for (int o = 16; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
      const unsigned ep = ld_word(a.ctr, 0) + 1u;
      if (cq == 0) put_word(hw_sh(a) + (size_t)slice * 16 + row, ep, ss);
      // every shared workgroup's sums (32 at a time, one per thread of the
      // row), then the row's 1 / RMS
      float tot = 0.f;
      for (int q0 = 0; q0 < a.n_sh; q0 += 32) {
        u64 v[1];
        const bool need[1] = {q0 + cq < a.n_sh};
        const u64* const p[1] = {hw_sh(a) + (size_t)(need[0] ? q0 + cq : 0) * 16 + row};
        v[0] = need[0] ? get_word(p[0]) : 0ull;
        wait_words<1>(v, p, need, ep, a.err, 16u);
        s_ssx[row][cq] = need[0] ? word_val(v[0]) : 0.f;
        __syncthreads();
        for (int q = 0; q < 32 && q0 + q < a.n_sh; ++q) tot += s_ssx[row][q];   // workgroup order
        __syncthreads();
      }
      const float rinv = 1.0f / sqrtf(tot / (float)a.Fs + a.eps);
      for (int j = 0; j < a.nsub; ++j) {
        const int q = slice * a.nsub + j;
        const int gcol0 = q * NCOL + col0;
        if (q < a.n_shs && row < a.T && gcol0 < a.Fs) {
          elem* srow = (elem*)a.srow + (size_t)row * a.Fsp + gcol0;
#pragma unroll
          for (int k = 0; k < CPT; ++k) srow[k] = DT::from_f32(silu_f(s_h[j][row][col0 + k] * rinv));
        }
      }
    }
    return;
  }

  // ---- routed: router logits of expert e for the 16 (padded) token rows;
  // each lane sums x[c][k] W_r[k][e] over its fragment entries, waves over d
  float lam_e, b_e;
  unsigned ep;
  // the first batch of the slice's NormSiLU-input stream, requested ahead of
  // time: before the routing decision (SPEC), or, for gated experts, before
  // the linear projection's stream, so that both first batches share a trip
  // (32-column slices: 64 more registers; the 64-column ones would spill)
  constexpr bool GPRE = GT && NP <= 2;
  constexpr bool WPRE = SPEC || GPRE;
  i32x4_t wsp[WPRE ? U : 1][NP];
  auto preload_wup = [&]() {
    const __amdgpu_buffer_rsrc_t rwu = buf_rsrc(a.Wup_p + (size_t)e * a.up_stride);
    const int p0s = slice * NP;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int kb = kb_lo + u < kb_hi ? kb_lo + u : kb_hi - 1;
      kb = kb < 0 ? 0 : kb;
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int pp = p0s + p < a.pF ? p0s + p : a.pF - 1;
        wsp[WPRE ? u : 0][p] = ld16_buf(rwu, 16u * l, (unsigned)frag_off(pp, kb, nkb));
      }
    }
  };
  {
    const char* wr = a.Wr_p + frag_off(e >> 4, 0, nkb) + (size_t)((e & 15) + 16 * g) * 16;
    const unsigned xoff = (unsigned)(((size_t)c * a.d + (size_t)DT::EPL * g) * sizeof(elem));
    float zp = 0.f;
    i32x4_t xv[U], wv[U];
    auto loads = [&](int kb0) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        // past the wave's range: a valid block (k-block 0 for a wave with
        // none), whose products are skipped
        int kb = kb0 + u < kb_hi ? kb0 + u : kb_hi - 1;
        kb = kb < 0 ? 0 : kb;
        xv[u] = ld16_buf(rx, xoff, (unsigned)(kb * DT::KB * sizeof(elem)));
        wv[u] = ld16(wr + (size_t)kb * FRAG_BYTES);
      }
    };
    auto products = [&](int kb0) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (kb0 + u < kb_hi) {
#pragma unroll
          for (int j = 0; j < DT::EPL; ++j) zp += DT::lane_elem(xv[u], j) * DT::lane_elem(wv[u], j);
        }
      }
    };
    // the first batch in straight-line code: in a loop, a register reused
    // across the back edge puts a wait for older loads in front of it
    loads(kb_lo);
    if constexpr (SPEC) preload_wup();
    // the call's epoch and the expert's router scalars, behind the batch
    ep = ld_word(a.ctr, 0) + 1u;
    lam_e = __uint_as_float(ld_word(a.lam, e));
    b_e = __uint_as_float(ld_word(a.b_r, e));
    // every load of the batch before the first product (the scheduler
    // otherwise sinks some below the first FMAs, a second round trip)
    __builtin_amdgcn_sched_barrier(0);
    products(kb_lo);
#pragma unroll
    for (int u = 0; u < U; ++u) x0[u] = xv[u];
    for (int kb0 = kb_lo + U; kb0 < kb_hi; kb0 += U) {
      loads(kb0);
      __builtin_amdgcn_sched_barrier(0);
      products(kb0);
    }
    zp += __shfl_xor(zp, 16);
    zp += __shfl_xor(zp, 32);
    if (g == 0) s_zr[w][c] = zp;
  }
  __syncthreads();
  if (tid < 16) {
    float zz = 0.f;
#pragma unroll
    for (int ww = 0; ww < DNW; ++ww) zz += s_zr[ww][tid];
    zz += b_e;
    s_zr[0][tid] = zz;   // read below by row tid only
    const bool act = tid < a.T && zz > 0.f && lam_e != 0.f;
    s_act[tid] = act;
    s_gate[tid] = act ? lam_e * zz : 0.f;
  }
  if (a.top_k > 0) {
    // TopK: every expert's logits are needed before any expert can be
    // skipped.  The expert's first slice publishes its logits; all routed
    // workgroups read every expert's, and one wave per token selects.
    __syncthreads();
    if (slice == 0 && tid < 16) put_word(hw_z(a) + (size_t)e * 16 + tid, ep, s_zr[0][tid]);
    constexpr int ZPT = 16 * 256 / DNT;   // words per thread (T x E <= 16 x 256)
    u64 v[ZPT];
    bool need[ZPT];
    const u64* p[ZPT];
#pragma unroll
    for (int k = 0; k < ZPT; ++k) {
      const int i = tid + DNT * k;
      need[k] = i < a.T * a.E;
      const int t = need[k] ? i / a.E : 0, ee = need[k] ? i % a.E : 0;
      p[k] = hw_z(a) + (size_t)ee * 16 + t;
      v[k] = need[k] ? get_word(p[k]) : 0ull;
    }
    wait_words<ZPT>(v, p, need, ep, a.err, 8u);
#pragma unroll
    for (int k = 0; k < ZPT; ++k) {
      const int i = tid + DNT * k;
      if (need[k]) s_zall[i / a.E][i % a.E] = word_val(v[k]);
    }
    __syncthreads();
    for (int t = w; t < a.T; t += DNW) {
      float zv[4];
      bool sel[4];
      float gate[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ee = 64 * j + l;
        zv[j] = ee < a.E ? s_zall[t][ee] : -__builtin_inff();
      }
      topk_wave<4>(zv, a.top_k, sel, gate);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (64 * j + l == e) {
          s_act[t] = sel[j];
          s_gate[t] = gate[j];
        }
    }
    // every wave's decisions are in before they are read (the predicate
    // below is evaluated before its barrier)
    __syncthreads();
  }
  const bool any = __syncthreads_or(tid < 16 && s_act[tid] != 0) != 0;
  if (slice == 0) {
    if (tid < a.T) {
      a.z[(size_t)tid * a.E + e] = s_zr[0][tid];
      a.g[(size_t)tid * a.E + e] = s_gate[tid];
      a.act8[(size_t)tid * a.E + e] = (unsigned char)(s_act[tid] != 0);
    }
    if (tid == 0) a.rflag[e] = any ? 2u : 1u;
  }
  if (!any) return;   // no token activated expert e: none of its weights are read

  const int gcol0 = slice * NCOL + col0;   // in F
  // the slice's up-projection (gated: the linear projection first, then the
  // NormSiLU input)
  const int p0 = slice * NP;
  if constexpr (GT) {
    if constexpr (GPRE && !SPEC) preload_wup();
    up_stream<DT, NP, false, true>(rx, buf_rsrc(a.Wlin_p + (size_t)e * a.up_stride), p0, a.pF, nkb, kb_lo,
                                   kb_hi, a.d, accu, x0);
    reduce_waves<NP, GT ? NCOL + 1 : 1>(s_red, accu, s_u);
  }
  bool xbad = false;
  up_stream<DT, NP, XH, true, WPRE>(rx, buf_rsrc(a.Wup_p + (size_t)e * a.up_stride), p0, a.pF, nkb, kb_lo,
                                    kb_hi, a.d, acc, x0, &xbad, wsp);
  if (xbad) atomicOr(a.err, 32u);   // an x value outside the fp16 range
  reduce_waves<NP, NCOL + 1>(s_red, acc, s_h[0]);

  // h~ = x . (W_up[e] - Wbar) (the mean term is folded into the packed
  // matrix), then the row's sum of squares over this slice
  float hv[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) hv[k] = s_h[0][row][col0 + k];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < CPT; ++k) ss += hv[k] * hv[k];
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
  if (a.S > 1) {
    // the other slices' sums of squares of the same rows, added in slice order
    if (cq == 0) put_word(hw_ss(a) + ((size_t)e * a.S + slice) * 16 + row, ep, ss);
    u64 v[1];
    const bool need[1] = {cq < a.S};
    const u64* const p[1] = {hw_ss(a) + ((size_t)e * a.S + (cq < a.S ? cq : 0)) * 16 + row};
    v[0] = need[0] ? get_word(p[0]) : 0ull;
    wait_words<1>(v, p, need, ep, a.err, 4u);
    if (cq < a.S) s_ssx[row][cq] = word_val(v[0]);
    __syncthreads();
    ss = 0.f;
    for (int q = 0; q < a.S; ++q) ss += s_ssx[row][q];
  }
  const float rinv = a.no_rms ? 1.0f : 1.0f / sqrtf(ss / (float)a.F + a.eps);
  const float gt = s_gate[row];
  if (row < a.T) {
    float av[CPT];
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      av[k] = gt != 0.f ? silu_f(hv[k] * rinv) * gt : 0.f;
      if constexpr (GT) av[k] *= s_u[row][col0 + k];
    }
    using DE = typename DN::elem;
    DE* ar = (DE*)a.arow + ((size_t)e * 16 + row) * a.Fp + gcol0;
    if constexpr (sizeof(DE) == 2) {
      // fp16 operand of the down-projection: a value past its range would be
      // stored as inf; report it (bit 5) instead of returning a silent inf
      bool bad = false;
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        bad |= !(fabsf(av[k]) <= 65504.f);
        ar[k] = (DE)DN::bits(av[k]);
      }
      if (bad) atomicOr(a.err, 32u);
    } else {
#pragma unroll
      for (int k = 0; k < CPT; ++k) ar[k] = av[k];
    }
  }
}

// --------------------------------------------------------------------------
// Down-projection, one workgroup per CG groups of 8 output columns.  Its
// reduction runs over the shared expert's rows and the rows of every expert
// the batch touched, in "column-pair" fragments: a 1 KiB fragment holds two
// k-blocks of 8 columns (columns 0-7 of the MFMA tile take the first k-block,
// columns 8-15 the second), and the token operand holds the same two k-blocks
// in its rows 0-7 and 8-15, so one 16x16 product covers both k-blocks and the
// result's diagonal quadrants are the two halves of the sum.  TH token halves
// of 8 rows (T <= 8: one; T <= 16: two); the CG column groups share each
// token fragment.  Fragment ("slot") order: the shared expert's, then each
// touched expert's in ascending expert order; wave w takes slots w, w + 8, ...
// Every batch of loads is issued without a branch: a slot past the end gets
// a vector offset past its buffer's range, which loads zeros without a memory
// access, so its product adds nothing.
template <class DT, int TH, int CG>
__global__ void __launch_bounds__(DNT) k_dec_down(DecArgs a) {
  using elem = typename DT::elem;
  using DN = typename DT::Down;
  using DE = typename DN::elem;
  constexpr int SB = 4;                                   // shared slots per wave, issued first
  constexpr int SPW = (TH == 2 && CG == 2) ? 8 : 12;      // expert slots per wave per batch
  constexpr unsigned OOR = 0x40000000u;                   // past every buffer range used here
  __shared__ f32x4_t s_red[DNW][CG][TH][64];
  __shared__ int s_list[DNW][256];
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
  const int r16 = l & 15, g = l >> 4, half = r16 >> 3;
  const int cg0 = blockIdx.x * CG;   // first of the workgroup's column groups
  const int kps = a.kps, kpe = a.kpe;
  // the call counter the next call's up kernel takes its epoch from (this
  // call's up kernel has read it; nothing waits for the result).  Every
  // decode call that launches the up kernel launches this one after it on
  // the same stream; a call whose second launch failed leaves the counter
  // behind, and its error is returned to the caller.
  if (blockIdx.x == 0 && tid == 0) __hip_atomic_fetch_add(a.ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // routing flags first, so the shared slots' loads queue behind them
  unsigned rf[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = 64 * j + l;
    rf[j] = a.rflag[e < a.E ? e : a.E - 1];
  }
  // the lane's token row (r16 & 7) and k offset; rows 8-15 of the tile take
  // the second k-block of the pair (in the vector offset, so the scalar
  // offset stays uniform)
  const unsigned tok_s = (unsigned)(((r16 & 7) * (size_t)a.Fsp + (size_t)half * DT::KB + (size_t)DT::EPL * g) *
                                    sizeof(elem));
  const unsigned tok_r = (unsigned)(((r16 & 7) * (size_t)a.Fp + (size_t)half * DN::KB + (size_t)DN::EPL * g) *
                                    sizeof(DE));
  const unsigned th_s = (unsigned)(8 * (size_t)a.Fsp * sizeof(elem));
  const unsigned th_r = (unsigned)(8 * (size_t)a.Fp * sizeof(DE));
  const __amdgpu_buffer_rsrc_t rs = buf_rsrc(a.srow, (unsigned)((size_t)a.T * a.Fsp * sizeof(elem)));
  const __amdgpu_buffer_rsrc_t rws =
      buf_rsrc(a.Wsd8_p + (size_t)cg0 * kps * FRAG_BYTES, (unsigned)((size_t)CG * kps * FRAG_BYTES));
  auto load_sh = [&](int gi, i32x4_t (&wv)[CG], i32x4_t (&av)[TH]) {
    const bool ok = gi < kps;
    const int gc = ok ? gi : 0;
    const unsigned vo = ok ? 0u : OOR;
#pragma unroll
    for (int c = 0; c < CG; ++c) wv[c] = ld16_buf(rws, 16u * l + vo, (unsigned)(((size_t)c * kps + gc) * FRAG_BYTES));
#pragma unroll
    for (int th = 0; th < TH; ++th)
      av[th] = ld16_buf(rs, tok_s + th * th_s + vo, (unsigned)(2 * gc * DT::KB * sizeof(elem)));
  };
  i32x4_t sw[SB][CG], sa[SB][TH];
#pragma unroll
  for (int k = 0; k < SB; ++k) load_sh(w + DNW * k, sw[k], sa[k]);

  // the touched experts in ascending order, as a list in this wave's LDS row
  unsigned long long mk[4];
  int n_act = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // (bitwise, so every flag load stays unconditional and ahead of the
    // shared loads: a load sunk into a branch would be waited for with them)
    mk[j] = __ballot((j < a.W) & (64 * j + l < a.E) & (rf[j] == 2u));
    if ((mk[j] >> l) & 1ull) s_list[w][n_act + __popcll(mk[j] & ((1ull << l) - 1ull))] = 64 * j + l;
    n_act += __popcll(mk[j]);
  }
  __builtin_amdgcn_wave_barrier();
  const int n_exp = n_act * kpe;
  const int ksh = __builtin_ctz(kpe);   // kpe is a power of two (F is)
  // a batch of expert slots q = base + w + 8 k: the experts from the list
  // first (one LDS round trip for the batch), then the loads.  Past the end
  // the list entry is stale or unset; it is clamped to a valid expert and the
  // slot reads zeros.
  auto load_ex = [&](int base, auto& wv, auto& av) {
    constexpr int NS = sizeof(wv) / sizeof(wv[0]);
    int ev[NS];
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      const int q = base + w + DNW * k;
      ev[k] = s_list[w][(q < n_exp ? q : 0) >> ksh];
    }
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      const int q = base + w + DNW * k;
      const bool ok = q < n_exp;
      const int kp = (ok ? q : 0) & (kpe - 1);
      int e = __builtin_amdgcn_readfirstlane(ev[k]);
      e = e < 0 ? 0 : (e >= a.E ? a.E - 1 : e);
      const unsigned vo = ok ? 0u : OOR;
      const __amdgpu_buffer_rsrc_t rw = buf_rsrc(a.Wdn8_p + (size_t)e * a.dn8_stride + (size_t)cg0 * kpe * FRAG_BYTES,
                                                 (unsigned)((size_t)CG * kpe * FRAG_BYTES));
#pragma unroll
      for (int c = 0; c < CG; ++c)
        wv[k][c] = ld16_buf(rw, 16u * l + vo, (unsigned)(((size_t)c * kpe + kp) * FRAG_BYTES));
      const __amdgpu_buffer_rsrc_t ra =
          buf_rsrc((const DE*)a.arow + (size_t)e * 16 * a.Fp, (unsigned)((size_t)a.T * a.Fp * sizeof(DE)));
#pragma unroll
      for (int th = 0; th < TH; ++th)
        av[k][th] = ld16_buf(ra, tok_r + th * th_r + vo, (unsigned)(2 * kp * DN::KB * sizeof(DE)));
    }
  };

  f32x4_t acc[CG][TH];
#pragma unroll
  for (int c = 0; c < CG; ++c)
#pragma unroll
    for (int th = 0; th < TH; ++th) acc[c][th] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  {
    // first expert batch, then the shared products (their loads are older)
    i32x4_t wv[SPW][CG], av[SPW][TH];
    load_ex(0, wv, av);
    __builtin_amdgcn_sched_barrier(0);   // every load of the batch before the first product
#pragma unroll
    for (int k = 0; k < SB; ++k)
#pragma unroll
      for (int c = 0; c < CG; ++c)
#pragma unroll
        for (int th = 0; th < TH; ++th) DT::mma(acc[c][th], sa[k][th], sw[k][c]);
#pragma unroll
    for (int k = 0; k < SPW; ++k)
#pragma unroll
      for (int c = 0; c < CG; ++c)
#pragma unroll
        for (int th = 0; th < TH; ++th) DN::mma(acc[c][th], av[k][th], wv[k][c]);
  }
  for (int base = DNW * SPW; base < n_exp; base += DNW * SPW) {
    i32x4_t wv[SPW][CG], av[SPW][TH];
    load_ex(base, wv, av);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < SPW; ++k)
#pragma unroll
      for (int c = 0; c < CG; ++c)
#pragma unroll
        for (int th = 0; th < TH; ++th) DN::mma(acc[c][th], av[k][th], wv[k][c]);
  }
  for (int s0 = DNW * SB; s0 < kps; s0 += DNW * SB) {   // shared slots past the first batch
    i32x4_t wv[SB][CG], av[SB][TH];
#pragma unroll
    for (int k = 0; k < SB; ++k) load_sh(s0 + w + DNW * k, wv[k], av[k]);
#pragma unroll
    for (int k = 0; k < SB; ++k)
#pragma unroll
      for (int c = 0; c < CG; ++c)
#pragma unroll
        for (int th = 0; th < TH; ++th) DT::mma(acc[c][th], av[k][th], wv[k][c]);
  }
  // sum the waves' products, then the two diagonal quadrants: lane
  // (col cc, group g < 2) holds C[4 g + i][cc] (first k-block of each
  // pair), lane (cc + 8, g + 2) holds C[8 + 4 g + i][cc + 8] (second)
#pragma unroll
  for (int c = 0; c < CG; ++c)
#pragma unroll
    for (int th = 0; th < TH; ++th) s_red[w][c][th][l] = acc[c][th];
  __syncthreads();
  for (int q = tid; q < CG * TH * 64; q += DNT) {
    const int c = q / (TH * 64), th = (q >> 6) % TH, rem = q & 63;
    const int g2 = rem >> 5, cc = (rem >> 2) & 7, i = rem & 3;
    const int t = 8 * th + 4 * g2 + i;
    float v = 0.f;
#pragma unroll
    for (int ww = 0; ww < DNW; ++ww) {
      const f32x4_t p1 = s_red[ww][c][th][cc + 16 * g2];
      const f32x4_t p2 = s_red[ww][c][th][cc + 8 + 16 * (g2 + 2)];
      v += p1[i] + p2[i];
    }
    if (t < a.T) ((elem*)a.out)[(size_t)t * a.d + 8 * (cg0 + c) + cc] = DT::from_f32(v);
  }
}

template <class DT, int NP>
void (*up_kernel_np(int var))(DecArgs) {
  switch (var) {
    case 0: return k_dec_up<DT, NP, 0>;
    case 1: return k_dec_up<DT, NP, 1>;
    case 2: return k_dec_up<DT, NP, 2>;
    case 3: return k_dec_up<DT, NP, 3>;
    case 4: return k_dec_up<DT, NP, 4>;
    case 5: return k_dec_up<DT, NP, 5>;
    case 6: return k_dec_up<DT, NP, 6>;
    default: return k_dec_up<DT, NP, 7>;
  }
}
template <class DT>
void (*up_kernel(int np, int var, bool spec = false))(DecArgs) {
  if (spec && var == 0) return np == 4 ? k_dec_up<DT, 4, 0, true> : k_dec_up<DT, 2, 0, true>;
  return np == 4 ? up_kernel_np<DT, 4>(var) : up_kernel_np<DT, 2>(var);
}

// From this batch size on, a routed slice requests its first W_up batch
// before its expert's routing decision: the batch then touches nearly every
// expert (about 1 - (1 - p)^T of them at activation ratio p), so the few
// inactive experts' requests cost less than the router's load trip in front
// of the stream (on the d = 2048 layer: 0.6 us faster per call at T = 16,
// even at T = 8, where a fifth of the experts are idle).  Not with TopK routing (its decision waits on every expert's
// logits), and only when each wave's share of the router is one batch of
// k-blocks (a second router batch would wait for the speculative requests).
#ifndef DECO_DEC_SPEC_T
#define DECO_DEC_SPEC_T 16
#endif
bool dec_spec(const deco_moe_layer* L, int T) {
  return T >= DECO_DEC_SPEC_T && L->cfg.top_k == 0 && (L->nkb_d + DNW - 1) / DNW <= 8;
}

int dec_variant(const deco_moe_layer* L) {
  return (L->gated ? DV_GATED : 0) | ((L->cfg.normsilu & DECO_NORMSILU_NO_MEAN) ? DV_NO_MEAN : 0) |
         (L->cfg.shared_rms ? DV_SHARED_RMS : 0);
}

DecArgs dec_args(const deco_moe_layer* L, const void* x, int T, void* out) {
  DecArgs a;
  memset(&a, 0, sizeof(a));
  a.x = x;
  a.out = out;
  a.T = T;
  a.d = L->d;
  a.E = L->E;
  a.F = L->F;
  a.Fs = L->Fs;
  a.W = L->W;
  a.nkb_d = L->nkb_d;
  a.S = L->dec_S;
  a.n_sh = L->dec_n_sh;
  a.nsub = L->dec_nsub;
  a.n_shs = L->dec_n_shs;
  a.pF = L->pF;
  a.pFs = L->pFs;
  a.top_k = L->cfg.top_k;
  a.no_rms = (L->cfg.normsilu & DECO_NORMSILU_NO_RMS) != 0;
  a.eps = L->cfg.rms_eps;
  a.Wr_p = L->Wr_p;
  // the mean term folded into the experts' matrices (x . (W_up[e] - Wbar)),
  // or plain W_up with the mean-term ablation
  a.Wup_p = L->Wupm_p ? L->Wupm_p : L->Wup_p;
  a.Wlin_p = L->Wlin_p;
  a.Wbar_p = L->Wbar_p;
  a.Wsu_p = L->Wsu_p;
  a.Wdn8_p = L->Wdn8_p;
  a.Wsd8_p = L->Wsd8_p;
  a.up_stride = L->up_stride;
  a.dn8_stride = L->dn8_stride;
  a.b_r = L->b_r;
  a.lam = L->lam;
  a.z = L->z;
  a.g = L->g;
  a.act8 = L->act8;
  a.rflag = L->rflag;
  a.hw = (u64*)L->hwords;
  a.ctr = L->dec_ctr;
  a.arow = L->arow;
  a.srow = L->srow;
  a.Fp = L->dec_Fp;
  a.Fsp = L->dec_Fsp;
  a.kpe = L->dec_kpe;
  a.kps = L->dec_kps;
  a.err = L->dec_err;
  return a;
}

template <class DT>
void (*down_kernel(const deco_moe_layer* L, int T, int* grid))(DecArgs) {
  // two column groups per workgroup once one per group would exceed the CU count
  const int cgw = L->d / 8 > L->n_cu ? 2 : 1;
  *grid = L->d / (8 * cgw);
  return T <= 8 ? (cgw == 2 ? k_dec_down<DT, 1, 2> : k_dec_down<DT, 1, 1>)
                : (cgw == 2 ? k_dec_down<DT, 2, 2> : k_dec_down<DT, 2, 1>);
}

template <class DT>
hipError_t decode(const deco_moe_layer* L, const void* x, int T, void* out, hipStream_t s) {
  const DecArgs a = dec_args(L, x, T, out);
  hipError_t err = deco_host::launch(deco_host::KS_DEC_UP, up_kernel<DT>(L->dec_np, dec_variant(L), dec_spec(L, T)),
                                     dim3((unsigned)L->dec_grid_up), dim3(DNT), s, a);
  if (err != hipSuccess) return err;
  int grid = 0;
  void (*down)(DecArgs) = down_kernel<DT>(L, T, &grid);
  err = deco_host::launch(deco_host::KS_DEC_DOWN, down, dim3((unsigned)grid), dim3(DNT), s, a);
  if (err != hipSuccess) return err;
  return hipGetLastError();
}

// --------------------------------------------------------------------------
// Allocation-free decode.  The same two kernels, with everything they hand to
// each other (hand-off words, epoch counters, routing flags, decisions,
// logits and gates, activation rows) in one file-scope device array instead
// of the layer's workspace; a fill kernel clears it at the start of every
// call, so each call runs with epoch 1.  Only the error flags go to the layer.
// Every call on a device shares that device's array: calls that overlap on
// one device race.
constexpr size_t SCRATCH_BYTES = (size_t)4 << 20;
static __device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];

// device-scope stores of zero (the hand-off words are read with device-scope
// atomics by workgroups on every XCD)
__global__ void __launch_bounds__(256) k_scratch_clear(unsigned* __restrict__ p, unsigned n) {
  for (unsigned i = blockIdx.x * 256u + threadIdx.x; i < n; i += gridDim.x * 256u)
    __hip_atomic_store(p + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct ScratchPlan {
  size_t o_hw, o_ct, o_rf, o_a8, o_z, o_g, o_ar, o_sr, bytes;
};
size_t al256(size_t v) { return (v + 255) / 256 * 256; }
ScratchPlan scratch_plan(const deco_moe_layer* L) {
  ScratchPlan p;
  size_t o = 0;
  p.o_hw = o;
  o += al256(sizeof(u64) * (size_t)L->n_hwords);
  p.o_ct = o;
  o += al256(sizeof(unsigned));
  p.o_rf = o;
  o += al256(sizeof(unsigned) * (size_t)L->E);
  p.o_a8 = o;
  o += al256((size_t)16 * L->E);
  p.o_z = o;
  o += al256(sizeof(float) * 16 * L->E);
  p.o_g = o;
  o += al256(sizeof(float) * 16 * L->E);
  p.o_ar = o;
  o += al256((size_t)(L->esz == 2 ? 2 : 4) * L->E * 16 * L->dec_Fp);
  p.o_sr = o;
  o += al256((size_t)L->esz * 16 * L->dec_Fsp);
  p.bytes = o;
  return p;
}

// the address of `scratch` on each device, taken once per device with that
// device current (each device holds its own copy of the array)
std::mutex g_scr_mu;
std::map<int, char*> g_scr_ptr;
hipError_t scratch_base(char** out) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  std::lock_guard<std::mutex> lk(g_scr_mu);
  auto it = g_scr_ptr.find(dev);
  if (it != g_scr_ptr.end()) {
    *out = it->second;
    return hipSuccess;
  }
  void* p = nullptr;
  err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (err != hipSuccess) return err;
  g_scr_ptr[dev] = (char*)p;
  *out = (char*)p;
  return hipSuccess;
}

template <class DT>
hipError_t decode_scratch(const deco_moe_layer* L, const void* x, int T, void* out, char* base,
                          const ScratchPlan& sp, hipStream_t s) {
  DecArgs a = dec_args(L, x, T, out);
  a.hw = (u64*)(base + sp.o_hw);
  a.ctr = (unsigned*)(base + sp.o_ct);
  a.rflag = (unsigned*)(base + sp.o_rf);
  a.act8 = (unsigned char*)(base + sp.o_a8);
  a.z = (float*)(base + sp.o_z);
  a.g = (float*)(base + sp.o_g);
  a.arow = base + sp.o_ar;
  a.srow = base + sp.o_sr;
  const unsigned nw = (unsigned)(sp.bytes / 4);
  hipLaunchKernelGGL(k_scratch_clear, dim3(std::min(1024u, (nw + 255) / 256)), dim3(256), 0, s, (unsigned*)base, nw);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(up_kernel<DT>(L->dec_np, dec_variant(L), dec_spec(L, T)), dim3((unsigned)L->dec_grid_up),
                     dim3(DNT), 0, s, a);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  int grid = 0;
  void (*down)(DecArgs) = down_kernel<DT>(L, T, &grid);
  hipLaunchKernelGGL(down, dim3((unsigned)grid), dim3(DNT), 0, s, a);
  return hipGetLastError();
}

// the routing masks of the last decode call, as bit words
__global__ void __launch_bounds__(256) k_dec_mask(const unsigned char* __restrict__ act8, int T, int E, int W,
                                                  uint64_t* __restrict__ mask) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= T * W) return;
  const int t = idx / W, wi = idx % W;
  uint64_t word = 0;
  for (int b = 0; b < 64; ++b) {
    const int e = wi * 64 + b;
    if (e < E && act8[(size_t)t * E + e]) word |= 1ull << b;
  }
  mask[idx] = word;
}

}  // namespace

namespace deco_host {

// Decode launch shape, chosen at load (sizes before the workspace is carved,
// the residency check once the kernels' occupancy is known).  Routed experts
// are cut into column slices of 32 columns (S = F / 32) when every routed
// slice and group of shared slices fits on the device at once (one
// workgroup per CU), else of 64 columns; the shared expert is cut into
// slices of the same width, nsub of them per workgroup
// (the smallest nsub <= 4 that lets the whole grid fit).  The waits of the up
// kernel need every group of workgroups that wait on each other (an
// expert's slices; with the RMS-only shared expert, all shared workgroups;
// with TopK routing, the whole grid) to fit on the device at once.
static void dec_sizes(deco_moe_layer* L, int np, int cap) {
  const int ncol = 16 * np;
  L->dec_np = np;
  L->dec_S = L->F / ncol;
  L->dec_n_shs = (L->Fs + ncol - 1) / ncol;
  int nsub = 1;
  while (nsub < NSUB_MAX && (L->dec_n_shs + nsub - 1) / nsub + L->E * L->dec_S > cap) nsub *= 2;
  L->dec_nsub = nsub;
  L->dec_n_sh = (L->dec_n_shs + nsub - 1) / nsub;
  L->dec_grid_up = L->dec_n_sh + L->E * L->dec_S;
}

void plan_decode_sizes(deco_moe_layer* L, int n_cu) {
  dec_sizes(L, 2, n_cu);
  if (L->F >= 64 && L->dec_grid_up > n_cu) dec_sizes(L, 4, n_cu);
  const int kp_rows = 2 * L->KB;   // rows of one column-pair fragment
  L->dec_Fp = (L->F + kp_rows - 1) / kp_rows * kp_rows;
  L->dec_Fsp = (L->Fs + kp_rows - 1) / kp_rows * kp_rows;
  L->dec_kpe = L->dec_Fp / kp_rows;
  L->dec_kps = L->dec_Fsp / kp_rows;
  L->n_hwords = L->E * L->dec_S * 16 + L->E * 16 + L->dec_n_sh * 16;
}

hipError_t plan_decode(deco_moe_layer* L) {
  void (*up)(DecArgs) = L->cfg.dtype == DECO_DT_BF16 ? up_kernel<BF16>(L->dec_np, dec_variant(L))
                                                     : up_kernel<F32>(L->dec_np, dec_variant(L));
  int occ = 0;
  hipError_t err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, up, DNT, 0);
  if (err != hipSuccess) return err;
  if (dec_variant(L) == 0) {   // the speculative variant runs too: the smaller occupancy
    void (*sp)(DecArgs) = L->cfg.dtype == DECO_DT_BF16 ? up_kernel<BF16>(L->dec_np, 0, true)
                                                       : up_kernel<F32>(L->dec_np, 0, true);
    int occ2 = 0;
    err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ2, sp, DNT, 0);
    if (err != hipSuccess) return err;
    occ = std::min(occ, occ2);
  }
  const long long cap = (long long)(occ < 1 ? 0 : occ) * L->n_cu;
  bool ok = cap >= L->dec_S && cap >= (L->cfg.shared_rms ? L->dec_n_sh : 0);
  if (L->cfg.top_k > 0) ok = ok && cap >= L->dec_grid_up;
  L->dec_ok = ok ? 1 : 0;
  return hipSuccess;
}

hipError_t launch_decode(const deco_moe_layer* L, const void* x, int T, void* out, hipStream_t s) {
  if (L->cfg.dtype == DECO_DT_BF16) return decode<BF16>(L, x, T, out, s);
  return decode<F32>(L, x, T, out, s);
}

size_t decode_scratch_bytes(const deco_moe_layer* L) { return scratch_plan(L).bytes; }
size_t decode_scratch_limit() { return SCRATCH_BYTES; }

hipError_t launch_decode_scratch(const deco_moe_layer* L, const void* x, int T, void* out, hipStream_t s) {
  const ScratchPlan sp = scratch_plan(L);
  if (sp.bytes > SCRATCH_BYTES) return hipErrorInvalidValue;   // the caller checks the size first
  char* base = nullptr;
  hipError_t err = scratch_base(&base);
  if (err != hipSuccess) return err;
  if (L->cfg.dtype == DECO_DT_BF16) return decode_scratch<BF16>(L, x, T, out, base, sp, s);
  return decode_scratch<F32>(L, x, T, out, base, sp, s);
}

hipError_t launch_dec_mask(const deco_moe_layer* L, int T, uint64_t* mask, hipStream_t s) {
  const int n = T * L->W;
  k_dec_mask<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(L->act8, T, L->E, L->W, mask);
  return hipGetLastError();
}

}  // namespace deco_host
