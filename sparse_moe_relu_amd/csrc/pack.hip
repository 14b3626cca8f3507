// pack.hip - load-time preprocessing: inter-expert mean of the up-projections
// and packing of every weight matrix into the fragment layout of deco_common.h.
//
// The NormSiLU mean term is a fixed matrix at inference (the average of all
// routed experts' up-projection weights; qidianchuan.cn write-up of DECO,
// section 二, expert design), so Wbar is built once here, in fp32, and also
// packed in the layer dtype for the forward kernels, which compute x.Wbar
// once per token and subtract it from every expert's up-projection.  (Folding
// Wbar into each expert's packed weights would save that product but rounds
// W_up[e] - Wbar to the dtype, which costs about 1 % of RMS(out) in bf16.)
#include <string.h>

#include "deco_common.h"
#include "deco_internal.h"

using namespace deco;

namespace {

// Wbar[k][f] = (1/E) * sum_e W_up[e][k][f], fp32, summed in ascending e.
template <class DT>
__global__ void __launch_bounds__(256) k_mean_up(const typename DT::elem* __restrict__ W_up, int E,
                                                 size_t dF, float* __restrict__ wbar) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= dF) return;
  float s = 0.f;
  for (int e = 0; e < E; ++e) s += DT::to_f32(W_up[(size_t)e * dF + i]);
  wbar[i] = s / (float)E;
}

// Fragments of W_up[e] - Wbar (row-major [d][F] sources, `batch` experts):
// the difference in fp32 (W_up values are exact in fp32, Wbar is fp32),
// rounded once to OUT (fp16 for bf16 layers: 11 significant bits instead of
// bf16's 8 keep the folded matrix about as accurate as subtracting a
// separately formed mean term).
template <class DT, class OUT>
__global__ void __launch_bounds__(256) k_pack_minus_mean(const typename DT::elem* __restrict__ src, size_t src_bstride,
                                                         const float* __restrict__ wbar, int K, int N, int P, int nkb,
                                                         char* __restrict__ dst, size_t dst_bstride) {
  const int b = blockIdx.y;
  const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t total = (size_t)P * nkb * WAVE;
  if (t >= total) return;
  const int l = (int)(t % WAVE);
  const int kb = (int)((t / WAVE) % nkb);
  const int p = (int)(t / ((size_t)WAVE * nkb));
  const int g = l >> 4, c = l & 15;
  const int n = p * 16 + c;
  const typename DT::elem* s = src + (size_t)b * src_bstride;
  float f[DT::EPL];
#pragma unroll
  for (int j = 0; j < DT::EPL; ++j) {
    const int k = kb * DT::KB + DT::frag_k(g, j);
    const size_t i = (size_t)k * N + n;
    f[j] = (k < K && n < N) ? DT::to_f32(s[i]) - wbar[i] : 0.f;
  }
  st16(dst + (size_t)b * dst_bstride + frag_off(p, kb, nkb) + (size_t)l * 16, OUT::pack(f));
}

// Pack the K x N matrix src(k, n) = src[k*sk + n*sn] (`batch` matrices
// `src_bstride` elements apart; sk = ld, sn = 1 for a row-major [K][N]
// matrix, sk = 1, sn = ld for the transpose of a row-major [N][K] one) into
// fragments: panel p (16 columns), k-block kb_off + kb of a layout with
// nkb_tot k-blocks, lane l.  Entries outside K x N are zero.  Values are
// rounded once to the element type.
__device__ __forceinline__ float src_f32(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
__device__ __forceinline__ float src_f32(const float* p, size_t i) { return p[i]; }

// LO: pack v - bf16(v), the part of an fp32 value a bf16 copy drops
template <class DT, class SRC, bool LO = false>
__global__ void __launch_bounds__(256) k_pack(const SRC* __restrict__ src, size_t src_bstride,
                                              int K, int N, size_t sk, size_t sn, int P, int nkb,
                                              int kb_off, int nkb_tot,
                                              char* __restrict__ dst, size_t dst_bstride) {
  const int b = blockIdx.y;
  const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t total = (size_t)P * nkb * WAVE;
  if (t >= total) return;
  const int l = (int)(t % WAVE);
  const int kb = (int)((t / WAVE) % nkb);
  const int p = (int)(t / ((size_t)WAVE * nkb));
  const int g = l >> 4, c = l & 15;
  const int n = p * 16 + c;
  const SRC* s = src + (size_t)b * src_bstride;
  float f[DT::EPL];
#pragma unroll
  for (int j = 0; j < DT::EPL; ++j) {
    const int k = kb * DT::KB + DT::frag_k(g, j);
    f[j] = (k < K && n < N) ? src_f32(s, (size_t)k * sk + (size_t)n * sn) : 0.f;
    if constexpr (LO) f[j] -= bf16_to_f32(f32_to_bf16(f[j]));
  }
  st16(dst + (size_t)b * dst_bstride + frag_off(p, kb_off + kb, nkb_tot) + (size_t)l * 16, DT::pack(f));
}

// Column-pair packing of the K x N row-major matrix src (`batch` matrices
// `src_bstride` elements apart) for the decode down-projection: fragment
// (column group cg of 8 columns, k-pair kp) holds, in lane l (c = l & 15,
// g = l >> 4), rows (2 kp + c / 8) * KB + frag_k(g, j) of column 8 cg + c % 8,
// so MFMA tile columns 0-7 take the first k-block of the pair and columns
// 8-15 the second.  Layout [cg][kp], entries outside K x N zero.
template <class DT, class SRC>
__global__ void __launch_bounds__(256) k_pack_pair(const SRC* __restrict__ src, size_t src_bstride, int K, int N,
                                                   int ncg, int nkp, char* __restrict__ dst, size_t dst_bstride) {
  const int b = blockIdx.y;
  const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (size_t)ncg * nkp * WAVE) return;
  const int l = (int)(t % WAVE);
  const int kp = (int)((t / WAVE) % nkp);
  const int cg = (int)(t / ((size_t)WAVE * nkp));
  const int g = l >> 4, c = l & 15;
  const int n = 8 * cg + (c & 7);
  const SRC* s = src + (size_t)b * src_bstride;
  float f[DT::EPL];
#pragma unroll
  for (int j = 0; j < DT::EPL; ++j) {
    const int k = (2 * kp + (c >> 3)) * DT::KB + DT::frag_k(g, j);
    f[j] = (k < K && n < N) ? src_f32(s, (size_t)k * N + n) : 0.f;
  }
  st16(dst + (size_t)b * dst_bstride + ((size_t)cg * nkp + kp) * FRAG_BYTES + (size_t)l * 16, DT::pack(f));
}

// Largest |W_down| of a bf16 layer, as fp32 bits (non-negative floats order
// like their bit patterns; NaN patterns sort above inf, so they count as out
// of range): bf16 layers feed W_down to the down-projection in fp16.
__global__ void __launch_bounds__(256) k_absmax_bf16(const uint16_t* __restrict__ w, size_t n,
                                                     unsigned* __restrict__ out) {
  unsigned m = 0;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const unsigned b = ((unsigned)w[i] << 16) & 0x7FFFFFFFu;
    m = b > m ? b : m;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const unsigned y = (unsigned)__shfl_xor((int)m, o);
    m = y > m ? y : m;
  }
  if ((threadIdx.x & 63) == 0) atomicMax(out, m);
}

dim3 pack_grid(int P, int nkb, int batch) {
  size_t thr = (size_t)P * nkb * WAVE;
  return dim3((unsigned)((thr + 255) / 256), (unsigned)batch);
}

// row-major [K][N] source, whole layout
template <class DT, class SRC>
void pack_rm(const void* src, size_t bstride, int K, int N, int P, int nkb, char* dst, size_t dstride, int batch,
             hipStream_t s) {
  k_pack<DT, SRC><<<pack_grid(P, nkb, batch), 256, 0, s>>>((const SRC*)src, bstride, K, N, (size_t)N, 1, P, nkb, 0,
                                                           nkb, dst, dstride);
}

// transpose of a row-major [N][K] source (element (k, n) = src[n*K + k]),
// written to k-blocks kb_off .. of a layout with nkb_tot k-blocks
template <class DT, class SRC>
void pack_tr(const void* src, size_t bstride, int K, int N, int P, int nkb, int kb_off, int nkb_tot, char* dst,
             size_t dstride, int batch, hipStream_t s) {
  k_pack<DT, SRC><<<pack_grid(P, nkb, batch), 256, 0, s>>>((const SRC*)src, bstride, K, N, 1, (size_t)K, P, nkb,
                                                           kb_off, nkb_tot, dst, dstride);
}

// W_up here is the projection NormSiLU acts on (a gated expert's gate
// projection); W_lin, when given, is a gated expert's up-projection.
template <class DT>
hipError_t pack_all(deco_moe_layer* L, const void* W_r, const void* W_up, const void* W_lin,
                    const void* W_down, const void* Ws_up, const void* Ws_down, hipStream_t s) {
  using E_t = typename DT::elem;
  using DN = typename DT::Down;
  const int d = L->d, E = L->E, F = L->F, Fs = L->Fs;
  const size_t dF = (size_t)d * F;
  k_mean_up<DT><<<(unsigned)((dF + 255) / 256), 256, 0, s>>>((const E_t*)W_up, E, dF, L->wbar);
  // router: K = d, N = E (padded to multiples of 64 columns)
  pack_rm<DT, E_t>(W_r, 0, d, E, L->pR, L->nkb_d, L->Wr_p, 0, 1, s);
  // routed up: K = d, N = F
  pack_rm<DT, E_t>(W_up, dF, d, F, L->pF, L->nkb_d, L->Wup_p, L->up_stride, E, s);
  if (L->Wupm_p)
    k_pack_minus_mean<DT, DN><<<pack_grid(L->pF, L->nkb_d, E), 256, 0, s>>>((const E_t*)W_up, dF, L->wbar, d, F,
                                                                           L->pF, L->nkb_d, L->Wupm_p, L->up_stride);
  if (W_lin) pack_rm<DT, E_t>(W_lin, dF, d, F, L->pF, L->nkb_d, L->Wlin_p, L->up_stride, E, s);
  // inter-expert mean, in the layer dtype: K = d, N = F
  pack_rm<DT, float>(L->wbar, 0, d, F, L->pF, L->nkb_d, L->Wbar_p, 0, 1, s);
  // routed down: K = F, N = d
  pack_rm<DT, E_t>(W_down, dF, F, d, L->pD, L->nkb_F, L->Wdn_p, L->dn_stride, E, s);
  // routed down again in fp16 for bf16 layers (the down-projection operand)
  if constexpr (sizeof(E_t) == 2)
    pack_rm<FP16, E_t>(W_down, dF, F, d, L->pD, L->nkb_F, L->Wdn16_p, L->dn_stride, E, s);
  // shared up: K = d, N = Fs; shared down: K = Fs, N = d
  pack_rm<DT, E_t>(Ws_up, 0, d, Fs, L->pFs, L->nkb_d, L->Wsu_p, 0, 1, s);
  pack_rm<DT, E_t>(Ws_down, 0, Fs, d, L->pD, L->nkb_Fs, L->Wsd_p, 0, 1, s);
  // the decode down-projection's column-pair copies: routed W_down in the
  // down operand type, Ws_down in the layer dtype
  {
    const int ncg = d / 8;
    const size_t thr_r = (size_t)ncg * L->dec_kpe * WAVE, thr_s = (size_t)ncg * L->dec_kps * WAVE;
    k_pack_pair<DN, E_t><<<dim3((unsigned)((thr_r + 255) / 256), (unsigned)E), 256, 0, s>>>(
        (const E_t*)W_down, dF, F, d, ncg, L->dec_kpe, L->Wdn8_p, L->dn8_stride);
    k_pack_pair<DT, E_t><<<dim3((unsigned)((thr_s + 255) / 256), 1u), 256, 0, s>>>(
        (const E_t*)Ws_down, 0, Fs, d, ncg, L->dec_kps, L->Wsd8_p, 0);
  }
  if (L->cfg.backward) {
    // W_down[e]^T: K = d, N = F (the ungated output gradient times W_down^T)
    pack_tr<DT, E_t>(W_down, dF, d, F, L->pF, L->nkb_d, 0, L->nkb_d, L->WdnT_p, L->up_stride, E, s);
    // W_up[e]^T: K = F, N = d, in the down-projection operand type
    pack_tr<DN, E_t>(W_up, dF, F, d, L->pD, L->nkb_F, 0, L->nkb_F, L->WupT_p, L->dn_stride, E, s);
    // Ws_down^T: K = d, N = Fs
    pack_tr<DT, E_t>(Ws_down, 0, d, Fs, L->pFs, L->nkb_d, 0, L->nkb_d, L->WsdT_p, 0, 1, s);
    // [Wbar^T; W_r^T; Ws_up^T]: K = Fp + Ep + Fsp, N = d (sections zero-padded)
    const int KB = DT::KB;
    pack_tr<DT, float>(L->wbar, 0, F, d, L->pD, L->Fp / KB, 0, L->nkb_cat, L->Bcat_p, 0, 1, s);
    pack_tr<DT, E_t>(W_r, 0, E, d, L->pD, L->Ep / KB, L->Fp / KB, L->nkb_cat, L->Bcat_p, 0, 1, s);
    pack_tr<DT, E_t>(Ws_up, 0, Fs, d, L->pD, L->Fsp / KB, (L->Fp + L->Ep) / KB, L->nkb_cat, L->Bcat_p, 0, 1, s);
    // the low part of Wbar (K = d, N = F): the backward's mean term is x . (Wbar_bf16 + Wbar_lo)
    if constexpr (sizeof(E_t) == 2)
      k_pack<DT, float, true><<<pack_grid(L->pF, L->nkb_d, 1), 256, 0, s>>>(L->wbar, 0, d, F, (size_t)F, 1, L->pF,
                                                                            L->nkb_d, 0, L->nkb_d, L->WbarLo_p, 0);
  }
  return hipGetLastError();
}

}  // namespace

namespace deco_host {

// bf16 layers: is every |W_down| within the fp16 range (the down-projection's
// operand type)?  Synchronous (load time); uses the layer's mbuf as scratch.
// *ok = every |w[i]| <= limit, for n bf16 values on the device
static hipError_t check_abs_below(deco_moe_layer* L, const void* w, size_t n, float limit, hipStream_t s, bool* ok) {
  unsigned* word = (unsigned*)L->mbuf;
  hipError_t err = hipMemsetAsync(word, 0, sizeof(unsigned), s);
  if (err != hipSuccess) return err;
  k_absmax_bf16<<<1024, 256, 0, s>>>((const uint16_t*)w, n, word);
  err = hipGetLastError();
  unsigned bits = 0;
  if (err == hipSuccess) err = hipMemcpyAsync(&bits, word, sizeof(bits), hipMemcpyDeviceToHost, s);
  if (err == hipSuccess) err = hipStreamSynchronize(s);
  if (err != hipSuccess) return err;
  unsigned lim = 0;
  memcpy(&lim, &limit, sizeof(lim));
  *ok = bits <= lim;
  return hipSuccess;
}

hipError_t check_down_range(deco_moe_layer* L, const void* W_down, const void* W_norm, hipStream_t s, bool* ok) {
  *ok = true;
  if (L->cfg.dtype != DECO_DT_BF16) return hipSuccess;
  const size_t n = (size_t)L->E * L->F * L->d;
  hipError_t err = check_abs_below(L, W_down, n, 65504.f, s, ok);
  // the decode path's folded NormSiLU input W - Wbar in fp16: |W - Wbar| <=
  // 2 max |W| stays in range below half the fp16 maximum
  if (err == hipSuccess && *ok && (L->cfg.normsilu & DECO_NORMSILU_NO_MEAN) == 0)
    err = check_abs_below(L, W_norm, n, 32752.f, s, ok);
  return err;
}

hipError_t launch_pack_all(deco_moe_layer* L, const void* W_r, const void* W_norm, const void* W_lin,
                           const void* W_down, const void* Ws_up, const void* Ws_down, hipStream_t s) {
  if (L->cfg.dtype == DECO_DT_BF16) return pack_all<BF16>(L, W_r, W_norm, W_lin, W_down, Ws_up, Ws_down, s);
  return pack_all<F32>(L, W_r, W_norm, W_lin, W_down, Ws_up, Ws_down, s);
}

}  // namespace deco_host
