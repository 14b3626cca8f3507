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

// Pack src [K][N] (row stride ld; `batch` matrices `src_bstride` elements
// apart) into fragments: panel p (16 columns), k-block kb, lane l.  Entries
// outside K x N are zero.  Values are rounded once to the element type.
__device__ __forceinline__ float src_f32(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
__device__ __forceinline__ float src_f32(const float* p, size_t i) { return p[i]; }

template <class DT, class SRC>
__global__ void __launch_bounds__(256) k_pack(const SRC* __restrict__ src, size_t src_bstride,
                                              int K, int N, int ld, int P, int nkb,
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
    f[j] = (k < K && n < N) ? src_f32(s, (size_t)k * ld + n) : 0.f;
  }
  st16(dst + (size_t)b * dst_bstride + frag_off(p, kb, nkb) + (size_t)l * 16, DT::pack(f));
}

// W_up here is the projection NormSiLU acts on (a gated expert's gate
// projection); W_lin, when given, is a gated expert's up-projection.
template <class DT>
hipError_t pack_all(deco_moe_layer* L, const void* W_r, const void* W_up, const void* W_lin,
                    const void* W_down, const void* Ws_up, const void* Ws_down, hipStream_t s) {
  using E_t = typename DT::elem;
  const int d = L->d, E = L->E, F = L->F, Fs = L->Fs;
  const size_t dF = (size_t)d * F;
  k_mean_up<DT><<<(unsigned)((dF + 255) / 256), 256, 0, s>>>((const E_t*)W_up, E, dF, L->wbar);
  auto grid = [](int P, int nkb, int batch) {
    size_t thr = (size_t)P * nkb * WAVE;
    return dim3((unsigned)((thr + 255) / 256), (unsigned)batch);
  };
  // router: K = d, N = E (padded to multiples of 64 columns)
  k_pack<DT, E_t><<<grid(L->pR, L->nkb_d, 1), 256, 0, s>>>((const E_t*)W_r, 0, d, E, E, L->pR, L->nkb_d,
                                                           L->Wr_p, 0);
  // routed up: K = d, N = F
  k_pack<DT, E_t><<<grid(L->pF, L->nkb_d, E), 256, 0, s>>>((const E_t*)W_up, dF, d, F, F, L->pF, L->nkb_d,
                                                           L->Wup_p, L->up_stride);
  if (W_lin)
    k_pack<DT, E_t><<<grid(L->pF, L->nkb_d, E), 256, 0, s>>>((const E_t*)W_lin, dF, d, F, F, L->pF, L->nkb_d,
                                                             L->Wlin_p, L->up_stride);
  // inter-expert mean, in the layer dtype: K = d, N = F
  k_pack<DT, float><<<grid(L->pF, L->nkb_d, 1), 256, 0, s>>>(L->wbar, 0, d, F, F, L->pF, L->nkb_d,
                                                            L->Wbar_p, 0);
  // routed down: K = F, N = d
  k_pack<DT, E_t><<<grid(L->pD, L->nkb_F, E), 256, 0, s>>>((const E_t*)W_down, dF, F, d, d, L->pD, L->nkb_F,
                                                           L->Wdn_p, L->dn_stride);
  // routed down again in fp16 for the prefill path of bf16 layers
  if constexpr (sizeof(E_t) == 2)
    k_pack<FP16, E_t><<<grid(L->pD, L->nkb_F, E), 256, 0, s>>>((const E_t*)W_down, dF, F, d, d, L->pD,
                                                               L->nkb_F, L->Wdn16_p, L->dn_stride);
  // shared up: K = d, N = Fs
  k_pack<DT, E_t><<<grid(L->pFs, L->nkb_d, 1), 256, 0, s>>>((const E_t*)Ws_up, 0, d, Fs, Fs, L->pFs,
                                                            L->nkb_d, L->Wsu_p, 0);
  // shared down: K = Fs, N = d
  k_pack<DT, E_t><<<grid(L->pD, L->nkb_Fs, 1), 256, 0, s>>>((const E_t*)Ws_down, 0, Fs, d, d, L->pD,
                                                            L->nkb_Fs, L->Wsd_p, 0);
  return hipGetLastError();
}

}  // namespace

namespace deco_host {

hipError_t launch_pack_all(deco_moe_layer* L, const void* W_r, const void* W_norm, const void* W_lin,
                           const void* W_down, const void* Ws_up, const void* Ws_down, hipStream_t s) {
  if (L->cfg.dtype == DECO_DT_BF16) return pack_all<BF16>(L, W_r, W_norm, W_lin, W_down, Ws_up, Ws_down, s);
  return pack_all<F32>(L, W_r, W_norm, W_lin, W_down, Ws_up, Ws_down, s);
}

}  // namespace deco_host
