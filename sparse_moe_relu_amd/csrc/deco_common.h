// deco_common.h - shared device helpers of the DECO MoE HIP library (gfx950).
//
// Fragment convention used by every kernel.  A "k-block" is KB consecutive
// reduction indices; one 16-byte vector per lane of a 64-lane wave (1 KiB)
// holds a 16 x KB operand tile of an MFMA 16x16 product:
//   lane l serves row/column (l & 15) and lane group g = l >> 4, and holds
//   the EPL consecutive reduction indices k = EPL g + j (j = 0 .. EPL - 1);
//   bf16 (KB = 32, EPL = 8): consumed by one v_mfma_f32_16x16x32_bf16;
//   fp32 (KB = 16, EPL = 4): element j feeds the j-th of four
//                   v_mfma_f32_16x16x4_f32 (that MFMA sums k = 4 g + j over
//                   the four lane groups; the four together cover the block).
// The 16x16 fp32 result of a lane holds rows 4 g + i (i = 0..3) of column
// (l & 15).  Weights are packed once, at load, into this layout so each lane
// fetches its operand with one 16-byte load (a wave reads 1 KiB contiguous),
// and a row-major activation row supplies a fragment lane with one 16-byte
// load as well.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace deco {

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4_t;

constexpr int WAVE = 64;
constexpr int FRAG_BYTES = 1024;   // one k-block x 16 columns, all 64 lanes

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// round-to-nearest-even float -> bf16 bits (inputs are finite)
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;

// fp16 operands (same fragment layout as bf16).  Used for the prefill
// down-projection of bf16 layers: W_down is packed once more in fp16 (every
// bf16 value within fp16's normal range converts exactly) and the NormSiLU
// activations are rounded to fp16 (11-bit significand) instead of being split
// into two bf16 parts, which halves that projection's MFMA work.
struct FP16 {
  using elem = uint16_t;           // storage bits
  static constexpr int KB = 32;
  static constexpr int EPL = 8;
  __host__ __device__ static constexpr int frag_k(int g, int j) { return 8 * g + j; }
  __host__ __device__ static constexpr int frag_g(int w) { return w >> 3; }
  __host__ __device__ static constexpr int frag_j(int w) { return w & 7; }
  __device__ static void mma(f32x4_t& acc, const i32x4_t& a, const i32x4_t& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                 __builtin_bit_cast(f16x8_t, b), acc, 0, 0, 0);
  }
  __device__ static uint32_t bits(float f) { return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f); }
  __device__ static i32x4_t pack(const float* f) {
    i32x4_t v;
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = (int)(bits(f[2 * q]) | (bits(f[2 * q + 1]) << 16));
    return v;
  }
};

struct BF16 {
  using elem = uint16_t;
  static constexpr int KB = 32;    // k per fragment
  static constexpr int EPL = 8;    // elements per lane
  // per-(token, expert) outputs kept between the expert and combine kernels
  using pair = _Float16;
  // operand type of the prefill down-projection
  using Down = FP16;
  __host__ __device__ static constexpr int frag_k(int g, int j) { return 8 * g + j; }
  __device__ static float to_f32(elem v) { return bf16_to_f32(v); }
  __device__ static elem from_f32(float f) { return (elem)f32_to_bf16(f); }
  // lane group / element index holding in-block k index `w` (inverse of frag_k)
  __host__ __device__ static constexpr int frag_g(int w) { return w >> 3; }
  __host__ __device__ static constexpr int frag_j(int w) { return w & 7; }
  __device__ static float lane_elem(const i32x4_t& v, int j) {
    uint32_t w = (uint32_t)v[j >> 1];
    return bf16_to_f32((j & 1) ? (w >> 16) : (w & 0xFFFFu));
  }
  // acc(16x16) += A(16 x 32) * B(32 x 16)
  __device__ static void mma(f32x4_t& acc, const i32x4_t& a, const i32x4_t& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
  }
  // pack 8 floats (j order) into one lane vector
  __device__ static i32x4_t pack(const float* f) {
    i32x4_t v;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      v[q] = (int)(f32_to_bf16(f[2 * q]) | (f32_to_bf16(f[2 * q + 1]) << 16));
    return v;
  }
};

struct F32 {
  using elem = float;
  static constexpr int KB = 16;
  static constexpr int EPL = 4;
  using pair = float;
  using Down = F32;
  __host__ __device__ static constexpr int frag_k(int g, int j) { return 4 * g + j; }
  __host__ __device__ static constexpr int frag_g(int w) { return w >> 2; }
  __host__ __device__ static constexpr int frag_j(int w) { return w & 3; }
  __device__ static float to_f32(elem v) { return v; }
  __device__ static elem from_f32(float f) { return f; }
  __device__ static float lane_elem(const i32x4_t& v, int j) { return __int_as_float(v[j]); }
  __device__ static void mma(f32x4_t& acc, const i32x4_t& a, const i32x4_t& b) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__int_as_float(a[j]), __int_as_float(b[j]), acc, 0, 0, 0);
  }
  __device__ static i32x4_t pack(const float* f) {
    i32x4_t v;
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = __float_as_int(f[q]);
    return v;
  }
};

__device__ __forceinline__ i32x4_t ld16(const void* p) { return *reinterpret_cast<const i32x4_t*>(p); }
__device__ __forceinline__ void st16(void* p, const i32x4_t& v) { *reinterpret_cast<i32x4_t*>(p) = v; }
__device__ __forceinline__ i32x4_t zero16() { i32x4_t z = {0, 0, 0, 0}; return z; }

__device__ __forceinline__ float silu_f(float v) { return v / (1.0f + __expf(-v)); }

// Operand fragment of row-major data: lane (c = l & 15, g) of k-block kb of
// row `row` (elements kb*KB + frag_k(g, j)).
template <class DT>
__device__ __forceinline__ i32x4_t load_row_frag(const typename DT::elem* row, int kb, int g);
template <>
__device__ __forceinline__ i32x4_t load_row_frag<BF16>(const uint16_t* row, int kb, int g) {
  return ld16(row + kb * 32 + 8 * g);
}
template <>
__device__ __forceinline__ i32x4_t load_row_frag<F32>(const float* row, int kb, int g) {
  return ld16(row + kb * 16 + 4 * g);
}

// Byte offset, inside an array of [k-block][64 lanes][16 B] fragments, of the
// element at operand row `row` (0..15) and reduction index k.
template <class DT>
__host__ __device__ __forceinline__ size_t frag_elem_off(int row, int k) {
  const int kb = k / DT::KB, w = k % DT::KB;
  return (size_t)kb * FRAG_BYTES + (size_t)(row + 16 * DT::frag_g(w)) * 16 +
         (size_t)DT::frag_j(w) * sizeof(typename DT::elem);
}

// every memory operation this thread issued has completed
__device__ __forceinline__ void wait_all_mem() { __builtin_amdgcn_s_waitcnt(0); }

// TopK selection over one token's logits, by a wave: lane l holds
// z[j] = logit of expert 64 j + l (-inf past the last expert).  Logits map to
// unsigned keys in the same order; a bitwise binary search with ballots and
// popcounts finds the k-th largest key (32 steps, no cross-lane data
// movement), every expert above it is kept, and experts equal to it are kept
// in ascending index order until k are kept (ties to the lower index).  The
// largest key is found the same way.  Gates are the softmax of the kept
// logits: gate[j] = exp(z - zmax) / sum over kept (0 where not kept).
__device__ __forceinline__ unsigned order_key(float v) {
  const unsigned u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int NJ>
__device__ __forceinline__ unsigned kth_largest_key(const unsigned (&key)[NJ], int k) {
  unsigned prefix = 0u;
  for (int bit = 31; bit >= 0; --bit) {
    const unsigned cand = prefix | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < NJ; ++j) cnt += __popcll(__ballot(key[j] >= cand));
    if (cnt >= k) prefix = cand;
  }
  return prefix;
}

template <int NJ>
__device__ __forceinline__ void topk_wave(const float (&z)[NJ], int k, bool (&sel)[NJ], float (&gate)[NJ]) {
  const int l = threadIdx.x & 63;
  unsigned key[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) key[j] = order_key(z[j]);
  const unsigned kth = kth_largest_key<NJ>(key, k);
  const unsigned kmax = kth_largest_key<NJ>(key, 1);
  int above = 0;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    sel[j] = key[j] > kth;
    above += __popcll(__ballot(sel[j]));
  }
  int need = k - above;   // >= 1: at least one key equals the k-th largest
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    unsigned long long tie = __ballot(key[j] == kth);
    while (need > 0 && tie != 0ull) {
      const int b = __builtin_ctzll(tie);
      if (l == b) sel[j] = true;
      tie &= tie - 1ull;
      --need;
    }
  }
  // the largest logit, from its key (the map is invertible)
  const float zmax = __uint_as_float((kmax & 0x80000000u) ? (kmax & 0x7FFFFFFFu) : ~kmax);
  float part = 0.f;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    gate[j] = sel[j] ? expf(z[j] - zmax) : 0.f;
    part += gate[j];
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) part += __shfl_xor(part, o);
  const float inv = 1.0f / part;
#pragma unroll
  for (int j = 0; j < NJ; ++j) gate[j] *= inv;
}

// Offset (bytes) of k-block kb of 16-column panel p in a packed matrix with nkb k-blocks.
__host__ __device__ __forceinline__ size_t frag_off(int p, int kb, int nkb) {
  return ((size_t)p * nkb + kb) * FRAG_BYTES;
}

}  // namespace deco
