// gemm_tile.h - LDS-staged MFMA tile used by the prefill kernels (gfx950).
//
// A workgroup of 4 waves computes a BM x (16*BNP) tile of C += A.B, with the
// waves in a 2 x 2 grid (each wave: BM/2 rows x BNP/2 panels).  K advances in
// steps of 2 k-blocks (128 bytes of each A row) through a ring of NS stages
// in LDS.  Operands go from global memory straight into LDS
// (global_load_lds_dwordx4: lane l's 16 bytes land at 16-byte slot l of a
// 1 KiB block):
//   A: row-major rows (any row addresses: gathered or strided).  One block
//      holds 8 rows x 128 bytes, so each load instruction reads 8 whole
//      128-byte lines.  Slot 8 r + s of a block holds 16-byte chunk s ^ r of
//      row r (an XOR swizzle): the 8 lanes that read chunk j of 8 different
//      rows hit 8 different bank groups.
//   B: weights packed in MFMA fragment order (16-column panels of 1 KiB
//      k-blocks, deco_common.h), copied as is.
// No operand passes through registers on its way in, and NS - 1 steps of
// loads are in flight while one step computes.  Waits are explicit vmcnt
// counts (each wave issues the same number of loads per step) followed by an
// LDS-only barrier.  A kernel using the tile keeps all its LDS in one array:
// the compiler cannot tell the LDS-DMA writes of one array from reads of
// another and would otherwise wait for every DMA before every LDS read.
#pragma once

#include "deco_common.h"

namespace deco {

typedef __attribute__((address_space(3))) void* lds_ptr_t;

template <class DT, int BM_, int BNP_, int NS_>
struct Tile {
  static constexpr int NT = 256;                  // threads per workgroup
  static constexpr int BM = BM_, BNP = BNP_, KS = 2, NS = NS_;
  static constexpr int MB = BM / 32;              // 16-row blocks per wave
  static constexpr int NBW = BNP / 2;             // panels per wave
  static constexpr int NA = BM / 8;               // A blocks (8 rows x 128 bytes) per step
  static constexpr int NB = BNP * KS;             // B fragments per step
  static constexpr int NAW = NA / 4, NBL = NB / 4;   // per wave
  static constexpr int LPW = NAW + NBL;           // loads per wave per step
  static constexpr int A_V = NA * 64;             // 16-byte LDS slots of A in one stage
  static constexpr int B_V = NB * 64;
  static constexpr int STAGE_V = A_V + B_V;
  static constexpr int LDS_V = NS * STAGE_V;      // slots of the whole ring
  static_assert(BM % 32 == 0 && BNP % 2 == 0, "tile shape");
  static_assert(NA % 4 == 0 && NB % 4 == 0, "blocks must divide over the 4 waves");
  static_assert(KS * DT::KB * sizeof(typename DT::elem) == 128, "a step covers 128 bytes of an A row");
  static_assert(NS >= 2, "at least two stages");
};

// s_waitcnt with vmcnt <= N and the other counters unconstrained (gfx9
// encoding: vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for LDS hand-offs.  It waits for this wave's LDS reads
// and writes (lgkmcnt 0) but not for its global loads, stores or LDS-DMA
// loads: a memory fence (__syncthreads(), or even an LDS-only fence, since
// DMA loads in flight are pending LDS writes) would wait for all of those
// and empty every prefetch ring at every barrier.  Where a DMA stage must
// have landed, the caller waits for it with wait_vmcnt first.  The empty asm
// statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt unconstrained
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

__device__ __forceinline__ void load_lds16(const void* src, i32x4_t* lds_block) {
  __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)lds_block, 16, 0, 0);
}

// acc[i][j] += A(wave rows block i) . B(wave panel j) over the first kb_lim
// (<= KS) k-blocks of one stage.  SWAP = false: lane (c, g) of acc[i][j]
// holds rows 4 g + ii, column c of the 16 x 16 block.  SWAP = true: the MFMA
// operands are swapped (the A and B fragments share one lane layout), so the
// lane holds row c and the 4 consecutive columns 4 g + ii: epilogues then
// store 8 or 16 bytes of one row per lane instead of 4 scattered elements.
template <class DT, class TC, bool SWAP>
__device__ __forceinline__ void tile_mma(const i32x4_t* lds_a, const i32x4_t* lds_b,
                                         f32x4_t (&acc)[TC::MB][TC::NBW], int wm, int wn, int kb_lim) {
  const int l = threadIdx.x & 63;
#pragma unroll
  for (int kb = 0; kb < TC::KS; ++kb) {
    if (kb < kb_lim) {
      i32x4_t av[TC::MB], bv[TC::NBW];
#pragma unroll
      for (int i = 0; i < TC::MB; ++i) {
        // row 16 (wm*MB + i) + c lives in block 2 (wm*MB + i) + c / 8 at row c % 8;
        // this lane's chunk is k-block kb, quarter g
        const int c = l & 15, rl = c & 7;
        av[i] = lds_a[(2 * (wm * TC::MB + i) + (c >> 3)) * 64 + rl * 8 + ((kb * 4 + (l >> 4)) ^ rl)];
      }
#pragma unroll
      for (int j = 0; j < TC::NBW; ++j) bv[j] = lds_b[((wn * TC::NBW + j) * TC::KS + kb) * 64 + l];
#pragma unroll
      for (int i = 0; i < TC::MB; ++i)
#pragma unroll
        for (int j = 0; j < TC::NBW; ++j) {
          if constexpr (SWAP) DT::mma(acc[i][j], bv[j], av[i]);
          else DT::mma(acc[i][j], av[i], bv[j]);
        }
    }
  }
}

// Full K loop: acc += A[BM x K] . B[K x 16 BNP], K = nkb k-blocks, with the
// ring in `lds` (TC::LDS_V slots).  row(r) (r < BM) returns row r's element
// pointer and panel(p) (p < BNP) panel p's base (k-block 0); both must be
// readable for nkb k-blocks even where the result is not wanted (padding rows
// or panels: point them at any valid row or panel and drop those outputs).
// Wave w = threadIdx.x / 64 computes rows (w / 2) * BM / 2 and panels
// (w % 2) * BNP / 2 of the tile.  Ends with a barrier, so the caller may
// reuse the ring at once.  `tid` is the thread's index in its group of 256
// (a larger workgroup runs one tile per group of four waves, each group with
// its own ring and the same number of steps, so the barriers line up).
template <class DT, class TC, bool SWAP, class RowF, class PanelF>
__device__ __forceinline__ void tile_gemm(i32x4_t* lds, RowF row, PanelF panel, int nkb,
                                          f32x4_t (&acc)[TC::MB][TC::NBW], int tid) {
  using elem = typename DT::elem;
  const int w = tid >> 6, l = tid & 63, wm = w >> 1, wn = w & 1;
  const int nsteps = (nkb + TC::KS - 1) / TC::KS;
  // this wave's loads: A blocks fa = w*NAW + i (rows 8 fa ..; lane l loads
  // row 8 fa + l / 8, chunk ch = (l % 8) ^ (l / 8)), B fragments fb = w*NBL + i
  // (panel fb / KS, k-block fb % KS)
  const int ch = (l & 7) ^ (l >> 3);
  const elem* rp[TC::NAW];
#pragma unroll
  for (int i = 0; i < TC::NAW; ++i) {
    const int fa = w * TC::NAW + i;
    rp[i] = row(8 * fa + (l >> 3)) + (ch & 3) * DT::EPL;
  }
  const char* pp[TC::NBL];
#pragma unroll
  for (int i = 0; i < TC::NBL; ++i) {
    const int fb = w * TC::NBL + i;
    pp[i] = panel(fb / TC::KS) + l * 16;
  }
  auto issue = [&](int s) {
    i32x4_t* st = lds + (s % TC::NS) * TC::STAGE_V;
    int kba = s * TC::KS + (ch >> 2);
    kba = kba < nkb ? kba : nkb - 1;   // past the end: a valid block, its MFMAs are skipped
#pragma unroll
    for (int i = 0; i < TC::NAW; ++i) load_lds16(rp[i] + kba * DT::KB, st + (w * TC::NAW + i) * 64);
#pragma unroll
    for (int i = 0; i < TC::NBL; ++i) {
      const int fb = w * TC::NBL + i;
      int kb = s * TC::KS + fb % TC::KS;
      kb = kb < nkb ? kb : nkb - 1;
      load_lds16(pp[i] + (size_t)kb * FRAG_BYTES, st + TC::A_V + fb * 64);
    }
  };
#pragma unroll
  for (int s = 0; s < TC::NS - 1; ++s)
    if (s < nsteps) issue(s);
  for (int s = 0; s < nsteps; ++s) {
    // this wave's loads of step s are done once at most the later steps'
    // loads are outstanding; the barrier then makes every wave's visible,
    // and shows that every wave has finished reading step s - 1's stage
    if (s + TC::NS - 2 < nsteps) wait_vmcnt<(TC::NS - 2) * TC::LPW>();
    else wait_vmcnt<0>();
    lds_barrier();
    if (s + TC::NS - 1 < nsteps) issue(s + TC::NS - 1);
    const i32x4_t* st = lds + (s % TC::NS) * TC::STAGE_V;
    tile_mma<DT, TC, SWAP>(st, st + TC::A_V, acc, wm, wn, nkb - s * TC::KS);
  }
  lds_barrier();
}

template <class DT, class TC, bool SWAP, class RowF, class PanelF>
__device__ __forceinline__ void tile_gemm(i32x4_t* lds, RowF row, PanelF panel, int nkb,
                                          f32x4_t (&acc)[TC::MB][TC::NBW]) {
  tile_gemm<DT, TC, SWAP>(lds, row, panel, nkb, acc, (int)threadIdx.x);
}

}  // namespace deco
