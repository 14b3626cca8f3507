// prefill.hip - bucketed forward path for large batches.
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
//   k_pre_shared_combine (DECO_PATH_PREFILL_FUSED, in place of the shared
//                        tiles and k_pre_combine) the shared expert's
//                        down-projection per 128-token tile on MFMA plus each
//                        token's pair rows (slots 1..) in slot order, in
//                        fp32, rounded once: the combine fused with the
//                        shared expert.
//
// All GEMMs run on the LDS-staged tile of gemm_tile.h with swapped operands,
// so an accumulator lane holds 4 consecutive columns of one row.  Pair values
// are fp16 (11-bit significand): a bf16 pair buffer costs up to 4 % of
// RMS(out) on heavy-tailed gates.
#include <algorithm>

#include "prefill_kernels.h"

namespace {

template <class DT, int MODE, bool SMALL>
void (*expert_kernel_m(int pF))(PreArgs) {
  return pF == 2 ? k_pre_expert<DT, 2, MODE, SMALL>
       : pF == 4 ? k_pre_expert<DT, 4, MODE, SMALL>
       : pF == 8 ? k_pre_expert<DT, 8, MODE, SMALL> : k_pre_expert<DT, 16, MODE, SMALL>;
}
// activation-output variants (the token-major down-projection follows)
template <class DT, int MODE>
void (*expert_act_kernel_m(int pF))(PreArgs) {
  return pF == 2 ? k_pre_expert<DT, 2, MODE, false, true>
       : pF == 4 ? k_pre_expert<DT, 4, MODE, false, true> : k_pre_expert<DT, 8, MODE, false, true>;
}
template <class DT>
void (*dc_kernel(int nkf))(PreArgs) {
  return nkf == 1 ? k_pre_dc<DT, 1, 2> : nkf == 2 ? k_pre_dc<DT, 2, 2> : k_pre_dc<DT, 4, 2>;
}
template <class DT>
void (*expert_kernel(int pF, bool gated, bool small = false))(PreArgs) {
  if (gated) return expert_kernel_m<DT, XM_GATED, false>(pF);   // 64-row tiles already
  return small ? expert_kernel_m<DT, XM_FWD, true>(pF) : expert_kernel_m<DT, XM_FWD, false>(pF);
}

// 64-row expert tiles when the batch would not fill half the persistent grid
// with 128-row tiles.  The count is estimated before routing (no host wait):
// the shared expert's 128 x 128 tiles plus, per expert, the 128-row tiles of
// a quarter of the tokens (the method's typical activation is about 20 %).
// Measured (same box): 64-row tiles win up to T = 1024 on the d = 2048 layer
// and at T = 256 on the d = 4096 one, and lose from T = 2048 on.
// Token-major down-projection (k_pre_dc) instead of per-pair output rows
// and a combine: only when asked for (DECO_PATH_PREFILL_TOKEN).  Measured on
// the d = 2048 and d = 4096 layers at T = 128 .. 4096 it is slower than the
// expert-major tiles at every size (c3 T = 4096: 283-293 against 235 us per
// call): every (256-token, 128-column) block streams its column slice of all
// experts' W_down, 1.8 MiB, and one CU pulls 30-60 GB/s from beyond its L2.
int dc_nkf(const deco_moe_layer* L) { return L->F / L->KB; }
long long dc_blocks(const deco_moe_layer* L, int T) {
  return (long long)((T + 2 * GM - 1) / (2 * GM)) * ((L->pD + GP - 1) / GP);
}
bool use_dc(const deco_moe_layer* L, int T, int path) {
  (void)L;
  (void)T;
  return path == DECO_PATH_PREFILL_TOKEN;
}

long long est_shared_tiles(const deco_moe_layer* L, int T) {
  return (long long)((T + GM - 1) / GM) * ((L->pD + GP - 1) / GP);
}
long long est_expert_tiles(const deco_moe_layer* L, int T, int bm) { return (long long)L->E * ((T / 4 + bm - 1) / bm); }
bool small_tiles_at(const deco_moe_layer* L, int T, long long grid) {
  return 2 * (est_shared_tiles(L, T) + est_expert_tiles(L, T, GM)) < grid;
}
#ifndef DECO_PRE_FORCE_SMALL
#define DECO_PRE_FORCE_SMALL -1   // measurement builds: 0 / 1 force 128- / 64-row expert tiles
#endif
bool small_expert_tiles(const deco_moe_layer* L, int T) {
  if (DECO_PRE_FORCE_SMALL >= 0) return DECO_PRE_FORCE_SMALL != 0;
  return small_tiles_at(L, T, L->pre_grid);
}

// Small batches of a non-gated layer split each 64-row expert tile over nks
// k parts of the up-projection and ncb column blocks of the down-projection
// (k_pre_expert, PART): at T = 256 on the d = 4096 layer the 64-row tiles
// leave one thin tile per expert, and one CU streams 2 d F of weights for
// it.  nks: the k-blocks of d in 4 (or 2) parts of at least 8; ncb: the
// largest power of two up to 4 whose units, with the shared tiles, stay
// within one per workgroup of the persistent grid.
#ifndef DECO_SPLIT_NKS
#define DECO_SPLIT_NKS 0   // 0: chosen from the shape
#endif
#ifndef DECO_SPLIT_NCB
#define DECO_SPLIT_NCB 0
#endif
int split_nks(const deco_moe_layer* L);
bool use_split(const deco_moe_layer* L, int T) {
#ifdef DECO_NO_SPLIT
  return false;   // measurement builds: the unsplit 64-row tiles
#endif
  // and only while the k-part units fit the grid in one pass: with more
  // 64-row tiles per expert the unsplit tiles already spread the weights
  // (same-box A/B, us per call: d = 4096 layer T = 64 / 256 / 512: 141.7 /
  // 151.3 / 175.2 unsplit, 98.7 / 126.9 / 181.9 split; d = 2048 layer
  // T = 32 / 128 / 512: 78.0 / 80.4 / 84.8 against 51.1 / 57.6 / 76.3, and
  // T = 1024: 96.0 against 109.3)
  return L->hpart && !L->gated && T <= L->split_maxT && small_expert_tiles(L, T) &&
         est_expert_tiles(L, T, GM / 2) * split_nks(L) <= (long long)L->pre_grid;
}
int split_nks(const deco_moe_layer* L) {
  static_assert(DECO_SPLIT_NKS <= deco_host::SPLIT_NKS_MAX, "k parts beyond the buffer");
  if (DECO_SPLIT_NKS && L->nkb_d % DECO_SPLIT_NKS == 0) return DECO_SPLIT_NKS;
  for (int q : {deco_host::SPLIT_NKS_MAX, 2})
    if (L->nkb_d % q == 0 && L->nkb_d / q >= 8) return q;
  return 1;
}
int split_ncb(const deco_moe_layer* L, int T, int dp, bool fused) {
  const int nds = L->pD / dp;
  if (DECO_SPLIT_NCB) return nds % DECO_SPLIT_NCB == 0 ? DECO_SPLIT_NCB : 1;
  const long long units = est_expert_tiles(L, T, GM / 2);
  const long long shared =
      fused ? 0 : (long long)((T + GM - 1) / GM) * ((L->pD + DECO_SPLIT_SGP - 1) / DECO_SPLIT_SGP);
  int ncb = 1;
  while (ncb < 4 && nds % (2 * ncb) == 0 && shared + units * 2 * ncb <= (long long)L->pre_grid) ncb *= 2;
  return ncb;
}
template <class DT>
void (*split_kernel(int pF, int part))(PreArgs) {
  if (part == 1)
    return pF == 2 ? k_pre_expert<DT, 2, XM_FWD, true, false, 1>
         : pF == 4 ? k_pre_expert<DT, 4, XM_FWD, true, false, 1>
         : pF == 8 ? k_pre_expert<DT, 8, XM_FWD, true, false, 1> : k_pre_expert<DT, 16, XM_FWD, true, false, 1>;
  return pF == 2 ? k_pre_expert<DT, 2, XM_FWD, true, false, 2>
       : pF == 4 ? k_pre_expert<DT, 4, XM_FWD, true, false, 2>
       : pF == 8 ? k_pre_expert<DT, 8, XM_FWD, true, false, 2> : k_pre_expert<DT, 16, XM_FWD, true, false, 2>;
}

// The combine fused with the shared expert's down-projection
// (k_pre_shared_combine, DECO_PATH_PREFILL_FUSED): 128-token tiles 8 panels
// wide, or 4 or 2 when the batch makes fewer 8-panel tiles than CUs.  Only
// when asked for: same-box A/B, us per call, fused against the shared tiles
// inside k_pre_expert plus k_pre_combine: d = 2048 layer T = 4096 256.0 /
// 241.9, T = 128 70.6 / 55.9; d = 4096 layer T = 256 145.0 / 126.5, T = 2048
// 431.2 / 429.0.  The fused kernel's workgroups run the shared GEMM's K loop
// and then stream their tokens' pair rows, one after the other (76 us at
// T = 4096 against 38 us of combine and ~18 us of shared tiles that ran
// beside the expert tiles).
int shared_combine_sgp(const deco_moe_layer* L, int T) {
  const long long mt = (T + GM - 1) / GM;
  if (mt * ((L->pD + 7) / 8) >= L->n_cu) return 8;
  if (mt * ((L->pD + 3) / 4) >= L->n_cu) return 4;
  return 2;
}
template <class DT>
void (*shared_combine_kernel(int sgp))(PreArgs) {
  return sgp == 8 ? k_pre_shared_combine<DT, 8> : sgp == 4 ? k_pre_shared_combine<DT, 4> : k_pre_shared_combine<DT, 2>;
}

template <class DT>
hipError_t prefill(const deco_moe_layer* L, const void* x, int T, void* out, hipStream_t s, int path) {
  PreArgs a = fill_pre_args(L, x, T, out);
  a.fuse_shared = path == DECO_PATH_PREFILL_FUSED ? 1 : 0;
  using deco_host::launch;
  hipError_t err = launch_routing<DT>(L, a, T, s);
  if (use_dc(L, T, path)) {
    if (err == hipSuccess)
      err = launch(deco_host::KS_PRE_EXPERT,
                   L->gated ? expert_act_kernel_m<DT, XM_GATED>(L->pF) : expert_act_kernel_m<DT, XM_FWD>(L->pF),
                   dim3(L->pre_grid), dim3(256), s, a);
    if (err == hipSuccess)
      err = launch(deco_host::KS_PRE_DC, dc_kernel<DT>(dc_nkf(L)), dim3((unsigned)dc_blocks(L, T)), dim3(512), s, a);
  } else if (use_split(L, T)) {
    PreArgs b = a;
    b.nks = split_nks(L);
    b.ncb = split_ncb(L, T, (L->F / (L->cfg.dtype == DECO_DT_BF16 ? FP16::KB : F32::KB)) >= 8 ? 2 : 4, a.fuse_shared);
    if (err == hipSuccess)
      err = launch(deco_host::KS_PRE_UP_PART, split_kernel<DT>(L->pF, 1), dim3(L->pre_grid), dim3(256), s, b);
    if (err == hipSuccess)
      err = launch(deco_host::KS_PRE_EXPERT, split_kernel<DT>(L->pF, 2), dim3(L->pre_grid), dim3(256), s, b);
  } else {
    if (err == hipSuccess)
      err = launch(deco_host::KS_PRE_EXPERT, expert_kernel<DT>(L->pF, L->gated, small_expert_tiles(L, T)),
                   dim3(L->pre_grid), dim3(256), s, a);
  }
  if (!use_dc(L, T, path) && err == hipSuccess) {
    if (a.fuse_shared) {
      const int sgp = shared_combine_sgp(L, T);
      const unsigned grid = (unsigned)(((T + GM - 1) / GM) * ((L->pD + sgp - 1) / sgp));
      err = launch(deco_host::KS_PRE_COMBINE, shared_combine_kernel<DT>(sgp), dim3(grid), dim3(256), s, a);
    } else {
      err = launch(deco_host::KS_PRE_COMBINE, k_pre_combine<DT>,
                   dim3((unsigned)(((long long)T * (L->d / 8) + 255) / 256)), dim3(256), s, a);
    }
  }
  if (err != hipSuccess) return err;
  return hipGetLastError();
}

}  // namespace

namespace deco_host {

hipError_t launch_prefill(const deco_moe_layer* L, const void* x, int T, void* out, hipStream_t s, int path) {
  if (L->cfg.dtype == DECO_DT_BF16) return prefill<BF16>(L, x, T, out, s, path);
  return prefill<F32>(L, x, T, out, s, path);
}

bool prefill_token_ok(const deco_moe_layer* L) { return dc_nkf(L) <= 4; }

// Largest batch the small-batch split can take on a grid of `grid`
// workgroups (0 for gated layers, which keep their own tiles); the K-part
// buffer is sized for it at load.
int split_max_tokens(const deco_moe_layer* L, long long grid) {
  if (L->gated) return 0;
  const int tcap = std::min(L->maxT < 16 ? 16 : L->maxT, 2048);
  int best = 0;
  for (int T = 1; T <= tcap; ++T)
    if (small_tiles_at(L, T, grid) && est_expert_tiles(L, T, GM / 2) * split_nks(L) <= grid) best = T;
  return best;
}

// Persistent grid of the expert kernel: as many workgroups as fit on the
// device at once, a multiple of the 8 XCDs.
hipError_t plan_prefill(deco_moe_layer* L) {
  void (*kx)(PreArgs) = L->cfg.dtype == DECO_DT_BF16 ? expert_kernel<BF16>(L->pF, L->gated)
                                                    : expert_kernel<F32>(L->pF, L->gated);
  int occ = 0, cus = 0;
  hipError_t err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kx, 256, 0);
  if (err == hipSuccess) err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, L->device);
  if (err != hipSuccess) return err;
  int grid = (occ < 1 ? 1 : occ) * (cus < 1 ? 1 : cus);
  grid = (grid + NXCD - 1) / NXCD * NXCD;
  L->pre_grid = grid;
  L->n_cu = cus < 1 ? 1 : cus;
  return hipSuccess;
}

}  // namespace deco_host
