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
//
// All GEMMs run on the LDS-staged tile of gemm_tile.h with swapped operands,
// so an accumulator lane holds 4 consecutive columns of one row.  Pair values
// are fp16 (11-bit significand): a bf16 pair buffer costs up to 4 % of
// RMS(out) on heavy-tailed gates.
#include "prefill_kernels.h"

namespace {

template <class DT, int MODE, bool SMALL>
void (*expert_kernel_m(int pF))(PreArgs) {
  return pF == 2 ? k_pre_expert<DT, 2, MODE, SMALL>
       : pF == 4 ? k_pre_expert<DT, 4, MODE, SMALL>
       : pF == 8 ? k_pre_expert<DT, 8, MODE, SMALL> : k_pre_expert<DT, 16, MODE, SMALL>;
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
bool small_expert_tiles(const deco_moe_layer* L, int T) {
  const long long shared_tiles = (long long)((T + GM - 1) / GM) * ((L->pD + GP - 1) / GP);
  const long long expert_tiles = (long long)L->E * ((T / 4 + GM - 1) / GM);
  return 2 * (shared_tiles + expert_tiles) < (long long)L->pre_grid;
}

template <class DT>
hipError_t prefill(const deco_moe_layer* L, const void* x, int T, void* out, hipStream_t s) {
  const PreArgs a = fill_pre_args(L, x, T, out);
  using deco_host::launch;
  hipError_t err = launch_routing<DT>(L, a, T, s);
  if (err == hipSuccess)
    err = launch(deco_host::KS_PRE_EXPERT, expert_kernel<DT>(L->pF, L->gated, small_expert_tiles(L, T)),
                 dim3(L->pre_grid), dim3(256), s, a);
  if (err == hipSuccess)
    err = launch(deco_host::KS_PRE_COMBINE, k_pre_combine<DT>,
                 dim3((unsigned)(((long long)T * (L->d / 8) + 255) / 256)), dim3(256), s, a);
  if (err != hipSuccess) return err;
  return hipGetLastError();
}

}  // namespace

namespace deco_host {

hipError_t launch_prefill(const deco_moe_layer* L, const void* x, int T, void* out, hipStream_t s) {
  if (L->cfg.dtype == DECO_DT_BF16) return prefill<BF16>(L, x, T, out, s);
  return prefill<F32>(L, x, T, out, s);
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

hipError_t launch_copy_mask(const deco_moe_layer* L, int T, uint64_t* mask, hipStream_t s) {
  const int n = T * L->W;
  k_copy_mask<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(L->z, L->lam, T, L->E, L->W, mask);
  return hipGetLastError();
}

}  // namespace deco_host
