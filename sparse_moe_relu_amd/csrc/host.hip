// host.hip - the C ABI of include/deco_moe.h: validation, layer object,
// device buffers, path choice and per-kernel event timing.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <new>
#include <vector>

#include "deco_internal.h"

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int validate_cfg(const deco_moe_config* c) {
  if (!c) return DECO_ERR_INVALID_ARG;
  if (c->d_model <= 0 || c->n_experts < 1 || c->d_ff <= 0 || c->d_ff_shared <= 0 || c->max_tokens < 1)
    return DECO_ERR_INVALID_ARG;
  if (!(c->rms_eps >= 0.0f) || !isfinite(c->rms_eps)) return DECO_ERR_INVALID_ARG;
  if (c->top_k < 0 || c->top_k > c->n_experts) return DECO_ERR_INVALID_ARG;
  // the dtype field as the integer a C caller stored (a C++ load of an enum
  // outside its listed values is undefined)
  static_assert(sizeof(deco_dtype) == sizeof(int32_t), "deco_dtype is stored as a 32-bit int");
  int32_t dt = 0;
  memcpy(&dt, &c->dtype, sizeof(dt));
  if (dt != DECO_DT_BF16 && dt != DECO_DT_F32) return DECO_ERR_UNSUPPORTED;
  if (c->d_model % 64 != 0 || c->d_model > 32768) return DECO_ERR_UNSUPPORTED;
  if (c->n_experts > 256) return DECO_ERR_UNSUPPORTED;
  if (c->d_ff != 32 && c->d_ff != 64 && c->d_ff != 128 && c->d_ff != 256) return DECO_ERR_UNSUPPORTED;
  if (c->d_ff_shared % 32 != 0 || c->d_ff_shared > 16384) return DECO_ERR_UNSUPPORTED;
  if (c->max_tokens > (1 << 20)) return DECO_ERR_UNSUPPORTED;
  // every packed matrix stays below 2 GiB (32-bit buffer offsets)
  {
    const size_t esz = c->dtype == DECO_DT_BF16 ? 2 : 4;
    const size_t lim = (size_t)1 << 31;
    if ((size_t)c->d_model * c->d_ff_shared * esz >= lim || (size_t)c->d_model * c->d_ff * esz >= lim)
      return DECO_ERR_UNSUPPORTED;
  }
  if (c->backward != 0 && c->backward != 1) return DECO_ERR_INVALID_ARG;
  if (c->normsilu < 0 || c->normsilu > 3 || (c->scalar_lambda != 0 && c->scalar_lambda != 1) ||
      (c->shared_rms != 0 && c->shared_rms != 1) || (c->shared_workspace != 0 && c->shared_workspace != 1))
    return DECO_ERR_INVALID_ARG;
  if (c->backward && (c->normsilu || c->scalar_lambda || c->shared_rms)) return DECO_ERR_UNSUPPORTED;
  // one routed expert: the mean term equals its projection, h~ = 0 and every
  // routed gradient vanishes (NormSiLU divides 0 by sqrt(eps))
  if (c->backward && c->n_experts < 2) return DECO_ERR_UNSUPPORTED;
  return DECO_OK;
}

// derived sizes (no allocation)
void derive(deco_moe_layer* L) {
  const deco_moe_config& c = L->cfg;
  L->d = c.d_model;
  L->E = c.n_experts;
  L->F = c.d_ff;
  L->Fs = c.d_ff_shared;
  L->maxT = c.max_tokens;
  L->esz = c.dtype == DECO_DT_BF16 ? 2 : 4;
  L->KB = c.dtype == DECO_DT_BF16 ? 32 : 16;
  L->nkb_d = L->d / L->KB;
  L->nkb_F = L->F / L->KB;
  L->nkb_Fs = L->Fs / L->KB;
  L->pR = (L->E + 63) / 64 * 4;
  L->pF = L->F / 16;
  L->pD = L->d / 16;
  L->pFs = L->Fs / 16;
  L->W = (L->E + 63) / 64;
  L->pre_grid = 1024;
  auto r64 = [](int v) { return (v + 63) / 64 * 64; };
  L->Fp = r64(L->F);
  L->Ep = r64(L->E);
  L->Fsp = r64(L->Fs);
  L->nkb_cat = (L->Fp + L->Ep + L->Fsp) / L->KB;
}

struct Carve {
  size_t off = 0;
  size_t take(size_t bytes) {
    size_t o = off;
    off += align_up(bytes);
    return o;
  }
};

// ---- per-kernel event timing ----------------------------------------------
struct PendingPair {
  hipEvent_t a, b;
  int slot;
};
bool g_timing = false;
std::vector<hipEvent_t> g_pool;
std::vector<PendingPair> g_pending;
double g_total_ms[deco_host::KS_COUNT];
int64_t g_count[deco_host::KS_COUNT];

hipEvent_t get_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

void drain_pending() {
  for (const PendingPair& p : g_pending) {
    float ms = 0.f;
    if (hipEventSynchronize(p.b) == hipSuccess && hipEventElapsedTime(&ms, p.a, p.b) == hipSuccess) {
      g_total_ms[p.slot] += ms;
      g_count[p.slot] += 1;
    }
    g_pool.push_back(p.a);
    g_pool.push_back(p.b);
  }
  g_pending.clear();
}

// Point L's prefill/backward buffers into the workspace at `base`.
void bind_pws(deco_moe_layer* L, char* base) {
  const PwsOff& o = L->pwo;
  const bool bwd = L->cfg.backward != 0, split = bwd && L->esz == 2;
  L->pws = base;
  L->tok_off = (int*)(base + o.to);
  L->ecnt = (int*)(base + o.ec);
  L->list_tok = (int*)(base + o.lt);
  L->sbuf = base + o.sb;
  L->ybuf = base + o.yb;
  L->sraw = L->cfg.shared_rms ? (float*)(base + o.sr) : nullptr;
  L->hpart = o.hp ? (float*)(base + o.hp) : nullptr;
  if (bwd) {
    L->dgbuf = (float*)(base + o.dg);
    L->dhbuf = base + o.dh;
    L->agbuf = base + o.ag;
    L->slot_list = (int*)(base + o.sl);
    L->dcat = base + o.dc;
    L->dzbuf = (float*)(base + o.dz);
    L->dlz = (float*)(base + o.dl);
    L->gbuf = (float*)(base + o.gb);
    L->colpart = (float*)(base + o.cp);
    L->wpart = (float*)(base + o.wp);
    L->wpart2 = (float*)(base + o.wp2);
    L->sb_hi = base + o.sbh;
    if (split) {
      L->dhbuf_lo = base + o.dhl;
      L->agbuf_lo = base + o.agl;
      L->dcat_lo = base + o.dcl;
      L->sb_lo = base + o.sbl;
    }
  }
}

// One prefill/backward workspace per device for the layers that share it,
// sized for the largest.  Growing it (a larger layer loads) waits for the
// device, replaces the buffer and points every sharing layer at the new one.
struct SharedWs {
  char* p = nullptr;
  size_t bytes = 0;
  std::vector<deco_moe_layer*> users;
};
std::mutex g_ws_mu;
std::map<int, SharedWs> g_ws;

hipError_t shared_ws_acquire(deco_moe_layer* L) {
  std::lock_guard<std::mutex> lk(g_ws_mu);
  SharedWs& a = g_ws[L->device];
  if (L->pws_bytes > a.bytes) {
    hipError_t err = hipDeviceSynchronize();
    char* np = nullptr;
    if (err == hipSuccess) err = hipMalloc((void**)&np, L->pws_bytes);
    if (err != hipSuccess) return err;
    if (a.p) (void)hipFree(a.p);
    a.p = np;
    a.bytes = L->pws_bytes;
    for (deco_moe_layer* u : a.users) bind_pws(u, a.p);
  }
  a.users.push_back(L);
  bind_pws(L, a.p);
  return hipSuccess;
}

void shared_ws_release(deco_moe_layer* L) {
  std::lock_guard<std::mutex> lk(g_ws_mu);
  auto it = g_ws.find(L->device);
  if (it == g_ws.end()) return;
  SharedWs& a = it->second;
  a.users.erase(std::remove(a.users.begin(), a.users.end(), L), a.users.end());
  if (a.users.empty()) {
    if (a.p) (void)hipFree(a.p);
    g_ws.erase(it);
  }
}

}  // namespace

namespace deco_host {

const char* kernel_slot_name(int slot) {
  switch (slot) {
    case KS_PACK: return "load_pack";
    case KS_DEC_UP: return "k_dec_up";
    case KS_DEC_DOWN: return "k_dec_down";
    case KS_PRE_TOPK: return "k_pre_topk";
    case KS_PRE_ROUTER_SHARED: return "k_pre_router_shared";
    case KS_PRE_DISPATCH: return "k_pre_dispatch";
    case KS_PRE_EXPERT: return "k_pre_expert";
    case KS_PRE_COMBINE: return "k_pre_combine";
    case KS_PRE_DC: return "k_pre_dc";
    case KS_PRE_UP_PART: return "k_pre_expert_kpart";
    case KS_BWD_SHARED: return "k_bwd_shared";
    case KS_BWD_EXPERT: return "k_bwd_expert";
    case KS_BWD_TOKEN: return "k_bwd_token";
    case KS_BWD_COLSUM: return "k_bwd_colsum";
    case KS_BWD_DENSE_DX: return "k_bwd_dense_dx";
    case KS_BWD_COMBINE: return "k_bwd_combine";
    case KS_BWD_WGRAD: return "k_bwd_wgrad";
    default: return "?";
  }
}

void timing_events(int slot, hipEvent_t* start, hipEvent_t* stop) {
  *start = *stop = nullptr;
  if (!g_timing) return;
  hipEvent_t a = get_event();
  hipEvent_t b = a ? get_event() : nullptr;
  if (!a || !b) {
    if (a) g_pool.push_back(a);
    return;
  }
  *start = a;
  *stop = b;
  g_pending.push_back(PendingPair{a, b, slot});
  if (g_pending.size() > 8192) drain_pending();
}

}  // namespace deco_host

extern "C" {

int deco_moe_check_config(const deco_moe_config* cfg) { return validate_cfg(cfg); }

const char* deco_moe_status_string(int status) {
  switch (status) {
    case DECO_OK: return "ok";
    case DECO_ERR_INVALID_ARG: return "invalid argument";
    case DECO_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case DECO_ERR_OUT_OF_MEMORY: return "device out of memory";
    case DECO_ERR_HIP: return "HIP runtime or launch error";
    default: return "unknown status";
  }
}

void deco_moe_free(deco_moe_layer* L) {
  if (!L) return;
  if (L->wmem) (void)hipFree(L->wmem);
  if (L->ws) (void)hipFree(L->ws);
  if (L->pws_shared) shared_ws_release(L);
  else if (L->pws) (void)hipFree(L->pws);
  for (hipEvent_t& e : L->bwd_ev)
    if (e) (void)hipEventDestroy(e);
  for (hipStream_t& st : L->bwd_side)
    if (st) (void)hipStreamDestroy(st);
  delete L;
}

// Both loaders.  W_norm is the projection NormSiLU acts on (W_up, or W_gate
// of gated experts) and the one Wbar averages; W_lin is gated experts' W_up.
static int load_layer(const deco_moe_config* cfg, const void* W_r, const float* b_r, const float* lambda,
                      const void* W_norm, bool gated, const void* W_lin, const void* W_down,
                      const void* Ws_up, const void* Ws_down, void* stream, deco_moe_layer** out_layer) {
  if (!out_layer) return DECO_ERR_INVALID_ARG;
  *out_layer = nullptr;
  int st = validate_cfg(cfg);
  if (st != DECO_OK) return st;
  if (!W_r || !b_r || !lambda || !W_norm || !W_down || !Ws_up || !Ws_down) return DECO_ERR_INVALID_ARG;
  if (gated && !W_lin) return DECO_ERR_INVALID_ARG;
  if (gated && cfg->backward) return DECO_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;

  deco_moe_layer* L = new (std::nothrow) deco_moe_layer();
  if (!L) return DECO_ERR_OUT_OF_MEMORY;
  memset(L, 0, sizeof(*L));
  L->cfg = *cfg;
  L->gated = gated;
  derive(L);
  int n_cu = 0;
  if (hipGetDevice(&L->device) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, L->device) != hipSuccess) {
    delete L;
    return DECO_ERR_HIP;
  }
  deco_host::plan_decode_sizes(L, n_cu < 1 ? 1 : n_cu);
  const size_t KBy = 1024;
  const int E = L->E;
  // packed weights
  Carve w;
  size_t o_wr = w.take((size_t)L->pR * L->nkb_d * KBy);
  L->up_stride = (size_t)L->pF * L->nkb_d * KBy;
  L->dn_stride = (size_t)L->pD * L->nkb_F * KBy;
  size_t o_up = w.take(L->up_stride * E);
  size_t o_lin = L->gated ? w.take(L->up_stride * E) : 0;
  // the decode path's NormSiLU input with the mean term folded in,
  // W_up[e] - Wbar (not with the mean-term ablation)
  const bool fold = (L->cfg.normsilu & DECO_NORMSILU_NO_MEAN) == 0;
  size_t o_upm = fold ? w.take(L->up_stride * E) : 0;
  size_t o_wbp = w.take((size_t)L->pF * L->nkb_d * KBy);
  size_t o_dn = w.take(L->dn_stride * E);
  size_t o_dn16 = L->cfg.dtype == DECO_DT_BF16 ? w.take(L->dn_stride * E) : o_dn;
  size_t o_su = w.take((size_t)L->pFs * L->nkb_d * KBy);
  size_t o_sd = w.take((size_t)L->pD * L->nkb_Fs * KBy);
  L->dn8_stride = (size_t)(L->d / 8) * L->dec_kpe * KBy;
  size_t o_dn8 = w.take(L->dn8_stride * E);
  size_t o_sd8 = w.take((size_t)(L->d / 8) * L->dec_kps * KBy);
  size_t o_b = w.take(sizeof(float) * E);
  size_t o_l = w.take(sizeof(float) * E);
  size_t o_wb = w.take(sizeof(float) * (size_t)L->d * L->F);
  const bool bwd = L->cfg.backward != 0;
  size_t o_dnT = bwd ? w.take(L->up_stride * E) : 0;
  size_t o_upT = bwd ? w.take(L->dn_stride * E) : 0;
  size_t o_sdT = bwd ? w.take((size_t)L->pFs * L->nkb_d * KBy) : 0;
  size_t o_cat = bwd ? w.take((size_t)L->pD * L->nkb_cat * KBy) : 0;
  size_t o_wbl = (bwd && L->esz == 2) ? w.take((size_t)L->pF * L->nkb_d * KBy) : 0;
  L->wmem_bytes = w.off;
  // workspace
  const size_t Tcap = (size_t)(L->maxT < 16 ? 16 : L->maxT);
  Carve k;
  size_t o_z = k.take(sizeof(float) * Tcap * E);
  size_t o_g = k.take(sizeof(float) * Tcap * E);
  size_t o_m = k.take(sizeof(uint64_t) * Tcap * L->W);
  size_t o_mb = k.take(sizeof(float) * Tcap * L->F);
  // decode hand-offs and activations (zeroed at load: flags start clear, and
  // the activation rows' padding columns must read as zero)
  size_t o_rf = k.take(sizeof(unsigned) * E);
  size_t o_er = k.take(sizeof(unsigned));
  size_t o_a8 = k.take((size_t)16 * E);
  size_t o_hw = k.take(sizeof(uint64_t) * (size_t)L->n_hwords);
  size_t o_ct = k.take(sizeof(unsigned));   // the decode call counter
  const size_t dn_esz = L->esz == 2 ? 2 : 4;   // fp16 operands for bf16 layers
  size_t o_ar = k.take(dn_esz * (size_t)E * 16 * L->dec_Fp);
  size_t o_sr2 = k.take((size_t)L->esz * 16 * L->dec_Fsp);
  size_t o_to = k.take(sizeof(int) * (Tcap + 1));
  size_t o_ec = k.take(sizeof(int) * E);
  size_t o_lt = k.take(sizeof(int) * (size_t)E * Tcap);
  size_t o_sb = k.take((size_t)L->esz * Tcap * L->Fs);
  // pair buffer plus one scratch row that takes the stores of padding rows
  // (large batches: the pair slots' activation rows, F values of the
  // down-projection operand type, in the same memory)
  size_t o_yb = k.take(std::max((size_t)L->esz * L->d, dn_esz * L->F) * (Tcap * (E + 1) + 1));
  const size_t n_slots = Tcap * (E + 1) + 1;
  size_t o_sr = L->cfg.shared_rms ? k.take(sizeof(float) * Tcap * L->Fs) : 0;
  size_t o_dg = bwd ? k.take(sizeof(float) * Tcap * E) : 0;
  size_t o_dh = bwd ? k.take((size_t)L->esz * n_slots * L->F) : 0;
  size_t o_ag = bwd ? k.take((size_t)L->esz * n_slots * L->F) : 0;
  size_t o_sl = bwd ? k.take(sizeof(int) * (size_t)E * Tcap) : 0;
  size_t o_dc = bwd ? k.take((size_t)L->esz * Tcap * (L->Fp + L->Ep + L->Fsp)) : 0;
  size_t o_dz = bwd ? k.take(sizeof(float) * Tcap * E) : 0;
  size_t o_dl = bwd ? k.take(sizeof(float) * Tcap * E) : 0;
  size_t o_gb = bwd ? k.take(sizeof(float) * (size_t)L->d * L->F) : 0;
  size_t o_cp = bwd ? k.take(sizeof(float) * 2 * ((Tcap + 63) / 64) * E) : 0;
  size_t o_wp = bwd ? k.take(sizeof(float) * 4 * (size_t)L->d * (L->Fp + L->Ep + L->Fsp)) : 0;
  size_t o_wp2 = bwd ? k.take(sizeof(float) * 4 * (size_t)L->Fs * L->d) : 0;
  const bool split = bwd && L->esz == 2;   // low parts of the backward's bf16 operands
  size_t o_dhl = split ? k.take((size_t)L->esz * n_slots * L->F) : 0;
  size_t o_agl = split ? k.take((size_t)L->esz * n_slots * L->F) : 0;
  size_t o_dcl = split ? k.take((size_t)L->esz * Tcap * (L->Fp + L->Ep + L->Fsp)) : 0;
  size_t o_sbh = bwd ? k.take((size_t)L->esz * Tcap * L->Fs) : 0;
  size_t o_sbl = split ? k.take((size_t)L->esz * Tcap * L->Fs) : 0;
  // small-batch prefill split: fp32 k-part sums of x . W_up[e] per pair slot,
  // for batches up to split_maxT (estimated here on the grid the expert
  // kernel's occupancy gives; a larger real grid only lowers the split's use)
  L->split_maxT = deco_host::split_max_tokens(L, (long long)(n_cu < 1 ? 1 : n_cu) * (L->esz == 2 ? 2 : 1));
  size_t o_hp = L->split_maxT
                    ? k.take(sizeof(float) * deco_host::SPLIT_NKS_MAX * (size_t)L->split_maxT * (E + 1) * L->F)
                    : 0;
  // the per-layer part ends where the prefill/backward workspace starts
  L->ws_bytes = o_to;
  L->pws_bytes = k.off - o_to;
  L->pwo = PwsOff{o_to - o_to, o_ec - o_to, o_lt - o_to, o_sb - o_to, o_yb - o_to,
                  o_sr ? o_sr - o_to : 0, o_dg ? o_dg - o_to : 0, o_dh ? o_dh - o_to : 0,
                  o_ag ? o_ag - o_to : 0, o_sl ? o_sl - o_to : 0, o_dc ? o_dc - o_to : 0,
                  o_dz ? o_dz - o_to : 0, o_dl ? o_dl - o_to : 0, o_gb ? o_gb - o_to : 0,
                  o_cp ? o_cp - o_to : 0, o_wp ? o_wp - o_to : 0, o_dhl ? o_dhl - o_to : 0,
                  o_agl ? o_agl - o_to : 0, o_dcl ? o_dcl - o_to : 0, o_sbh ? o_sbh - o_to : 0,
                  o_sbl ? o_sbl - o_to : 0, o_hp ? o_hp - o_to : 0, o_wp2 ? o_wp2 - o_to : 0};

  if (hipMalloc((void**)&L->wmem, L->wmem_bytes) != hipSuccess) {
    (void)hipGetLastError();
    deco_moe_free(L);
    return DECO_ERR_OUT_OF_MEMORY;
  }
  if (hipMalloc((void**)&L->ws, L->ws_bytes) != hipSuccess) {
    (void)hipGetLastError();
    deco_moe_free(L);
    return DECO_ERR_OUT_OF_MEMORY;
  }
  if (L->cfg.shared_workspace) {
    if (shared_ws_acquire(L) != hipSuccess) {
      (void)hipGetLastError();
      deco_moe_free(L);   // not registered: frees nothing shared
      return DECO_ERR_OUT_OF_MEMORY;
    }
    L->pws_shared = 1;
  } else {
    char* p = nullptr;
    if (hipMalloc((void**)&p, L->pws_bytes) != hipSuccess) {
      (void)hipGetLastError();
      deco_moe_free(L);
      return DECO_ERR_OUT_OF_MEMORY;
    }
    bind_pws(L, p);
  }
  L->Wr_p = L->wmem + o_wr;
  L->Wup_p = L->wmem + o_up;
  L->Wlin_p = L->gated ? L->wmem + o_lin : nullptr;
  L->Wupm_p = fold ? L->wmem + o_upm : nullptr;
  L->Wbar_p = L->wmem + o_wbp;
  L->Wdn_p = L->wmem + o_dn;
  L->Wdn16_p = L->wmem + o_dn16;
  L->Wsu_p = L->wmem + o_su;
  L->Wsd_p = L->wmem + o_sd;
  L->Wdn8_p = L->wmem + o_dn8;
  L->Wsd8_p = L->wmem + o_sd8;
  L->b_r = (float*)(L->wmem + o_b);
  L->lam = (float*)(L->wmem + o_l);
  L->wbar = (float*)(L->wmem + o_wb);
  if (bwd) {
    L->WdnT_p = L->wmem + o_dnT;
    L->WupT_p = L->wmem + o_upT;
    L->WsdT_p = L->wmem + o_sdT;
    L->Bcat_p = L->wmem + o_cat;
    L->WbarLo_p = L->esz == 2 ? L->wmem + o_wbl : nullptr;
  }
  L->z = (float*)(L->ws + o_z);
  L->g = (float*)(L->ws + o_g);
  L->mask = (uint64_t*)(L->ws + o_m);
  L->mbuf = (float*)(L->ws + o_mb);
  L->rflag = (unsigned*)(L->ws + o_rf);
  L->dec_err = (unsigned*)(L->ws + o_er);
  L->act8 = (unsigned char*)(L->ws + o_a8);
  L->hwords = L->ws + o_hw;
  L->dec_ctr = (unsigned*)(L->ws + o_ct);
  L->arow = L->ws + o_ar;
  L->srow = L->ws + o_sr2;

  hipError_t err = hipSuccess;
  // counters, flags and activation fragments start at zero; the rest of the
  // workspace is always written before it is read
  size_t zero_end = o_to;
  err = hipMemsetAsync(L->ws, 0, zero_end, s);
  if (err == hipSuccess) err = hipMemcpyAsync(L->b_r, b_r, sizeof(float) * E, hipMemcpyDeviceToDevice, s);
  if (err == hipSuccess) {
    if (L->cfg.scalar_lambda)   // ablation: lambda[0] for every expert
      for (int e = 0; e < E && err == hipSuccess; ++e)
        err = hipMemcpyAsync(L->lam + e, lambda, sizeof(float), hipMemcpyDeviceToDevice, s);
    else
      err = hipMemcpyAsync(L->lam, lambda, sizeof(float) * E, hipMemcpyDeviceToDevice, s);
  }
  bool down_ok = true;
  if (err == hipSuccess) err = deco_host::check_down_range(L, W_down, W_norm, s, &down_ok);
  if (err == hipSuccess && !down_ok) {
    // bf16 layers run the down-projection and the decode path's folded
    // NormSiLU input on fp16 operands: an entry past their range is refused
    // rather than turned into inf
    deco_moe_free(L);
    return DECO_ERR_UNSUPPORTED;
  }
  if (err == hipSuccess) err = deco_host::launch_pack_all(L, W_r, W_norm, W_lin, W_down, Ws_up, Ws_down, s);
  if (err == hipSuccess) err = deco_host::plan_prefill(L);   // also reads the CU count
  if (err == hipSuccess) err = deco_host::plan_decode(L);
  if (err == hipSuccess && bwd) err = deco_host::plan_backward(L);
  if (err == hipSuccess) err = hipStreamSynchronize(s);
  if (err != hipSuccess) {
    (void)hipGetLastError();
    deco_moe_free(L);
    return DECO_ERR_HIP;
  }
  *out_layer = L;
  return DECO_OK;
}

int deco_moe_load_weights(const deco_moe_config* cfg, const void* W_r, const float* b_r,
                          const float* lambda, const void* W_up, const void* W_down, const void* Ws_up,
                          const void* Ws_down, void* stream, deco_moe_layer** out_layer) {
  return load_layer(cfg, W_r, b_r, lambda, W_up, false, nullptr, W_down, Ws_up, Ws_down, stream, out_layer);
}

int deco_moe_load_weights_gated(const deco_moe_config* cfg, const void* W_r, const float* b_r,
                                const float* lambda, const void* W_gate, const void* W_up,
                                const void* W_down, const void* Ws_up, const void* Ws_down, void* stream,
                                deco_moe_layer** out_layer) {
  return load_layer(cfg, W_r, b_r, lambda, W_gate, true, W_up, W_down, Ws_up, Ws_down, stream, out_layer);
}

int deco_moe_forward_path(const deco_moe_layer* L, const void* x, int64_t T, void* out, void* stream,
                          int path) {
  if (!L || T < 0 || T > L->maxT) return DECO_ERR_INVALID_ARG;
  if (path < DECO_PATH_AUTO || path > DECO_PATH_PREFILL_FUSED) return DECO_ERR_INVALID_ARG;
  if (path == DECO_PATH_PREFILL_TOKEN && !deco_host::prefill_token_ok(L)) return DECO_ERR_UNSUPPORTED;
  if (T == 0) return DECO_OK;
  if (!x || !out) return DECO_ERR_INVALID_ARG;
  if (((uintptr_t)x % 16) != 0 || ((uintptr_t)out % 16) != 0) return DECO_ERR_INVALID_ARG;
  const size_t bytes = (size_t)T * L->d * L->esz;
  const char* xb = (const char*)x;
  const char* ob = (const char*)out;
  if (xb < ob + bytes && ob < xb + bytes) return DECO_ERR_INVALID_ARG;   // x and out overlap
  if (path == DECO_PATH_AUTO)
    path = (T <= DECO_DECODE_MAX_T && L->dec_ok) ? DECO_PATH_DECODE : DECO_PATH_PREFILL;
  if (path == DECO_PATH_DECODE && T > DECO_DECODE_MAX_T) return DECO_ERR_INVALID_ARG;
  if (path == DECO_PATH_DECODE && !L->dec_ok) return DECO_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  hipError_t err = path == DECO_PATH_DECODE ? deco_host::launch_decode(L, x, (int)T, out, s)
                                            : deco_host::launch_prefill(L, x, (int)T, out, s, path);
  // which path's routing state deco_moe_copy_routing returns
  const_cast<deco_moe_layer*>(L)->last_path = path;
  return err == hipSuccess ? DECO_OK : DECO_ERR_HIP;
}

int deco_moe_forward(const deco_moe_layer* L, const void* x, int64_t T, void* out, void* stream) {
  return deco_moe_forward_path(L, x, T, out, stream, DECO_PATH_AUTO);
}

int deco_moe_forward_decode_noalloc(const deco_moe_layer* L, const void* x, int64_t T, void* out, void* stream) {
  if (!L || T < 0 || T > L->maxT || T > DECO_DECODE_MAX_T) return DECO_ERR_INVALID_ARG;
  if (T == 0) return DECO_OK;
  if (!x || !out) return DECO_ERR_INVALID_ARG;
  if (((uintptr_t)x % 16) != 0 || ((uintptr_t)out % 16) != 0) return DECO_ERR_INVALID_ARG;
  const size_t bytes = (size_t)T * L->d * L->esz;
  const char* xb = (const char*)x;
  const char* ob = (const char*)out;
  if (xb < ob + bytes && ob < xb + bytes) return DECO_ERR_INVALID_ARG;
  if (!L->dec_ok) return DECO_ERR_UNSUPPORTED;
  if (deco_host::decode_scratch_bytes(L) > deco_host::decode_scratch_limit()) return DECO_ERR_UNSUPPORTED;
  const hipError_t err = deco_host::launch_decode_scratch(L, x, (int)T, out, (hipStream_t)stream);
  return err == hipSuccess ? DECO_OK : DECO_ERR_HIP;
}

int64_t deco_moe_decode_noalloc_bytes(const deco_moe_layer* L) {
  if (!L) return DECO_ERR_INVALID_ARG;
  return (int64_t)deco_host::decode_scratch_bytes(L);
}

int deco_moe_copy_routing(const deco_moe_layer* L, int64_t T, uint64_t* mask, float* logits, void* stream) {
  if (!L || T < 0 || T > L->maxT || !mask) return DECO_ERR_INVALID_ARG;
  if (T == 0) return DECO_OK;
  hipStream_t s = (hipStream_t)stream;
  // the decisions the kernels of the last call used: the decode up kernel's
  // per-expert decisions (packed into words here), or the mask words the
  // prefill dispatch read
  hipError_t err = L->last_path == DECO_PATH_DECODE
      ? deco_host::launch_dec_mask(L, (int)T, mask, s)
      : hipMemcpyAsync(mask, L->mask, sizeof(uint64_t) * (size_t)T * L->W, hipMemcpyDeviceToDevice, s);
  if (err == hipSuccess && logits)
    err = hipMemcpyAsync(logits, L->z, sizeof(float) * (size_t)T * L->E, hipMemcpyDeviceToDevice, s);
  return err == hipSuccess ? DECO_OK : DECO_ERR_HIP;
}

int deco_moe_copy_mean_up(const deco_moe_layer* L, float* wbar, void* stream) {
  if (!L || !wbar) return DECO_ERR_INVALID_ARG;
  hipError_t err = hipMemcpyAsync(wbar, L->wbar, sizeof(float) * (size_t)L->d * L->F, hipMemcpyDeviceToDevice,
                                  (hipStream_t)stream);
  return err == hipSuccess ? DECO_OK : DECO_ERR_HIP;
}

int deco_moe_backward(const deco_moe_layer* L, const void* x, const void* dout, int64_t T, float reg_coef,
                      const deco_moe_grads* gr, void* stream) {
  if (!L || !x || !dout || !gr || T < 1 || T > L->maxT) return DECO_ERR_INVALID_ARG;
  if (!gr->dx || !gr->dW_r || !gr->db_r || !gr->dlambda || !gr->dW_up || !gr->dW_down || !gr->dWs_up ||
      !gr->dWs_down)
    return DECO_ERR_INVALID_ARG;
  if (!isfinite(reg_coef) || (L->cfg.top_k > 0 && reg_coef != 0.0f)) return DECO_ERR_INVALID_ARG;
  if (!L->cfg.backward || L->gated) return DECO_ERR_UNSUPPORTED;
  if (((uintptr_t)x % 16) != 0 || ((uintptr_t)dout % 16) != 0 || ((uintptr_t)gr->dx % 16) != 0)
    return DECO_ERR_INVALID_ARG;
  hipError_t err = deco_host::launch_backward(L, x, dout, (int)T, reg_coef, gr, (hipStream_t)stream);
  return err == hipSuccess ? DECO_OK : DECO_ERR_HIP;
}

float deco_moe_sparsity_coef_update(float coef, float active_ratio, float target_ratio, float factor) {
  if (active_ratio > target_ratio) return coef * factor;
  if (active_ratio < target_ratio) return coef / factor;
  return coef;
}

int deco_moe_read_error_flags(const deco_moe_layer* L, uint32_t* flags) {
  if (!L || !flags) return DECO_ERR_INVALID_ARG;
  unsigned v = 0;
  hipError_t err = hipDeviceSynchronize();
  if (err == hipSuccess) err = hipMemcpy(&v, L->dec_err, sizeof(v), hipMemcpyDeviceToHost);
  if (err == hipSuccess && v) err = hipMemset(L->dec_err, 0, sizeof(v));
  *flags = v;
  return err == hipSuccess ? DECO_OK : DECO_ERR_HIP;
}

int deco_moe_timing_enable(int enable) {
  g_timing = enable != 0;
  return DECO_OK;
}

int deco_moe_timing_reset(void) {
  drain_pending();
  for (int i = 0; i < deco_host::KS_COUNT; ++i) {
    g_total_ms[i] = 0.0;
    g_count[i] = 0;
  }
  return DECO_OK;
}

int deco_moe_timing_read(int idx, const char** name, double* total_ms, int64_t* launches) {
  if (idx < 0 || idx >= deco_host::KS_COUNT) return DECO_ERR_INVALID_ARG;
  drain_pending();
  if (name) *name = deco_host::kernel_slot_name(idx);
  if (total_ms) *total_ms = g_total_ms[idx];
  if (launches) *launches = g_count[idx];
  return DECO_OK;
}

}  // extern "C"
