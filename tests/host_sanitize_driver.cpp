// Host-side checks of the C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code (tests/test_host_sanitize.py).
// Every call here must be rejected, or answered, before any HIP call: the
// program runs without a GPU.  Exit status 0 when every expectation holds.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "deco_moe.h"

static int g_fail = 0;

static void expect(int got, int want, const char* what) {
  if (got != want) {
    fprintf(stderr, "FAIL %s: got %d, want %d\n", what, got, want);
    ++g_fail;
  }
}

static deco_moe_config base_cfg(void) {
  deco_moe_config c;
  memset(&c, 0, sizeof(c));
  c.d_model = 2048;
  c.n_experts = 56;
  c.d_ff = 128;
  c.d_ff_shared = 1024;
  c.max_tokens = 4096;
  c.dtype = DECO_DT_BF16;
  c.rms_eps = 1e-6f;
  return c;
}

int main(void) {
  // configurations of the five synthetic workloads, and the edges of the
  // supported set, are accepted
  {
    deco_moe_config c = base_cfg();
    expect(deco_moe_check_config(&c), DECO_OK, "c2/c3 layer");
    c.d_model = 64; c.n_experts = 8; c.d_ff = 32; c.d_ff_shared = 64; c.max_tokens = 16; c.dtype = DECO_DT_F32;
    expect(deco_moe_check_config(&c), DECO_OK, "c1 layer");
    c = base_cfg();
    c.d_model = 4096; c.n_experts = 112; c.d_ff_shared = 2048;
    expect(deco_moe_check_config(&c), DECO_OK, "c4 layer");
    c = base_cfg();
    c.n_experts = 256; c.d_ff = 256; c.d_ff_shared = 16384; c.d_model = 32768; c.max_tokens = 1 << 20;
    expect(deco_moe_check_config(&c), DECO_OK, "largest shapes");
    c = base_cfg();
    c.top_k = c.n_experts;
    expect(deco_moe_check_config(&c), DECO_OK, "top_k = E");
    c = base_cfg();
    c.backward = 1;
    expect(deco_moe_check_config(&c), DECO_OK, "backward");
  }
  // rejected configurations
  {
    expect(deco_moe_check_config(NULL), DECO_ERR_INVALID_ARG, "null config");
    struct Case { void (*edit)(deco_moe_config*); int want; const char* what; };
    static const Case cases[] = {
        {[](deco_moe_config* c) { c->d_model = 0; }, DECO_ERR_INVALID_ARG, "d = 0"},
        {[](deco_moe_config* c) { c->d_model = -64; }, DECO_ERR_INVALID_ARG, "d < 0"},
        {[](deco_moe_config* c) { c->d_model = 96; }, DECO_ERR_UNSUPPORTED, "d not a multiple of 64"},
        {[](deco_moe_config* c) { c->d_model = 32768 + 64; }, DECO_ERR_UNSUPPORTED, "d too large"},
        {[](deco_moe_config* c) { c->n_experts = 0; }, DECO_ERR_INVALID_ARG, "E = 0"},
        {[](deco_moe_config* c) { c->n_experts = 257; }, DECO_ERR_UNSUPPORTED, "E > 256"},
        {[](deco_moe_config* c) { c->d_ff = 0; }, DECO_ERR_INVALID_ARG, "F = 0"},
        {[](deco_moe_config* c) { c->d_ff = 48; }, DECO_ERR_UNSUPPORTED, "F = 48"},
        {[](deco_moe_config* c) { c->d_ff = 512; }, DECO_ERR_UNSUPPORTED, "F = 512"},
        {[](deco_moe_config* c) { c->d_ff_shared = 0; }, DECO_ERR_INVALID_ARG, "Fs = 0"},
        {[](deco_moe_config* c) { c->d_ff_shared = 48; }, DECO_ERR_UNSUPPORTED, "Fs not a multiple of 32"},
        {[](deco_moe_config* c) { c->d_ff_shared = 16384 + 32; }, DECO_ERR_UNSUPPORTED, "Fs too large"},
        {[](deco_moe_config* c) { c->max_tokens = 0; }, DECO_ERR_INVALID_ARG, "max_tokens = 0"},
        {[](deco_moe_config* c) { c->max_tokens = (1 << 20) + 1; }, DECO_ERR_UNSUPPORTED, "max_tokens too large"},
        {[](deco_moe_config* c) { c->rms_eps = -1e-6f; }, DECO_ERR_INVALID_ARG, "eps < 0"},
        {[](deco_moe_config* c) { c->rms_eps = NAN; }, DECO_ERR_INVALID_ARG, "eps NaN"},
        {[](deco_moe_config* c) { c->rms_eps = INFINITY; }, DECO_ERR_INVALID_ARG, "eps inf"},
        {[](deco_moe_config* c) { c->top_k = -1; }, DECO_ERR_INVALID_ARG, "top_k < 0"},
        {[](deco_moe_config* c) { c->top_k = 57; }, DECO_ERR_INVALID_ARG, "top_k > E"},
        {[](deco_moe_config* c) { c->dtype = (deco_dtype)7; }, DECO_ERR_UNSUPPORTED, "dtype"},
        {[](deco_moe_config* c) { c->backward = 2; }, DECO_ERR_INVALID_ARG, "backward flag"},
        {[](deco_moe_config* c) { c->normsilu = 4; }, DECO_ERR_INVALID_ARG, "normsilu flag"},
        {[](deco_moe_config* c) { c->scalar_lambda = 2; }, DECO_ERR_INVALID_ARG, "scalar_lambda flag"},
        {[](deco_moe_config* c) { c->shared_rms = -1; }, DECO_ERR_INVALID_ARG, "shared_rms flag"},
        {[](deco_moe_config* c) { c->shared_workspace = 3; }, DECO_ERR_INVALID_ARG, "shared_workspace flag"},
        {[](deco_moe_config* c) { c->backward = 1; c->normsilu = 1; }, DECO_ERR_UNSUPPORTED, "backward + ablation"},
        {[](deco_moe_config* c) { c->backward = 1; c->n_experts = 1; }, DECO_ERR_UNSUPPORTED, "backward, E = 1"},
        // a packed matrix of 2 GiB or more (32-bit buffer offsets)
        {[](deco_moe_config* c) { c->dtype = DECO_DT_F32; c->d_model = 32768; c->d_ff_shared = 16384; },
         DECO_ERR_UNSUPPORTED, "2 GiB shared matrix"},
    };
    for (const Case& k : cases) {
      deco_moe_config c = base_cfg();
      k.edit(&c);
      expect(deco_moe_check_config(&c), k.want, k.what);
    }
  }
  // every status code has a message
  for (int s = -8; s <= 4; ++s) {
    const char* m = deco_moe_status_string(s);
    if (!m || !m[0]) {
      fprintf(stderr, "FAIL status_string(%d)\n", s);
      ++g_fail;
    }
  }
  // load: argument checks come before any allocation or HIP call
  {
    deco_moe_config c = base_cfg();
    char dummy[64];
    const void* p = dummy;
    const float* pf = (const float*)dummy;
    deco_moe_layer* L = (deco_moe_layer*)dummy;
    expect(deco_moe_load_weights(&c, p, pf, pf, p, p, p, p, NULL, NULL), DECO_ERR_INVALID_ARG, "load: null out");
    expect(deco_moe_load_weights(NULL, p, pf, pf, p, p, p, p, NULL, &L), DECO_ERR_INVALID_ARG, "load: null cfg");
    expect(deco_moe_load_weights(&c, NULL, pf, pf, p, p, p, p, NULL, &L), DECO_ERR_INVALID_ARG, "load: null W_r");
    expect(deco_moe_load_weights(&c, p, NULL, pf, p, p, p, p, NULL, &L), DECO_ERR_INVALID_ARG, "load: null b_r");
    expect(deco_moe_load_weights(&c, p, pf, NULL, p, p, p, p, NULL, &L), DECO_ERR_INVALID_ARG, "load: null lambda");
    expect(deco_moe_load_weights(&c, p, pf, pf, NULL, p, p, p, NULL, &L), DECO_ERR_INVALID_ARG, "load: null W_up");
    expect(deco_moe_load_weights(&c, p, pf, pf, p, NULL, p, p, NULL, &L), DECO_ERR_INVALID_ARG, "load: null W_down");
    expect(deco_moe_load_weights(&c, p, pf, pf, p, p, NULL, p, NULL, &L), DECO_ERR_INVALID_ARG, "load: null Ws_up");
    expect(deco_moe_load_weights(&c, p, pf, pf, p, p, p, NULL, NULL, &L), DECO_ERR_INVALID_ARG, "load: null Ws_down");
    expect(deco_moe_load_weights_gated(&c, p, pf, pf, p, NULL, p, p, p, NULL, &L), DECO_ERR_INVALID_ARG,
           "load gated: null W_up");
    c.d_ff = 48;
    expect(deco_moe_load_weights(&c, p, pf, pf, p, p, p, p, NULL, &L), DECO_ERR_UNSUPPORTED, "load: bad shape");
    c = base_cfg();
    c.backward = 1;
    expect(deco_moe_load_weights_gated(&c, p, pf, pf, p, p, p, p, p, NULL, &L), DECO_ERR_UNSUPPORTED,
           "load gated with backward");
  }
  // calls on a null layer
  {
    char buf[64];
    uint64_t mask[4];
    float f[4];
    uint32_t flags = 0;
    expect(deco_moe_forward(NULL, buf, 1, buf, NULL), DECO_ERR_INVALID_ARG, "forward: null layer");
    expect(deco_moe_forward_path(NULL, buf, 1, buf, NULL, DECO_PATH_DECODE), DECO_ERR_INVALID_ARG,
           "forward_path: null layer");
    expect(deco_moe_forward_decode_noalloc(NULL, buf, 1, buf, NULL), DECO_ERR_INVALID_ARG,
           "noalloc: null layer");
    expect(deco_moe_copy_routing(NULL, 1, mask, f, NULL), DECO_ERR_INVALID_ARG, "copy_routing: null layer");
    expect(deco_moe_copy_mean_up(NULL, f, NULL), DECO_ERR_INVALID_ARG, "copy_mean_up: null layer");
    expect(deco_moe_read_error_flags(NULL, &flags), DECO_ERR_INVALID_ARG, "read_error_flags: null layer");
    if (deco_moe_decode_noalloc_bytes(NULL) >= 0) {
      fprintf(stderr, "FAIL decode_noalloc_bytes(NULL) >= 0\n");
      ++g_fail;
    }
    deco_moe_free(NULL);   // a no-op
  }
  if (g_fail) {
    fprintf(stderr, "%d expectation(s) failed\n", g_fail);
    return 1;
  }
  printf("host checks passed\n");
  return 0;
}
