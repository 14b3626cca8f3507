/*
 * deco_moe.h - C ABI of the MI355X (gfx950) DECO sparse-MoE feed-forward layer.
 *
 * The layer (forward pass only), in the notation of the DECO paper
 * ("DECO: Sparse Mixture-of-Experts with Dense-Comparable Performance on
 * End-Side Devices", Sec. 1 Introduction and Sec. 2 Related work, paragraphs
 * "Router design" and "Expert design"; and the Chinese write-up of the same
 * paper on qidianchuan.cn, section 二, router and expert-design parts):
 *
 *   z      = x W_r + b_r                          router logits       [T, E]
 *   g      = lambda_e * max(z, 0)                 gates (ReLU routing with a
 *                                                 learned per-expert scale)
 *   active = (z > 0) and (lambda_e != 0)          variable experts per token
 *   Wbar   = (1/E) sum_e W_up[e]                  inter-expert mean, fixed at load
 *   for each active (t, e):
 *     h~   = x_t W_up[e] - x_t Wbar               NormSiLU step 1 (mean term)
 *     r    = sqrt(mean_f h~_f^2 + eps)            NormSiLU step 2 (RMS inside
 *     a    = SiLU(h~ / r)                         the expert), then SiLU
 *     out_t += g_te * a W_down[e]                 non-gated expert, weighted sum
 *   out_t += SiLU(x_t Ws_up) Ws_down               always-on shared expert
 *
 * Memory: every pointer argument of the compute calls is DEVICE memory,
 * row-major and contiguous, owned by the caller; `stream` is a hipStream_t
 * passed as void* (NULL = the default stream).  Weights and activations share
 * one element type (`dtype`); b_r and lambda are always float32.
 *
 * Errors: every call returns a deco_status (0 = OK, negative = error) and
 * launches nothing when it fails validation; output buffers are then left
 * untouched.  No C++ exception crosses this interface.  Non-finite inputs are
 * not detected.  A layer may be used by one stream at a time: calls that
 * overlap on one layer race on its workspace.
 */
#ifndef DECO_MOE_H
#define DECO_MOE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct deco_moe_layer deco_moe_layer;   /* opaque, owns all its device buffers */

typedef enum {
  DECO_OK = 0,
  DECO_ERR_INVALID_ARG = -1,     /* null pointer, T < 0, T > max_tokens, E < 1, ... */
  DECO_ERR_UNSUPPORTED = -2,     /* shape or dtype outside the supported set      */
  DECO_ERR_OUT_OF_MEMORY = -3,   /* device allocation failed                      */
  DECO_ERR_HIP = -4              /* a HIP runtime call or a launch failed         */
} deco_status;

typedef enum { DECO_DT_BF16 = 0, DECO_DT_F32 = 1 } deco_dtype;

typedef enum {
  DECO_PATH_AUTO = 0,     /* decode path for T <= DECO_DECODE_MAX_T, else prefill   */
  DECO_PATH_DECODE = 1,   /* weight-streaming path; requires T <= DECO_DECODE_MAX_T */
  DECO_PATH_PREFILL = 2,  /* bucketed grouped-MFMA path; any T (the _PAIRS variant) */
  DECO_PATH_PREFILL_PAIRS = 3,  /* prefill, expert-major down-projection into per-pair
                                 * output rows, then a combine kernel; any layer     */
  DECO_PATH_PREFILL_TOKEN = 4,  /* prefill, token-major down-projection and combine in
                                 * one kernel (no per-pair rows); slower than _PAIRS
                                 * on the measured layers; d_ff / k-block <= 4 (bf16:
                                 * d_ff <= 128, fp32: d_ff <= 64), else
                                 * DECO_ERR_UNSUPPORTED                              */
  DECO_PATH_PREFILL_FUSED = 5   /* prefill as _PAIRS, with the combine fused with the
                                 * shared expert's down-projection (one kernel forms
                                 * the shared term on MFMA and adds the pair rows);
                                 * slower than _PAIRS on the measured layers; any
                                 * layer                                             */
} deco_path;

#define DECO_DECODE_MAX_T 16

typedef struct {
  int32_t d_model;      /* d  : multiple of 64                                  */
  int32_t n_experts;    /* E  : 1 .. 256 routed experts                         */
  int32_t d_ff;         /* F  : routed expert width, one of 32, 64, 128, 256    */
  int32_t d_ff_shared;  /* Fs : shared expert width, multiple of 32, 32..16384  */
  int32_t max_tokens;   /* largest T passed to deco_moe_forward (>= 1)          */
  deco_dtype dtype;     /* element type of x, out and all weight matrices       */
  float rms_eps;        /* epsilon inside the NormSiLU RMS (e.g. 1e-6), >= 0    */
  int32_t top_k;        /* 0: DECO's ReLU routing (above).  1..E: the TopK      */
                        /* routing variant, the baseline of the DECO paper's    */
                        /* Sec. 4 acceleration experiment (Table 4): each token */
                        /* keeps the top_k largest logits z (ties to the lower  */
                        /* expert index), gates = softmax of the kept logits,   */
                        /* lambda unused; experts and shared expert unchanged.  */
  int32_t backward;     /* 0: inference only.  1: also keep the transposed      */
                        /* weight copies and the workspace deco_moe_backward    */
                        /* needs (non-gated experts, n_experts >= 2)            */
  /* Ablation switches (the qidianchuan.cn write-up, section 二, reports the   */
  /* NormSiLU steps removed one at a time and a scalar router scale in place   */
  /* of the per-expert one).  All 0 is the DECO layer; backward needs all 0.   */
  int32_t normsilu;     /* bit DECO_NORMSILU_NO_MEAN: no mean term (step 1);    */
                        /* bit DECO_NORMSILU_NO_RMS: no RMS step (r = 1); both: */
                        /* vanilla SiLU experts                                 */
  int32_t scalar_lambda;/* 1: lambda[0] scales every expert                     */
  int32_t shared_rms;   /* 1: the shared expert's SiLU input is divided by its  */
                        /* RMS over the Fs entries (eps inside the root)        */
  int32_t shared_workspace; /* 0: the layer owns its prefill/backward workspace. */
                        /* 1: one workspace per device, shared by every layer   */
                        /* loaded with 1 and sized for the largest of them; the */
                        /* prefill and backward calls of those layers must not  */
                        /* overlap on the device (run them on one stream).  The */
                        /* decode path's state stays per layer either way.      */
} deco_moe_config;

#define DECO_NORMSILU_NO_MEAN 1
#define DECO_NORMSILU_NO_RMS 2

/* Check a configuration without touching the GPU.  Returns DECO_OK,
 * DECO_ERR_INVALID_ARG (null, non-positive sizes, negative eps, top_k outside
 * 0..n_experts, a flag outside its range) or DECO_ERR_UNSUPPORTED (shape
 * outside the set documented in the struct, or backward = 1 with an ablation
 * switch on or a single routed expert). */
int deco_moe_check_config(const deco_moe_config* cfg);

/* Copy, pack and preprocess one layer's weights into library-owned device
 * buffers, and size the layer's workspace for cfg->max_tokens tokens.
 *   W_r     [d, E]      dtype     router projection
 *   b_r     [E]         float32   router bias
 *   lambda  [E]         float32   expert-wise router scaling
 *   W_up    [E, d, F]   dtype     routed up-projections
 *   W_down  [E, F, d]   dtype     routed down-projections
 *   Ws_up   [d, Fs]     dtype     shared-expert up-projection
 *   Ws_down [Fs, d]     dtype     shared-expert down-projection
 * Computes Wbar = mean over all E routed experts of W_up (the NormSiLU mean
 * term is precomputable because inference weights are fixed: qidianchuan.cn
 * write-up, section 二, expert design) in fp32 and packs it, in the layer
 * dtype, next to the experts' weights; the prefill path forms x.Wbar once per
 * token and subtracts it from every expert's up-projection.  The decode path
 * multiplies x by W_up[e] - Wbar instead, packed once more at load (the
 * difference in fp32, rounded once to fp16 for bf16 layers, fp32 for fp32
 * layers; not with the mean-term ablation).  Runs on
 * `stream` and synchronizes it
 * before returning, so the sources may be freed afterwards.  On success
 * *out_layer receives the new layer; on failure it is set to NULL and nothing
 * stays allocated.  bf16 layers run the routed down-projection on fp16
 * operands (W_down and the gated activations; the paths' fp32 accumulation
 * is unchanged): a W_down entry whose magnitude exceeds the fp16 range
 * (65504), or a NaN, gets DECO_ERR_UNSUPPORTED, and so does, with the mean
 * term, a W_up entry (the NormSiLU input) beyond 32752, half the fp16 range
 * (|W_up - Wbar| <= 2 max |W_up|).  Activations or pair rows that leave the
 * fp16 range at run time (very large gates), or an x value beyond it on the
 * decode path (x enters the folded product converted to fp16), set error
 * bit 5 (see deco_moe_read_error_flags). */
/* Device memory of a layer, besides its packed weights: a per-layer part of
 * about max(16, max_tokens) x (8E + 4F) bytes plus the decode path's
 * hand-off state (under 1 MB at the sizes here), and the prefill/backward
 * workspace, dominated by the token-major pair buffer of
 * (max_tokens (E + 1) + 1) x d values of 2 bytes (bf16 layers; 4 for fp32):
 * every token can activate every expert, so that is the bound the buffer is
 * sized for (956 MB for d = 2048, E = 56, max_tokens = 4096).  Non-gated
 * layers add 16 F (E + 1) bytes per token of the largest batch whose prefill
 * splits its expert tiles (fp32 partial sums; at most a few hundred tokens on
 * a 256-CU device: about 60 MB at d = 2048 and at d = 4096).  With
 * cfg.shared_workspace = 1 one such workspace serves every sharing layer on
 * the device (its size is the largest layer's), instead of one per layer. */
int deco_moe_load_weights(const deco_moe_config* cfg,
                          const void* W_r, const float* b_r, const float* lambda,
                          const void* W_up, const void* W_down,
                          const void* Ws_up, const void* Ws_down,
                          void* stream, deco_moe_layer** out_layer);

/* The gated-expert variant ("DECO (gated)" in the DECO paper's Sec. 2
 * "Expert design" comparison, which the paper sets against its non-gated
 * experts; the qidianchuan.cn write-up, section 二, describes gated MLPs as
 * carrying an extra multiplicative interaction).  Each routed expert has a
 * gate projection next to its up-projection, and NormSiLU acts on the gate
 * projection:
 *   Wbar    = (1/E) sum_e W_gate[e]               mean term from the gates
 *   h~      = x_t W_gate[e] - x_t Wbar,  r = sqrt(mean_f h~_f^2 + eps)
 *   out_t  += g_te * (SiLU(h~ / r) * (x_t W_up[e])) W_down[e]
 * Router, routing variants and shared expert are as in deco_moe_load_weights.
 *   W_gate  [E, d, F]   dtype     routed gate projections (NormSiLU input)
 *   W_up    [E, d, F]   dtype     routed up-projections (multiplied in)
 * Every other argument, the ownership and the error behaviour are those of
 * deco_moe_load_weights; deco_moe_copy_mean_up returns the mean of W_gate.
 * The forward calls below take either kind of layer. */
int deco_moe_load_weights_gated(const deco_moe_config* cfg,
                                const void* W_r, const float* b_r, const float* lambda,
                                const void* W_gate, const void* W_up, const void* W_down,
                                const void* Ws_up, const void* Ws_down,
                                void* stream, deco_moe_layer** out_layer);

/* One forward pass: out [T, d] = DECO layer(x [T, d]), both of the layer's
 * dtype, on device.  x and out must not overlap.  Asynchronous on `stream`;
 * allocates nothing and never waits on the host.  T == 0 returns DECO_OK and
 * launches nothing.  Same as deco_moe_forward_path(..., DECO_PATH_AUTO). */
int deco_moe_forward(const deco_moe_layer* L, const void* x, int64_t T, void* out, void* stream);

/* As deco_moe_forward, with the kernel family chosen explicitly (all give
 * the same result up to rounding and fp32 summation order).  DECO_PATH_DECODE
 * with T > DECO_DECODE_MAX_T returns DECO_ERR_INVALID_ARG; an unknown path
 * DECO_ERR_INVALID_ARG. */
int deco_moe_forward_path(const deco_moe_layer* L, const void* x, int64_t T, void* out,
                          void* stream, int path);

/* Allocation-free decode, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same result as deco_moe_forward_path(..., DECO_PATH_DECODE),
 * bit for bit (same kernels), with the scratch those kernels hand to each
 * other (hand-off words, epoch counters, routing flags, decisions, logits and
 * gates, activation rows: deco_moe_decode_noalloc_bytes(L) bytes) in one
 * static device array of 4 MiB per device instead of L's workspace.
 * Allocates nothing; asynchronous on `stream`.  T in 0..min(max_tokens,
 * DECO_DECODE_MAX_T), else DECO_ERR_INVALID_ARG; DECO_ERR_UNSUPPORTED when
 * the layer's scratch exceeds 4 MiB or its decode path is unavailable.  The
 * array is cleared at the start of every call and keeps the last call's
 * contents; all calls on one device share that device's array, so calls that
 * overlap on a device (another stream, another thread) race.  L's routing
 * state is left as it was (deco_moe_copy_routing describes the last regular
 * forward); timeouts still set L's error flags. */
int deco_moe_forward_decode_noalloc(const deco_moe_layer* L, const void* x, int64_t T, void* out,
                                    void* stream);

/* Scratch bytes deco_moe_forward_decode_noalloc needs for L (at most 4 MiB
 * is accepted); DECO_ERR_INVALID_ARG for NULL. */
int64_t deco_moe_decode_noalloc_bytes(const deco_moe_layer* L);

/* Routing state of the most recent forward on L, for the same T:
 *   mask   [T, ceil(E/64)] uint64 (device): bit e%64 of word e/64 of row t is
 *          set iff expert e was active for token t (z > 0 and lambda_e != 0;
 *          with top_k > 0: e among the token's top_k logits);
 *   logits [T, E] float32 (device, may be NULL): router logits z as computed
 *          on the GPU (fp32 accumulation of the dtype products, plus b_r).
 * T must equal the T of that forward (not checked beyond 0 <= T <= max). */
int deco_moe_copy_routing(const deco_moe_layer* L, int64_t T, uint64_t* mask, float* logits,
                          void* stream);

/* Copy the inter-expert mean Wbar [d, F] (float32, device) built at load
 * (of W_up, or of W_gate for a gated layer). */
int deco_moe_copy_mean_up(const deco_moe_layer* L, float* wbar, void* stream);

/* Gradients written by deco_moe_backward: float32 device buffers owned by
 * the caller, row-major, shaped like the weights (every one is overwritten,
 * none is accumulated into).  n_active_pairs may be NULL. */
typedef struct {
  float* dx;              /* [T, d]      */
  float* dW_r;            /* [d, E]      */
  float* db_r;            /* [E]         */
  float* dlambda;         /* [E]         */
  float* dW_up;           /* [E, d, F]   */
  float* dW_down;         /* [E, F, d]   */
  float* dWs_up;          /* [d, Fs]     */
  float* dWs_down;        /* [Fs, d]     */
  int32_t* n_active_pairs;/* [1] active (token, expert) pairs of the call    */
} deco_moe_grads;

/* Backward pass of the layer (the training side of the DECO paper: Sec. 2
 * "Router design", "Expert design" and "Auxiliary training objective";
 * qidianchuan.cn write-up, sections 二 and 三).  Gradients, with respect to
 * x and every weight, of
 *   Loss = sum(dout * layer(x)) + reg_coef * (1/T) sum_t H_t,
 * dout [T, d] (layer dtype, device) being the upstream gradient of the
 * output and H_t the router entropy of token t: the entropy of the token's
 * gates normalised over its active experts (0 without any; the pages name the
 * entropy penalty but print no formula, so this is a stated reading).  The
 * inter-expert mean Wbar is treated as the function of W_up it is during
 * training, so every expert's W_up receives (1/E) x^T dm.  The ReLU's
 * derivative at z = 0 is 0; experts with lambda_e = 0 get no gradient.  TopK
 * layers differentiate the softmax over the kept logits (reg_coef must be 0).
 * The routing is recomputed from x (the forward's kernels), so no state of a
 * previous forward call is needed.  Requires a layer loaded with
 * cfg.backward = 1 and non-gated experts (else DECO_ERR_UNSUPPORTED); T in
 * 1..max_tokens; asynchronous on `stream`; allocates nothing.  Part of the
 * work runs on two more streams the layer creates at load (default
 * priority), forked from `stream` and joined back into it by events, so the
 * call is ordered on `stream` as a whole.  Overwrites the layer's routing state
 * (deco_moe_copy_routing then describes x). */
int deco_moe_backward(const deco_moe_layer* L, const void* x, const void* dout, int64_t T,
                      float reg_coef, const deco_moe_grads* grads, void* stream);

/* The adaptive sparsity-regularisation coefficient (qidianchuan.cn write-up,
 * section 三; DECO paper Sec. 2 "Auxiliary training objective"), one step,
 * meant to run after every training iteration: returns coef * factor when the
 * measured activation ratio is above the target, coef / factor when below
 * (the pages' example factor is 1.002), coef when equal.  Host only. */
float deco_moe_sparsity_coef_update(float coef, float active_ratio, float target_ratio, float factor);

/* Health flags of L's device-side work, read synchronously (waits for all
 * work on the device) and cleared by the read.  Bit 0: an in-kernel
 * hand-off between workgroups of the decode path timed out (the output of
 * that call is not valid); the bit naming the hand-off is set with it:
 * 4 an expert's per-row sums of squares (NormSiLU's RMS across column
 * slices), 8 the TopK logits, 16 the shared expert's sums of squares
 * (shared_rms layers); bit 1 (2) is no longer used (the mean term is folded
 * into the decode path's matrices).  The prefill and backward kernels never
 * wait on other workgroups.  Bit 5 (32), any path of a bf16 layer: a value
 * of the down-projection's fp16 operands or of the fp16 pair rows left the
 * fp16 range (a gate too large for it), or, on the decode path, an x value
 * did (it enters the folded NormSiLU-input product in fp16); that call's
 * output is not valid.
 * Returns DECO_ERR_INVALID_ARG on NULL arguments. */
int deco_moe_read_error_flags(const deco_moe_layer* L, uint32_t* flags);

/* Release every device buffer of L (NULL is a no-op).  The caller must make
 * sure no work using L is still pending on any stream. */
void deco_moe_free(deco_moe_layer* L);

/* Static English description of a status code. */
const char* deco_moe_status_string(int status);

/* Per-kernel timing with HIP events, for measurement.  While enabled, every
 * forward records a start/stop event pair around each kernel it launches, on
 * the launch stream.  deco_moe_timing_read waits for those events and returns
 * for kernel slot `idx` its name, the summed elapsed milliseconds and the
 * number of launches since the last reset; it returns DECO_ERR_INVALID_ARG
 * once idx passes the last slot.  Not thread-safe; global to the library. */
int deco_moe_timing_enable(int enable);
int deco_moe_timing_reset(void);
int deco_moe_timing_read(int idx, const char** name, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* DECO_MOE_H */
