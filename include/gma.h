/*
 * gma.h -- C ABI of the MI355X (gfx950) Gaussian Mixture Attention forward library.
 *
 * Method: "Gaussian Mixture Attention: Linear-Time Sequence Mixing via
 * Probabilistic Latent Routing" (arXiv 2606.18283).  Queries and keys are
 * mapped to posterior responsibilities over K diagonal-Gaussian components
 * (Section "Gaussian routing components", Eqs. 2-3, and Eq. 16 which writes
 * the posterior as a softmax of log-prior plus log-density); keys write values
 * into a K-slot latent memory V~ = Gamma^K^T V_X with normaliser
 * Z = Gamma^K^T 1 (Eqs. 5-6); queries read O = Gamma^Q V~ / (Gamma^Q Z + eps)
 * (Eq. 7 and its footnote).  The causal variant replaces V~ and Z by inclusive
 * prefix sums over positions j <= i (Section "Causal GMA", Eq. 8b).
 *
 * Conventions shared by every entry point:
 *  - Every tensor pointer is DEVICE memory owned by the caller, contiguous,
 *    row-major, 16-byte aligned.  The library never allocates, frees, or keeps
 *    a pointer after a call returns.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream) and never synchronise it.  Argument validation is synchronous and
 *    happens before any launch; on a nonzero return nothing was launched
 *    (except GMA_ERR_HIP, which reports a failed launch).
 *  - Calls that share a workspace must not overlap in time; otherwise calls
 *    are reentrant.  No exception crosses this interface and the library never
 *    prints; gma_last_error() holds a message for the calling thread.
 *  - NaN / Inf inputs are not checked and propagate.
 */
#ifndef GMA_H
#define GMA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { GMA_F32 = 0, GMA_BF16 = 1 } gma_dtype;

typedef enum {
  GMA_OK = 0,
  GMA_ERR_INVALID_ARG = 1,   /* null pointer, bad size, misalignment, eps < 0 or not finite */
  GMA_ERR_UNSUPPORTED = 2,   /* valid but outside the supported shape set (see gma_dims) */
  GMA_ERR_WORKSPACE = 3,     /* workspace_bytes smaller than the *_workspace_bytes figure */
  GMA_ERR_HIP = 4            /* a HIP runtime call or kernel launch failed */
} gma_status;

/* Problem shape.  B batches x H heads x N positions.
 *  d_r  routing dimension of Q_X, K_X and the component means: 16, 32, 64 or 128
 *  d_v  value dimension of V_X and the output: 16, 32, 64 or 128
 *  K    number of Gaussian components: 1..256.  A causal shape whose scan kernel
 *       tiles do not fit in LDS (fp32 with K > 64 and d_v = 128 or K > 128;
 *       bf16 with K > 128 and d_v = 128) runs the causal form as a chain of
 *       fp32 products over stored responsibilities instead, which needs
 *       B*H*ceil(N/64) <= 65535 (else GMA_ERR_UNSUPPORTED) and a larger
 *       workspace; the result is the same to the fp32 rounding level
 *  dtype storage type of Q_X, K_X, V_X and out (gma_layer_forward: of X, W and out)
 *  chunk causal scan chunk length: 0 (= 64) or 64; the result does not depend on it */
typedef struct gma_dims {
  int64_t B, H, N;
  int32_t d_r, d_v, K;
  int32_t dtype;
  int32_t chunk;
} gma_dims;

/* Host-only check of a call's arguments, as the entry points make it before any
 * launch: the shape, eps and variant (the same rules as gma_forward, including
 * the product-path batch limit of the causal form), then each of the nptrs pointers in ptrs (each
 * must be non-NULL and 16-byte aligned; nptrs may be 0 and ptrs NULL), then
 * workspace_bytes against workspace_needed (a *_workspace_bytes figure).  No
 * pointer is dereferenced.  Returns GMA_OK, GMA_ERR_INVALID_ARG,
 * GMA_ERR_UNSUPPORTED or GMA_ERR_WORKSPACE. */
int gma_validate(const gma_dims* d, float eps, int causal, const void* const* ptrs, int nptrs,
                 size_t workspace_bytes, size_t workspace_needed);

/* Bytes of device workspace gma_forward needs for this shape and variant
 * (written to *bytes).  The same workspace also serves gma_responsibilities.
 * Bidirectional: a few tens of MB that do not grow with N (per-head tables
 * and per-split partial sums).  Causal with bf16 inputs: in addition the
 * keys' responsibilities as bf16 tiles, 2 * K_pad bytes per token-head
 * (K_pad: the smallest of 64, 128, 256 not below K), and at K_pad = 256 with half
 * scans 4 * d_v + 16 bytes per token-head of partial results. */
int gma_forward_workspace_bytes(const gma_dims* d, int causal, size_t* bytes);

/* GMA forward.
 *  Q_X, K_X    [B,H,N,d_r] of d->dtype: query and key routing vectors q_i, k_j
 *  V_X         [B,H,N,d_v] of d->dtype: values
 *  mu          [H,K,d_r] fp32: component means mu_k (one mixture per head, shared
 *              by queries and keys and by every batch)
 *  log_sigma2  [H,K,d_r] fp32: log of the diagonal covariance entries sigma^2_kd
 *  log_pi      [H,K] fp32: log mixture priors, up to an additive constant per head
 *              (the posterior does not depend on it; e.g. the prior logits of Eq. 15)
 *  eps         >= 0, finite: the stabiliser of Eq. 7 (also used by the causal form)
 *  causal      0: Eq. 7 over all keys; 1: inclusive prefix j <= i
 *  out         [B,H,N,d_v] of d->dtype: O
 *  assign_q    optional [B,H,N] int32: z_i = argmax_k gamma^Q_ik (lowest index on ties)
 *  assign_k    optional [B,H,N] int32: the same for keys
 *  workspace   device scratch of at least gma_forward_workspace_bytes bytes
 * Arithmetic: fp32 inputs run fp32 MFMA throughout; bf16 inputs run bf16 MFMA
 * with hi/lo operand splitting for the Gaussian scores and fp32 accumulation. */
int gma_forward(const void* Q_X, const void* K_X, const void* V_X,
                const float* mu, const float* log_sigma2, const float* log_pi,
                float eps, int causal, void* out, const gma_dims* d,
                int32_t* assign_q, int32_t* assign_k,
                void* workspace, size_t workspace_bytes, void* stream);

/* gma_forward from the unconstrained mixture parameters the optimiser updates
 * (the reparameterisations used for training, "Learning", Eqs. 14-15): the
 * prologue derives log sigma^2 = log(log(1 + exp(omega)) + eps_sigma) and
 * log pi = alpha - log sum exp(alpha) itself, with the arithmetic of
 * gma_reparameterize, so the result is bit for bit gma_reparameterize followed
 * by gma_forward, in one launch fewer and without the two derived arrays.
 *  omega  [H,K,d_r] fp32, alpha [H,K] fp32 (4-byte aligned); eps_sigma > 0,
 *         finite (else GMA_ERR_INVALID_ARG)
 * Every other argument, the workspace (gma_forward_workspace_bytes) and the
 * errors as gma_forward. */
int gma_forward_reparam(const void* Q_X, const void* K_X, const void* V_X,
                        const float* mu, const float* omega, const float* alpha,
                        float eps_sigma, float eps, int causal, void* out,
                        const gma_dims* d, int32_t* assign_q, int32_t* assign_k,
                        void* workspace, size_t workspace_bytes, void* stream);

/* gma_forward without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  It runs the same kernels as gma_forward, with the
 * workspace taken from a static device array of GMA_NOALLOC_SCRATCH_BYTES
 * that the library holds on each GPU it runs on until the process ends; the
 * call allocates nothing.  Shapes whose gma_forward_workspace_bytes exceed
 * that size return GMA_ERR_UNSUPPORTED before any launch.  Every call on a
 * GPU shares that GPU's array (no part of it needs to start at zero: each
 * kernel reads only what an earlier kernel of the same call wrote), so calls
 * that overlap in time on one GPU (different streams, or threads) race and
 * must be serialised by the caller.  Arguments and errors as gma_forward. */
#define GMA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int gma_forward_noalloc(const void* Q_X, const void* K_X, const void* V_X,
                        const float* mu, const float* log_sigma2, const float* log_pi,
                        float eps, int causal, void* out, const gma_dims* d,
                        int32_t* assign_q, int32_t* assign_k, void* stream);

/* Bytes of device workspace gma_layer_forward needs. */
int gma_layer_workspace_bytes(const gma_dims* d, int32_t d_model, int causal, size_t* bytes);

/* Projection layer followed by the GMA forward (Section "Projections", Eq. 4:
 * Q_X = X W_Q, K_X = X W_K, V_X = X W_V; no bias, no output projection).
 *  X          [B,N,d_model] of d->dtype (GMA_BF16 only)
 *  W_Q, W_K   [d_model, H*d_r] of d->dtype; head h uses columns [h*d_r, (h+1)*d_r)
 *  W_V        [d_model, H*d_v] of d->dtype; head h uses columns [h*d_v, (h+1)*d_v)
 *  d_model    multiple of 64, 64..8192
 * The projections are accumulated in fp32 (bf16 x bf16 products are exact in
 * fp32).  With d_r = 64 and K <= 64 (where the bf16 scan kernel takes the
 * shape) the projection's epilogue forms the routing responsibilities of
 * "Gaussian routing components" (Eq. 3) from the fp32 accumulators
 * and Q_X, K_X never reach memory; V_X is rounded to bf16.  Otherwise, where
 * the bf16 GMA kernels support the shape, Q_X and K_X are kept as bf16 pairs
 * hi + lo (16 significant bits), V_X is rounded to bf16, and the bf16 GMA
 * path runs on them; else all three stay fp32 and feed the fp32 GMA path
 * (gma_layer_projection_layout names the form).  out is [B,H,N,d_v] of
 * d->dtype.  The projections kept stay in the workspace after the call, at
 * the offsets gma_layer_projection_layout reports.  Other arguments as
 * gma_forward. */
int gma_layer_forward(const void* X, const void* W_Q, const void* W_K, const void* W_V,
                      int32_t d_model, const float* mu, const float* log_sigma2,
                      const float* log_pi, float eps, int causal, void* out,
                      const gma_dims* d, int32_t* assign_q, int32_t* assign_k,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Storage of the projections gma_layer_forward leaves in its workspace. */
typedef enum {
  GMA_PROJ_F32 = 0,        /* Q_X, K_X, V_X fp32 [B,H,N,d] at offsets[0..2] */
  GMA_PROJ_SPLIT_BF16 = 1, /* bf16 [B,H,N,d]: Q_X hi, Q_X lo, K_X hi, K_X lo, V_X at
                              offsets[0..4]; Q_X = hi + lo */
  GMA_PROJ_FUSED_BF16 = 2  /* Q_X and K_X are not stored (the projection's epilogue
                              forms the routing responsibilities from them); V_X bf16
                              [B,H,N,d_v] at offsets[4], offsets[0..3] = 0 */
} gma_proj_format;

/* Where gma_layer_forward leaves the projections for this shape and variant
 * (host only): *format is a gma_proj_format and offsets[m] the byte offset of
 * array m from the start of the workspace (unused entries 0).  offsets holds 5
 * entries.  Errors as gma_layer_workspace_bytes. */
int gma_layer_projection_layout(const gma_dims* d, int32_t d_model, int causal,
                                int32_t* format, size_t offsets[5]);

/* Responsibilities alone (Eq. 3), for testing and diagnostics.
 *  X_r    [B,H,N,d_r] of d->dtype; head h's parameters apply to [b,h,:,:]
 *  gamma  optional [B,H,N,K] fp32
 *  assign optional [B,H,N] int32 (lowest index on ties)
 * Uses the same arithmetic as gma_forward; workspace as gma_forward_workspace_bytes. */
int gma_responsibilities(const void* X_r, const float* mu, const float* log_sigma2,
                         const float* log_pi, const gma_dims* d, float* gamma,
                         int32_t* assign, void* workspace, size_t workspace_bytes,
                         void* stream);

/* Bytes of device workspace gma_backward needs for this shape and variant. */
int gma_backward_workspace_bytes(const gma_dims* d, int causal, size_t* bytes);

/* Gradients of a scalar loss L through the forward, given dL/dO ("Gradient
 * structure": the score gradient of Eq. 18, gamma times the upstream
 * gradient minus its gamma-weighted mean, chained through the Gaussian score
 * of Eqs. 2-3 and 16 to the routing vectors and the parameters, and through
 * Eqs. 5-7, or the prefix form of Eq. 8b when causal, to the values).
 *  Q_X, K_X, V_X, mu, log_sigma2, log_pi, eps, causal  as gma_forward
 *  dO         [B,H,N,d_v] of d->dtype: dL/dO
 *  dQ, dK     [B,H,N,d_r] of d->dtype: written
 *  dV         [B,H,N,d_v] of d->dtype: written
 *  dmu, dlog_sigma2  [H,K,d_r] fp32; dlog_pi [H,K] fp32: written (not
 *             accumulated), summed over batches and over queries and keys
 *  workspace  at least gma_backward_workspace_bytes bytes (it holds the
 *             responsibilities, their gradients and fp32 copies of the inputs:
 *             about 4 (2(2 d_r + 1) + 2(d_v + 1) + 4K + 2 d_r + d_v) bytes per
 *             token-head)
 * The forward quantities are recomputed; the output O is not an input.
 * fp32 arithmetic (products on fp32 MFMA); for bf16 inputs the
 * responsibilities are those of the bf16 forward.  N is limited to
 * 65535 * 64, and when causal B*H*ceil(N/64) to 65535 (else
 * GMA_ERR_UNSUPPORTED); the causal workspace also holds per-64-token-chunk
 * states and 64 x 64 chunk products. */
int gma_backward(const void* Q_X, const void* K_X, const void* V_X, const float* mu,
                 const float* log_sigma2, const float* log_pi, float eps, int causal,
                 const void* dO, const gma_dims* d, void* dQ, void* dK, void* dV,
                 float* dmu, float* dlog_sigma2, float* dlog_pi, void* workspace,
                 size_t workspace_bytes, void* stream);

/* Bytes of device workspace gma_usage_stats needs for this shape. */
int gma_usage_workspace_bytes(const gma_dims* d, size_t* bytes);

/* Component-usage diagnostics of the responsibilities (Eq. 3) of routing
 * vectors X_r, per head over all batches and positions -- the marginal use of
 * the mixture components and the hard assignments z_i = argmax_k gamma_ik that
 * the paper proposes to monitor for under-use and collapse.  With
 * T = B * N tokens per head:
 *  X_r         [B,H,N,d_r] of d->dtype (queries or keys); d->d_v is not used
 *              but must be a supported value
 *  util_threshold  finite; e.g. 0.1
 *  counts      optional [H,K] int32: tokens i with z_i = k (lowest index on ties)
 *  mean_gamma  optional [H,K] fp32: (1/T) sum_i gamma_ik
 *  utilization optional [H,K] fp32: (1/T) #{i : gamma_ik > util_threshold}
 *  head_stats  optional [H,3] fp32: mean token entropy (1/T) sum_i
 *              -sum_k gamma_ik ln gamma_ik (nats); usage entropy
 *              -sum_k p_k ln p_k / ln K with p_k = counts_k / T (0 when K = 1);
 *              the number of components with counts_k > 0
 *  workspace   at least gma_usage_workspace_bytes bytes
 * The responsibilities are those of gma_responsibilities (same arithmetic);
 * the statistics are reduced on the device, none per token reaches memory.
 * B*N must be below 2^31 (else GMA_ERR_UNSUPPORTED). */
int gma_usage_stats(const void* X_r, const float* mu, const float* log_sigma2,
                    const float* log_pi, const gma_dims* d, float util_threshold,
                    int32_t* counts, float* mean_gamma, float* utilization,
                    float* head_stats, void* workspace, size_t workspace_bytes,
                    void* stream);

/* Carried state of a causal prefix ("Causal GMA": the prefix memories of
 * Eq. 8b at the last position, i.e. Eqs. 5-6 over all N keys given):
 *  K_X        [B,H,N,d_r] of d->dtype: key routing vectors of the prefix
 *  V_X        [B,H,N,d_v] of d->dtype: its values
 *  mu, log_sigma2, log_pi  as gma_forward
 *  state_v    [B,H,K,d_v] fp32 (16-byte aligned): written, S = Gamma^K^T V_X
 *  state_z    [B,H,K] fp32: written, z = Gamma^K^T 1
 *  assign_k   optional [B,H,N] int32: key assignments (lowest index on ties)
 *  workspace  at least gma_forward_workspace_bytes(d, 0) bytes
 * The same kernels as the bidirectional write step of gma_forward (same
 * arithmetic); the pair (state_v, state_z) is what gma_decode_step carries. */
int gma_prefix_state(const void* K_X, const void* V_X, const float* mu,
                     const float* log_sigma2, const float* log_pi, float* state_v,
                     float* state_z, const gma_dims* d, int32_t* assign_k,
                     void* workspace, size_t workspace_bytes, void* stream);

/* One causal decode step ("Causal GMA", Eq. 8b at a new position i): with the
 * carried state S = sum_{j<i} gamma^K_j v_j^T and z = sum_{j<i} gamma^K_j,
 *   S' = S + gamma^K(k_i) v_i^T,  z' = z + gamma^K(k_i),
 *   o_i = gamma^Q(q_i)^T S' / (gamma^Q(q_i)^T z' + eps),
 * and S', z' overwrite S, z.  d->N must be 1 (else GMA_ERR_INVALID_ARG);
 * d->chunk is ignored.
 *  q, k       [B,H,1,d_r] of d->dtype: the new token's query and key routing vectors
 *  v          [B,H,1,d_v] of d->dtype: its value
 *  mu, log_sigma2, log_pi, eps  as gma_forward
 *  state_v    [B,H,K,d_v] fp32 (16-byte aligned): S in, S' out
 *  state_z    [B,H,K] fp32: z in, z' out (all zeros for an empty prefix)
 *  out        [B,H,1,d_v] of d->dtype: o_i
 *  assign_q, assign_k  optional [B,H] int32: argmax of gamma^Q, gamma^K
 * No workspace.  Responsibilities use the direct form of the diagonal
 * log-density in fp32; the state stays fp32.  Starting from zeros and stepping
 * through a sequence gives gma_forward's causal output row by row. */
int gma_decode_step(const void* q, const void* k, const void* v, const float* mu,
                    const float* log_sigma2, const float* log_pi, float eps,
                    float* state_v, float* state_z, void* out, const gma_dims* d,
                    int32_t* assign_q, int32_t* assign_k, void* stream);

/* Constrained mixture parameters from the unconstrained ones the optimiser
 * updates (the reparameterisations used for training, Eqs. 14-15):
 *   log_sigma2[h,k,j] = log(log(1 + exp(omega[h,k,j])) + eps_sigma)
 *   log_pi[h,k]       = alpha[h,k] - log sum_l exp(alpha[h,l])
 *  omega      [H,K,d_r] fp32: covariance parameters
 *  alpha      [H,K] fp32: mixture-prior logits
 *  eps_sigma  > 0, finite: the variance floor of Eq. 14
 *  log_sigma2 [H,K,d_r] fp32, log_pi [H,K] fp32: written; the arrays gma_forward,
 *             gma_layer_forward and gma_decode_step take
 * fp32 arithmetic; log(1 + exp(w)) is evaluated as max(w,0) + log1p(exp(-|w|)).
 * Pointers need 4-byte alignment here; H <= 65535, K * d_r <= 2^24 and
 * H * K * d_r <= 2^30 (else GMA_ERR_UNSUPPORTED).  Any H, K, d_r >= 1 is accepted. */
int gma_reparameterize(const float* omega, const float* alpha, float eps_sigma, int64_t H,
                       int32_t K, int32_t d_r, float* log_sigma2, float* log_pi,
                       void* stream);

/* Static description of a status code. */
const char* gma_status_string(int status);

/* Message describing the last failure of a call made by this thread ("" if none). */
const char* gma_last_error(void);

/* Kernel timing (profiling aid), per calling thread.  While a thread has it
 * enabled, every kernel the library launches from that thread is bracketed by
 * two hipEvents recorded on the launch stream.  gma_timing_collect synchronises
 * the calling thread's events, accumulates per-kernel totals, writes up to
 * `max` entries and the number of distinct kernels to *count, and resets them.
 * Other threads' calls are neither timed nor affected.  If creating, recording
 * or reading an event pair failed, that launch is left out of the totals,
 * every event is still released, and the call returns GMA_ERR_HIP. */
typedef struct gma_kernel_time {
  char name[48];
  int64_t launches;
  double total_ms;
} gma_kernel_time;

int gma_timing_enable(int enable);
int gma_timing_collect(gma_kernel_time* out, int max, int* count);

#ifdef __cplusplus
}
#endif

#endif /* GMA_H */
