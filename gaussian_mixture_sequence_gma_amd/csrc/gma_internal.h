// Host-side plan and launcher declarations shared by the GMA translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gma {

// Everything derived from a problem shape: padded sizes, kernel configuration,
// split counts and the workspace layout.  Computed identically by the
// workspace-size query and by the forward call.
struct Plan {
  bool bf = false;          // bf16 storage / split-bf16 arithmetic
  bool out_bf = false;      // output element type
  int64_t B = 0, H = 0, N = 0, BH = 0;
  int DR = 0, DV = 0, K = 0;
  int CT = 0;               // 16-wide component tiles (power of two)
  int CPW = 0, NG = 0;      // component tiles per wave, component groups per workgroup
  int Kp = 0;               // padded component count = 16 * CT
  int DRP = 0;              // padded routing dimension (multiple of the MFMA chunk span)
  int64_t tiles = 0;        // 64-token tiles per sequence
  int S = 0;                // workgroups per sequence for the write and read kernels
  int tiles_per_split = 0;
  int TG = 0;               // token groups per workgroup (partials per split)
  // causal
  int span_tiles = 0;       // 64-token chunks per causal span
  int nspan = 0;            // spans per sequence
  bool prod = false;        // causal on the product path (the scan kernel does not fit)
  bool khalf = false;       // causal scan or read-out once per half of K_pad = 256
                            // (causal_khalf, bidir_khalf)
  // workspace layout (bytes)
  size_t head_bytes = 0;
  size_t off_params = 0, off_partial = 0, off_partial_z = 0, off_vt = 0, off_z = 0, off_vtab = 0;
  size_t off_state = 0, off_state_z = 0, off_carry = 0, off_carry_z = 0;
  size_t off_gt = 0;        // causal token-owner scan: the keys' Gamma^K^T tiles
  size_t off_qpart = 0, off_qpart2 = 0;   // khalf: the first half's query partials
  size_t total = 0;
};

struct Tensors {
  const void* q = nullptr;
  const void* k = nullptr;
  const void* v = nullptr;
  const float* mu = nullptr;
  const float* ls2 = nullptr;
  const float* lpi = nullptr;
  void* out = nullptr;
  int32_t* assign_q = nullptr;
  int32_t* assign_k = nullptr;
  float* gamma = nullptr;
  float eps = 0.f;
  char* ws = nullptr;
  // routing vectors given as bf16 pairs (value = q + q_lo): the layer's
  // projections on the bf16 kernels
  const void* q_lo = nullptr;
  const void* k_lo = nullptr;
  // bidirectional launch that stops after the latent write: V~ [BH,K,d_v] and
  // Z [BH,K] of all the keys, unpadded (the carried state of a prefix)
  float* state_v = nullptr;
  float* state_z = nullptr;
  // forward from the unconstrained parameters (Eqs. 14-15): with omega set, the
  // prologue takes log sigma^2 = log(softplus(omega) + eps_sigma) and
  // log pi = alpha - logsumexp(alpha) in place of ls2 and lpi
  const float* omega = nullptr;
  const float* alpha = nullptr;
  float eps_sigma = 0.f;
  // usage statistics: per-workgroup partials and the utilisation threshold
  float* diag = nullptr;
  float thr = 0.f;
  // fused layer: the queries' exponentials from the projection epilogue
  // ([BH][N][kc] bf16; the keys' Gamma^K^T sit at off_gt) and kc
  void* eq = nullptr;
  int kc = 0;
  void* vtab = nullptr;   // bidirectional: the summed state as an operand table
};

// Launch helpers; each returns hipSuccess or the launch error.  `tag` names the
// kernel for the timing facility.
typedef void (*launch_hook_t)(const char* tag, hipStream_t s, int begin);
// Per calling thread (set by gma_timing_enable); null when timing is off.
extern thread_local launch_hook_t g_launch_hook;

hipError_t launch_prologue(const Plan& p, const Tensors& t, hipStream_t s);
// Sum PS partial states per sequence in slot order ([BH][PS][Kp][DV] and
// [BH][PS][Kp] fp32) into vt, z and, as the read-out's bf16 MFMA operand table
// ([BH][DV/16 + 1][Kp/32][64 lanes][8], the last block Z_hi, Z_lo, 1, zeros),
// vtab.
hipError_t launch_reduce_table(const float* partial, const float* partial_z, int PS, int64_t BH,
                               int Kp, int DV, float* vt, float* z, __bf16* vtab, hipStream_t s);
// Whether the bf16 kernels take split routing vectors (q_lo / k_lo) for this shape.
bool bidir_split_ok(const Plan& p);
bool causal_split_ok(const Plan& p);
hipError_t launch_bidir(const Plan& p, const Tensors& t, hipStream_t s);
hipError_t launch_causal(const Plan& p, const Tensors& t, hipStream_t s);
// The fused layer (bf16, d_r = 64, K <= 64, the scan kernel's shapes; p is the
// causal plan, K_pad 64, for either variant): after launch_proj's fused
// epilogue, span totals from the keys' Gamma^K^T at off_gt, then the scan
// (causal) or the read-out over every span's totals (bidirectional) on the
// given responsibilities (t.eq, t.kc).
bool layer_fused_ok(const Plan& p);
hipError_t launch_layer_fused(const Plan& p, const Tensors& t, bool causal, hipStream_t s);
hipError_t launch_resp(const Plan& p, const Tensors& t, hipStream_t s);
// Usage statistics of the responsibilities of t.q (per head, over batches and
// tokens); t.diag holds B*H*S*(3 K_pad + 4) floats of partials.
hipError_t launch_usage(const Plan& p, const Tensors& t, int32_t* counts, float* mean_gamma,
                        float* util, float* head_stats, hipStream_t s);
// One causal decode step (N = 1 per sequence) against the carried state
// state_v [BH,K,d_v], state_z [BH,K] (fp32, updated in place).
hipError_t launch_decode(const Plan& p, const Tensors& t, float* state_v, float* state_z,
                         hipStream_t s);
// Backward of the forward (bidirectional or causal): dO in, gradients out (dQ, dK, dV of
// the input dtype; parameter gradients fp32, written).
struct BwdTensors {
  const void* dO = nullptr;
  void* dQ = nullptr;
  void* dK = nullptr;
  void* dV = nullptr;
  float* dmu = nullptr;
  float* dls2 = nullptr;
  float* dlpi = nullptr;
};
// pp: the plan at the padded length (N rounded up to 64 when causal); N: the
// caller's sequence length.
size_t backward_workspace_bytes(const Plan& pp, bool causal, int64_t N);
hipError_t launch_backward(const Plan& pp, const Tensors& t, const BwdTensors& gt, bool causal,
                           int64_t N, hipStream_t s);
// The forward as a chain of fp32 products over stored responsibilities, for
// shapes whose fused scan kernel does not fit.  pp: the bidirectional plan at
// the padded length (N rounded up to 64 when causal); N: the caller's length;
// out_bf: the output type (the inputs are of pp's type).
size_t prod_forward_workspace_bytes(const Plan& pp, bool causal, int64_t N);
hipError_t launch_prod_forward(const Plan& pp, const Tensors& t, bool causal, int64_t N,
                               bool out_bf, hipStream_t s);
// log sigma^2 = log(softplus(omega) + eps_sigma) over [H,K,d_r] and
// log pi = alpha - logsumexp(alpha) over [H,K].
hipError_t launch_reparam(const float* omega, const float* alpha, float eps_sigma, int64_t H,
                          int K, int d_r, float* log_sigma2, float* log_pi, hipStream_t s);
// Q_X, K_X, V_X = X W_Q, X W_K, X W_V (W[0..2]) into fp32 head-major out[0..2].
// split = 0: out[0..2] are fp32.  split = 1: Q_X and K_X as bf16 pairs (out[m],
// lo[m]: value = out + lo, 16 significant bits), V_X as bf16 in out[2].
// fz (the fused form, d_r = 64): Q_X and K_X are not stored; the
// epilogue writes per query the exponentials exp2(s - max s) of its routing
// scores, bf16 [B,H,N][kc], and per 64-key chunk the keys' responsibilities
// transposed, bf16 [B,H,ceil(N/64)][kc][64] (and the assignments when given),
// from the prologue's tables; V_X as bf16 in out[2].
struct ProjFused {
  const char* params = nullptr;
  size_t head_bytes = 0;
  int Kp = 0, DRP = 0;
  int kc = 0;              // components formed: 32 or 64
  void* eq = nullptr;
  void* gt = nullptr;
  int32_t* assign_q = nullptr;
  int32_t* assign_k = nullptr;
};
hipError_t launch_proj(const void* X, const void* const W[3], void* const out[3],
                       void* const lo[2], int split, int64_t B, int64_t N, int H, int d_model,
                       int d_r, int d_v, hipStream_t s, const ProjFused* fz = nullptr);

}  // namespace gma
