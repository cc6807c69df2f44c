// Constrained mixture parameters from the unconstrained ones ("Gaussian
// Mixture Attention: Linear-Time Sequence Mixing via Probabilistic Latent
// Routing", the reparameterisations used for training, Eqs. 14-15):
//   log sigma^2_kj = log(log(1 + exp(omega_kj)) + eps_sigma)   [H,K,d_r]
//   log pi_k       = alpha_k - log sum_l exp(alpha_l)            [H,K]
// the two arrays the forward and the decode step take.  One launch: the first
// workgroups map the elements of omega, one workgroup per head follows for the
// prior normalisation (a wave-wide max and sum over the K logits).
#include <hip/hip_runtime.h>
#include <math.h>

#include "gma_device.h"
#include "gma_internal.h"

namespace gma {

namespace {

__global__ void __launch_bounds__(256) gma_reparam_kernel(const float* __restrict__ omega,
                                                          const float* __restrict__ alpha,
                                                          float eps_sigma, int64_t n,
                                                          int64_t elem_blocks, int K,
                                                          float* __restrict__ ls2,
                                                          float* __restrict__ lpi) {
  if ((int64_t)blockIdx.x < elem_blocks) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    // log(1 + exp(w)) as max(w, 0) + log1p(exp(-|w|)): no overflow for large w
    if (i < n) ls2[i] = reparam_log_var(omega[i], eps_sigma);
    return;
  }
  if (threadIdx.x >= 64) return;
  const int64_t h = (int64_t)blockIdx.x - elem_blocks;
  const int lane = threadIdx.x;
  const float* a = alpha + h * K;
  const float lse = wave_log_norm(a, K);
  for (int k = lane; k < K; k += 64) lpi[h * K + k] = a[k] - lse;
}

}  // namespace

hipError_t launch_reparam(const float* omega, const float* alpha, float eps_sigma, int64_t H,
                          int K, int d_r, float* log_sigma2, float* log_pi, hipStream_t s) {
  const int64_t n = H * K * (int64_t)d_r;
  const int64_t eb = (n + 255) / 256;
  if (g_launch_hook) g_launch_hook("gma_reparam", s, 1);
  hipLaunchKernelGGL(gma_reparam_kernel, dim3((unsigned)(eb + H)), dim3(256), 0, s, omega, alpha,
                     eps_sigma, n, eb, K, log_sigma2, log_pi);
  if (g_launch_hook) g_launch_hook("gma_reparam", s, 0);
  return hipGetLastError();
}

}  // namespace gma
