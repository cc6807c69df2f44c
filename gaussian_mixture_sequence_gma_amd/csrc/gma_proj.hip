// Projection GEMM of the GMA layer ("Gaussian Mixture Attention", Section
// "Projections", Eq. 4): Q_X = X W_Q, K_X = X W_K, V_X = X W_V with no bias.
// X is [B*N, d_model] bf16, each W is [d_model, H*d] bf16, and head h owns
// columns [h*d, (h+1)*d).  The products are accumulated in fp32 on bf16 MFMA
// and stored unrounded in fp32, head-major [B,H,N,d], which is the layout the
// GMA kernels stream.
//
// One launch covers all three matrices.  A workgroup owns 128 output features
// x 128 tokens and walks d_model in steps of 64; both operand tiles are copied
// global -> LDS directly (no register staging) into a double buffer, so the
// copy of step k+1 runs under the MFMAs of step k.  The product is formed as
// D^T = W^T X^T: W supplies the MFMA A operand through transpose reads of its
// row-major [k][feature] tile, X supplies the B operand with plain 16-byte
// reads of its row-major [token][k] tile, and each accumulator lane then holds
// four consecutive features of one token, stored as one 16-byte vector.
#include "gma_device.h"
#include "gma_internal.h"

namespace gma {
namespace {

constexpr int kPT = 128;   // tokens per workgroup tile
constexpr int kPF = 128;   // output features per workgroup tile
constexpr int kPK = 64;    // d_model step

struct ProjArgs {
  const bf16* X;
  const bf16* W[3];
  float* out[3];
  int ncols[3];      // H * d of each matrix (multiple of 16)
  int dh[3];         // d of each matrix
  int ft0[4];        // first feature tile of each matrix; ft0[3] = total feature tiles
  int64_t M, N;      // M = B * N tokens
  int H, Dm;
  int64_t blocks;
};

// X tile [128 tokens][64 k]: eight 16-byte chunks per row, chunk c of row r at
// c ^ xswz(r).  Eight consecutive rows, and the eight even (odd) rows of 16
// consecutive ones, read the same logical chunk from distinct banks.
__device__ __forceinline__ int xswz(int r) { return (r ^ (r >> 3)) & 7; }

__global__ void __launch_bounds__(kThreads, 2) gma_proj_kernel(ProjArgs a) {
  __shared__ __attribute__((aligned(16))) bf16 Xs[2][kPT * kPK];
  __shared__ __attribute__((aligned(16))) bf16 Ws[2][kPK * kPF];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int s16 = lane & 15, g = lane >> 4;

  // Consecutive logical tiles share the X token tile; group them on one XCD
  // (workgroups are dealt to the eight XCDs round-robin) so X stays in its L2.
  int64_t L = blockIdx.x;
  if ((a.blocks & 7) == 0) L = (L & 7) * (a.blocks >> 3) + (L >> 3);
  const int ftot = a.ft0[3];
  const int64_t mt = L / ftot;
  const int ft = (int)(L - mt * ftot);
  const int m = ft >= a.ft0[2] ? 2 : (ft >= a.ft0[1] ? 1 : 0);
  const int f0 = (ft - a.ft0[m]) * kPF;
  const int ncols = a.ncols[m];
  const int64_t tok0 = mt * kPT;
  const bf16* __restrict__ X = a.X;
  const bf16* __restrict__ W = a.W[m];

  // Per-lane global sources of the direct copies.  X: wave w fills 1 KB
  // segments w, w+4, w+8, w+12 (eight rows each); W: the same segments hold
  // four k-rows each.
  const bf16* xsrc[4];
  const bf16* wsrc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int seg = w + 4 * j;
    const int xr = 8 * seg + (lane >> 3);
    int64_t tok = tok0 + xr;
    if (tok >= a.M) tok = a.M - 1;                        // ragged tail: rows never stored
    const int xc = (lane & 7) ^ xswz(xr);
    xsrc[j] = X + tok * a.Dm + xc * 8;
    const int wr = 4 * seg + (lane >> 4);
    const int wc = (lane & 15) ^ ((2 * wr) & 14);          // swz_elem<16> layout
    int col = f0 + wc * 8;
    if (col >= ncols) col = ncols - 8;                     // ragged features: never stored
    wsrc[j] = W + (int64_t)wr * ncols + col;
  }
  auto stage = [&](int kstep, int buf) {
    const int64_t kx = (int64_t)kstep * kPK;
    const int64_t kw = kx * ncols;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      global_to_lds16(xsrc[j] + kx, &Xs[buf][(w + 4 * j) * 512]);
      global_to_lds16(wsrc[j] + kw, &Ws[buf][(w + 4 * j) * 512]);
    }
  };

  const int wf = w & 1, wt = w >> 1;   // wave owns features wf*64.., tokens wt*64..
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = a.Dm / kPK;
  stage(0, 0);
  wait_global_loads();
  lds_barrier();
  for (int it = 0; it < nk; ++it) {
    const int buf = it & 1;
    if (it + 1 < nk) stage(it + 1, buf ^ 1);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8 wa[4], xb[4];
#pragma unroll
      for (int fm = 0; fm < 4; ++fm)
        wa[fm] = tr_chunk_swz<16>(Ws[buf], kk * 32, wf * 64 + fm * 16);
#pragma unroll
      for (int tn = 0; tn < 4; ++tn) {
        const int r = wt * 64 + tn * 16 + s16;
        xb[tn] = ld16<bf16x8>(&Xs[buf][r * kPK + (((kk * 4 + g) ^ xswz(r)) << 3)]);
      }
#pragma unroll
      for (int fm = 0; fm < 4; ++fm)
#pragma unroll
        for (int tn = 0; tn < 4; ++tn) acc[fm][tn] = mma(wa[fm], xb[tn], acc[fm][tn]);
    }
    wait_global_loads();
    lds_barrier();
  }

  // Lane (s16, g) of tile (fm, tn) holds features f..f+3, f = 16 fm + 4 g, of
  // token 16 tn + s16; four consecutive features never straddle a head.
  const int dh = a.dh[m];
  float* __restrict__ out = a.out[m];
#pragma unroll
  for (int tn = 0; tn < 4; ++tn) {
    const int64_t t = tok0 + wt * 64 + tn * 16 + s16;
    if (t >= a.M) continue;
    const int64_t b = t / a.N, n = t - b * a.N;
#pragma unroll
    for (int fm = 0; fm < 4; ++fm) {
      const int f = f0 + wf * 64 + fm * 16 + 4 * g;
      if (f >= ncols) continue;
      const int h = f / dh, j = f - h * dh;
      st16(out + (((b * a.H + h) * a.N + n) * dh + j), acc[fm][tn]);
    }
  }
}

}  // namespace

hipError_t launch_proj(const void* X, const void* const W[3], float* const out[3], int64_t B,
                       int64_t N, int H, int d_model, int d_r, int d_v, hipStream_t s) {
  ProjArgs a{};
  a.X = static_cast<const bf16*>(X);
  const int d[3] = {d_r, d_r, d_v};
  int ft = 0;
  for (int m = 0; m < 3; ++m) {
    a.W[m] = static_cast<const bf16*>(W[m]);
    a.out[m] = out[m];
    a.dh[m] = d[m];
    a.ncols[m] = H * d[m];
    a.ft0[m] = ft;
    ft += (a.ncols[m] + kPF - 1) / kPF;
  }
  a.ft0[3] = ft;
  a.M = B * N;
  a.N = N;
  a.H = H;
  a.Dm = d_model;
  const int64_t mtiles = (a.M + kPT - 1) / kPT;
  a.blocks = mtiles * ft;
  if (a.blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (g_launch_hook) g_launch_hook("gma_proj", s, 1);
  gma_proj_kernel<<<dim3((unsigned)a.blocks), dim3(kThreads), 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (g_launch_hook) g_launch_hook("gma_proj", s, 0);
  return e;
}

}  // namespace gma
