// Backward of the forward, bidirectional and causal ("Gaussian Mixture
// Attention: Linear-Time Sequence Mixing via Probabilistic Latent Routing",
// "Gradient structure": the score gradient of Eq. 18, chained to Q_X, K_X, V_X
// and the mixture parameters).
//
// Per unit u = (b, h), with Gq, Gk the [N,K] responsibilities (Eq. 3):
//   [V~ | Z]   = Gk^T [V | 1]                    (Eqs. 5-6)
//   [n | d-e]  = Gq [V~ | Z],  o = n / d          (Eq. 7)
//   [a | b]    = [dO / d | -(dO . o) / d]
//   dGq        = [a | b] [V~ | Z]^T               (= a . V~_k + b Z_k)
//   [dV~ | dZ] = Gq^T [a | b]
//   dV         = Gk dV~,   dGk = [V | 1] [dV~ | dZ]^T
//   dS         = G (dG - rowsum(G dG))            (Eq. 18, queries and keys)
//   [P1 | P2]  = dS [w | mu w],  w = exp(-log sigma^2):  dX = -X P1 + P2
//   [R1|R2|r0] = dS^T [X | X^2 | 1],  summed over batches and over Q and K:
//     dmu = w (R1 - mu r0),  dlog sigma^2 = w (R2 - 2 mu R1 + mu^2 r0) / 2 - r0 / 2,
//     dlog pi = r0.
// Appending a column of ones to the right operand turns every normaliser and
// every rank-one term into part of a product, so the whole pass is a chain of
// batched fp32 products (MFMA 16x16x4 f32, split over the token dimension
// where the product contracts it; one column tile per workgroup for widths up
// to 144) and row-wise kernels.  Rows of the augmented operands are padded to
// a multiple of four floats.  The responsibilities come from the
// responsibility kernel of the forward path.
//
// Causal ("Causal GMA", Eq. 8b): the same chain per 64-token chunk, with the
// prefix states of the earlier chunks ([V~ | Z] totals per chunk, exclusive
// prefix) for the queries, the suffix states of the later chunks for the keys
// (Gq_c^T [a | b]_c, exclusive suffix), and inside a chunk the masked 64 x 64
// products Gq_c Gk_c^T and [a | b]_c [V | 1]_c^T.
#include <hip/hip_runtime.h>
#include <math.h>

#include "gma_device.h"
#include "gma_internal.h"

namespace gma {

namespace {

// ---- batched fp32 product C[u] = op(A[u]) op(B[u]) --------------------------
struct GemmArgs {
  const float* A;
  const float* B;
  float* C;          // result, or the split partials [U][ksplit][M][N]
  int M, N, K;
  int lda, ldb, ldc;
  int64_t sA, sB, sC;
  int bmod;          // > 0: B of unit u is B + (u % bmod) * sB
  int ksplit;
  int vec;           // bit 0: A rows 16-byte aligned; bit 1: B rows
  int accum;         // add to C instead of overwriting it (ksplit == 1 only)
  // softmax Jacobian in the epilogue (wide kernel, one column tile, ksplit 1):
  // C = G (C - rowsum(G C)) with G of unit u at G + u * sG, row stride ldg
  const float* G;
  int64_t sG;
  int ldg;
  // dX in the epilogue (wide kernel, ksplit 1, N = 2 d): the product is
  // [P1 | P2] and dX = -x P1 + P2 is stored instead, x of unit u at
  // X + u * sX (row stride ldx), dX row m of unit u at dx row u * dxN + m for
  // m < dxN, as bf16 (dx_bf) or fp32
  void* dx;
  int dx_bf;
  int64_t dxN;
  const float* X;
  int64_t sX;
  int ldx;
  // [a | b] in the epilogue (wide kernel, ksplit 1, N = d_v + 1): the product
  // is [n | d - eps] and a = dO / d, b = -(dO . n) / d^2 are stored instead,
  // dO row u * M + m (d_v wide, bf16 when dO_bf, else fp32)
  const void* dO;
  int dO_bf;
  float eps;
  // the result stored straight into the caller's tensor (wide kernel, ksplit
  // 1, M dividing soNp): global row u * M + m is row r of unit q (soNp rows
  // per unit), written to row q * soN + r when r < soN, N wide, bf16 when
  // so_bf, else fp32
  void* so;
  int so_bf;
  int64_t soN, soNp;
};

constexpr int kGT = 64;                 // output tile
constexpr int kGK = 16;                 // contraction step (a multiple of 16)
constexpr int kGQ = kGK / 16;           // four-element groups per thread and operand
constexpr int kGLD = kGK + 4;           // LDS row stride of [row][k] tiles (floats)
constexpr int kTLD = kGT + 4;           // LDS row stride of [k][row] tiles (floats)
constexpr int kLDS = kGT * kGLD > kGK * kTLD ? kGT * kGLD : kGK * kTLD;

// Row-major A is M x K (TA: stored K x M), B is K x N (TB: stored N x K).
// Four waves, each a 32 x 32 quarter of the 64 x 64 tile as 2 x 2 MFMA tiles.
// An operand whose rows run along k is kept as [row][k] in LDS and a lane
// reads its four contraction values as one 16-byte load; a transposed operand
// (rows along m or n) is kept as it arrives, [k][row], and read as four
// conflict-free 4-byte loads.  Each thread moves kGQ x 4 consecutive elements of
// a row of A and of B per step: 16-byte loads where the operand allows it
// (g.vec bit 0 for A, bit 1 for B: leading dimension, unit stride and base
// 16-byte aligned) and the four are in bounds, else four checked loads; the
// next step's elements are loaded while the current step multiplies.
template <bool TA, bool TB>
__global__ void __launch_bounds__(256) gma_bgemm_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) float As[kLDS];
  __shared__ __attribute__((aligned(16))) float Bs[kLDS];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int r = lane & 15, gq = lane >> 4;
  const int wr = wave >> 1, wc = wave & 1;
  const int n0 = blockIdx.x * kGT, m0 = blockIdx.y * kGT;
  const int u = blockIdx.z / g.ksplit, ks = blockIdx.z % g.ksplit;
  const int kchunk = ((g.K + g.ksplit - 1) / g.ksplit + kGK - 1) / kGK * kGK;
  const int kb = ks * kchunk, ke = min(g.K, kb + kchunk);
  const float* A = g.A + (size_t)u * g.sA;
  const float* B = g.B + (size_t)(g.bmod > 0 ? u % g.bmod : u) * g.sB;
  const bool va = g.vec & 1, vb = (g.vec >> 1) & 1;

  // this thread's kGQ x 4 elements: along k (A: row m; B^T: row n) or along m / n
  constexpr int TPK = 16 / kGQ;                 // threads per k row of a transposed operand
  const int ar = TA ? t / TPK : t >> 2, ac = TA ? (t % TPK) * 4 * kGQ : (t & 3) * 4 * kGQ;
  const int br = TB ? t >> 2 : t / TPK, bc = TB ? (t & 3) * 4 * kGQ : (t % TPK) * 4 * kGQ;
  float ra[4 * kGQ], rb[4 * kGQ];
  // four consecutive elements of a row: p[0..3], valid while idx + e < lim
  auto quad = [](bool vec, const float* p, bool row_ok, int idx, int lim, float* dst) {
    if (vec && row_ok && idx + 3 < lim) {
      const f32x4 v = ld16<f32x4>(p);
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[e] = v[e];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[e] = (row_ok && idx + e < lim) ? p[e] : 0.f;
    }
  };
  auto load = [&](int k0) {
#pragma unroll
    for (int h = 0; h < kGQ; ++h) {
      if (!TA) {                                 // A[m][k], m = m0 + ar, k = k0 + ac + 4h + e
        const int gm = m0 + ar, gk = k0 + ac + 4 * h;
        quad(va, A + (size_t)gm * g.lda + gk, gm < g.M, gk, ke, ra + 4 * h);
      } else {                                   // A[k][m], k = k0 + ar, m = m0 + ac + 4h + e
        const int gk = k0 + ar, gm = m0 + ac + 4 * h;
        quad(va, A + (size_t)gk * g.lda + gm, gk < ke, gm, g.M, ra + 4 * h);
      }
      if (TB) {                                  // B[n][k], n = n0 + br, k = k0 + bc + 4h + e
        const int gn = n0 + br, gk = k0 + bc + 4 * h;
        quad(vb, B + (size_t)gn * g.ldb + gk, gn < g.N, gk, ke, rb + 4 * h);
      } else {                                   // B[k][n], k = k0 + br, n = n0 + bc + 4h + e
        const int gk = k0 + br, gn = n0 + bc + 4 * h;
        quad(vb, B + (size_t)gk * g.ldb + gn, gk < ke, gn, g.N, rb + 4 * h);
      }
    }
  };

  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (kb < ke) load(kb);
  for (int k0 = kb; k0 < ke; k0 += kGK) {
    // stage each operand as its rows arrive: A as [m][k] (or, transposed, as
    // [k][m]) and B as [n][k] (or [k][n]); always 16-byte stores
#pragma unroll
    for (int h = 0; h < kGQ; ++h) {
      const f32x4 va4 = f32x4{ra[4 * h], ra[4 * h + 1], ra[4 * h + 2], ra[4 * h + 3]};
      const f32x4 vb4 = f32x4{rb[4 * h], rb[4 * h + 1], rb[4 * h + 2], rb[4 * h + 3]};
      if (!TA) st16(&As[ar * kGLD + ac + 4 * h], va4);
      else st16(&As[ar * kTLD + ac + 4 * h], va4);
      if (TB) st16(&Bs[br * kGLD + bc + 4 * h], vb4);
      else st16(&Bs[br * kTLD + bc + 4 * h], vb4);
    }
    __syncthreads();
    if (k0 + kGK < ke) load(k0 + kGK);
#pragma unroll
    for (int kk = 0; kk < kGK / 16; ++kk) {
      // lane (r, gq) takes contraction indices 16 kk + 4 gq + e of row r
      f32x4 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int m = 32 * wr + 16 * i + r;
        if (!TA) {
          a[i] = ld16<f32x4>(&As[m * kGLD + 16 * kk + 4 * gq]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) a[i][e] = As[(16 * kk + 4 * gq + e) * kTLD + m];
        }
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = 32 * wc + 16 * j + r;
        if (TB) {
          b[j] = ld16<f32x4>(&Bs[n * kGLD + 16 * kk + 4 * gq]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) b[j][e] = Bs[(16 * kk + 4 * gq + e) * kTLD + n];
        }
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mma(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }

  // D layout: lane (r, gq) holds rows 4 gq + e, column r of each 16 x 16 tile
  float* C;
  int ldc;
  if (g.ksplit > 1) {
    C = g.C + ((size_t)u * g.ksplit + ks) * g.M * g.N;
    ldc = g.N;
  } else {
    C = g.C + (size_t)u * g.sC;
    ldc = g.ldc;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + 32 * wr + 16 * i + 4 * gq + e, n = n0 + 32 * wc + 16 * j + r;
        if (m < g.M && n < g.N) {
          float* c = C + (size_t)m * ldc + n;
          *c = g.accum ? *c + acc[i][j][e] : acc[i][j][e];
        }
      }
}

// The same product for 64 < N <= 16 TN (the augmented widths d + 1 and K):
// one workgroup covers every column of 64 rows, so the left operand is read
// once rather than once per 64 columns.  Four waves of 16 rows x 16 TN columns
// (TN MFMA tiles each); staging and operand reads as in gma_bgemm_kernel.
template <bool TA, bool TB, int TN>
__global__ void __launch_bounds__(256) gma_bgemm_wide_kernel(GemmArgs g) {
  constexpr int BN = 16 * TN;
  constexpr int BLD = BN + 4;                       // [k][n] row stride
  constexpr int BQ = BN * kGK / 4;                  // four-element groups of the B tile
  constexpr int QPT = (BQ + 255) / 256;             // per thread
  __shared__ __attribute__((aligned(16))) float As[kLDS];
  __shared__ __attribute__((aligned(16))) float Bs[(BN * kGLD > kGK * BLD) ? BN * kGLD : kGK * BLD];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int r = lane & 15, gq = lane >> 4;
  const int m0 = blockIdx.y * kGT;
  const int u = blockIdx.z / g.ksplit, ks = blockIdx.z % g.ksplit;
  const int kchunk = ((g.K + g.ksplit - 1) / g.ksplit + kGK - 1) / kGK * kGK;
  const int kb = ks * kchunk, ke = min(g.K, kb + kchunk);
  const float* A = g.A + (size_t)u * g.sA;
  const float* B = g.B + (size_t)(g.bmod > 0 ? u % g.bmod : u) * g.sB;
  const bool va = g.vec & 1, vb = (g.vec >> 1) & 1;

  constexpr int TPK = 16 / kGQ;
  const int ar = TA ? t / TPK : t >> 2, ac = TA ? (t % TPK) * 4 * kGQ : (t & 3) * 4 * kGQ;
  float ra[4 * kGQ], rb[4 * QPT];
  auto quad = [](bool vec, const float* p, bool row_ok, int idx, int lim, float* dst) {
    if (vec && row_ok && idx + 3 < lim) {
      const f32x4 v = ld16<f32x4>(p);
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[e] = v[e];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[e] = (row_ok && idx + e < lim) ? p[e] : 0.f;
    }
  };
  // B group q: TB -> row n = q / (kGK / 4), k = 4 (q % (kGK / 4));
  //            else -> k = q / (BN / 4), n = 4 (q % (BN / 4))
  auto bq_row = [](int q) { return TB ? q / (kGK / 4) : q / (BN / 4); };
  auto bq_col = [](int q) { return TB ? 4 * (q % (kGK / 4)) : 4 * (q % (BN / 4)); };
  auto load = [&](int k0) {
#pragma unroll
    for (int h = 0; h < kGQ; ++h) {
      if (!TA) {
        const int gm = m0 + ar, gk = k0 + ac + 4 * h;
        quad(va, A + (size_t)gm * g.lda + gk, gm < g.M, gk, ke, ra + 4 * h);
      } else {
        const int gk = k0 + ar, gm = m0 + ac + 4 * h;
        quad(va, A + (size_t)gk * g.lda + gm, gk < ke, gm, g.M, ra + 4 * h);
      }
    }
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
      const int q = t + 256 * j;
      if (q >= BQ) break;
      if (TB) {
        const int gn = bq_row(q), gk = k0 + bq_col(q);
        quad(vb, B + (size_t)gn * g.ldb + gk, gn < g.N, gk, ke, rb + 4 * j);
      } else {
        const int gk = k0 + bq_row(q), gn = bq_col(q);
        quad(vb, B + (size_t)gk * g.ldb + gn, gk < ke, gn, g.N, rb + 4 * j);
      }
    }
  };

  f32x4 acc[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // the epilogue's other input for this lane's elements (dO for [a | b], x
  // for dX, G for the softmax Jacobian), requested before the main loop so
  // that it arrives while the loop runs
  float gv[TN][4];
  if (g.dO) {
    // dO of this lane's columns below d_v
    const int dvv = g.N - 1;
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + 16 * wave + 4 * gq + e, n = 16 * j + r;
        const size_t i = ((size_t)u * g.M + m) * dvv + n;
        const bool ok = m < g.M && n < dvv;
        gv[j][e] = !ok ? 0.f
                       : (g.dO_bf ? (float)static_cast<const bf16*>(g.dO)[i]
                                  : static_cast<const float*>(g.dO)[i]);
      }
  } else if (g.dx) {
    // x of this lane's P1 columns (tiles j < TN / 2)
    const float* Xu = g.X + (size_t)u * g.sX;
#pragma unroll
    for (int j = 0; j < TN / 2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + 16 * wave + 4 * gq + e, n = 16 * j + r;
        gv[j][e] = m < g.M && n < g.N / 2 ? Xu[(size_t)m * g.ldx + n] : 0.f;
      }
  } else if (g.G) {
    const float* Gu = g.G + (size_t)u * g.sG;
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + 16 * wave + 4 * gq + e, n = 16 * j + r;
        gv[j][e] = m < g.M && n < g.N ? Gu[(size_t)m * g.ldg + n] : 0.f;
      }
  }

  if (kb < ke) load(kb);
  for (int k0 = kb; k0 < ke; k0 += kGK) {
#pragma unroll
    for (int h = 0; h < kGQ; ++h) {
      const f32x4 va4 = f32x4{ra[4 * h], ra[4 * h + 1], ra[4 * h + 2], ra[4 * h + 3]};
      if (!TA) st16(&As[ar * kGLD + ac + 4 * h], va4);
      else st16(&As[ar * kTLD + ac + 4 * h], va4);
    }
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
      const int q = t + 256 * j;
      if (q >= BQ) break;
      const f32x4 vb4 = f32x4{rb[4 * j], rb[4 * j + 1], rb[4 * j + 2], rb[4 * j + 3]};
      if (TB) st16(&Bs[bq_row(q) * kGLD + bq_col(q)], vb4);
      else st16(&Bs[bq_row(q) * BLD + bq_col(q)], vb4);
    }
    __syncthreads();
    if (k0 + kGK < ke) load(k0 + kGK);
#pragma unroll
    for (int kk = 0; kk < kGK / 16; ++kk) {
      f32x4 a;
      const int m = 16 * wave + r;
      if (!TA) {
        a = ld16<f32x4>(&As[m * kGLD + 16 * kk + 4 * gq]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) a[e] = As[(16 * kk + 4 * gq + e) * kTLD + m];
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = 16 * j + r;
        f32x4 b;
        if (TB) {
          b = ld16<f32x4>(&Bs[n * kGLD + 16 * kk + 4 * gq]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) b[e] = Bs[(16 * kk + 4 * gq + e) * BLD + n];
        }
        acc[j] = mma(a, b, acc[j]);
      }
    }
    __syncthreads();
  }

  float* C;
  int ldc;
  if (g.ksplit > 1) {
    C = g.C + ((size_t)u * g.ksplit + ks) * g.M * g.N;
    ldc = g.N;
  } else {
    C = g.C + (size_t)u * g.sC;
    ldc = g.ldc;
  }
  if (g.so) {
    // M divides Np (whole units, or 64-row chunks of them): the unit and the
    // first row follow from u alone
    const int64_t base = (int64_t)u * g.M, q = base / g.soNp, r0 = base - q * g.soNp;
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + 16 * wave + 4 * gq + e, n = 16 * j + r;
        if (m < g.M && n < g.N) {
          const float v = (g.accum ? C[(size_t)m * ldc + n] : 0.f) + acc[j][e];
          const int64_t rr = r0 + m;
          if (rr < g.soN) {
            const size_t i = (size_t)(q * g.soN + rr) * g.N + n;
            if (g.so_bf) static_cast<bf16*>(g.so)[i] = to_bf16(v);
            else static_cast<float*>(g.so)[i] = v;
          }
        }
      }
    return;
  }
  if (g.dO) {
    // [a | b] = [dO / d | -(dO . o) / d], o = n / d (the output's gradient
    // through Eq. 7): d is column d_v of the row (lane r = d_v mod 16 of tile
    // d_v / 16), dO . n a row sum, both over the 16-lane DPP row
    const int dvv = g.N - 1;
    float nv[TN][4];
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + 16 * wave + 4 * gq + e, n = 16 * j + r;
        const bool ok = m < g.M && n < g.N;
        const float prev = ok && g.accum ? C[(size_t)m * ldc + n] : 0.f;
        nv[j][e] = ok ? prev + acc[j][e] : 0.f;
      }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float dp = 0.f, dt = 0.f;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = 16 * j + r;
        dp += n == dvv ? nv[j][e] : 0.f;
        dt += n < dvv ? gv[j][e] * nv[j][e] : 0.f;
      }
      const float den = row16_sum(dp) + g.eps;
      const float dot = row16_sum(dt);
      const float inv = 1.f / den;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int m = m0 + 16 * wave + 4 * gq + e, n = 16 * j + r;
        if (m < g.M && n <= dvv) C[(size_t)m * ldc + n] = n < dvv ? gv[j][e] * inv : -dot * inv * inv;
      }
    }
    return;
  }
  if (g.dx) {
    // dX = -x P1 + P2 ("Gradient structure": the score's routing-vector
    // gradient): P1 in tiles j, P2 in tiles j + TN / 2 of the same lane
    const int d = g.N / 2;
#pragma unroll
    for (int j = 0; j < TN / 2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + 16 * wave + 4 * gq + e, n = 16 * j + r;
        if (m < g.M && m < g.dxN && n < d) {
          const float v = acc[j + TN / 2][e] - gv[j][e] * acc[j][e];
          const size_t i = ((size_t)u * g.dxN + m) * d + n;
          if (g.dx_bf) static_cast<bf16*>(g.dx)[i] = to_bf16(v);
          else static_cast<float*>(g.dx)[i] = v;
        }
      }
    return;
  }
  if (g.G) {
    // dS = G (dG - sum_l G_l dG_l) ("Gradient structure", Eq. 18): a row's
    // columns 16 j + r lie in this lane's TN tiles and the 16 lanes of its
    // DPP row, so the row sum is an in-lane sum and a 16-lane butterfly
    float dv[TN][4];
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + 16 * wave + 4 * gq + e, n = 16 * j + r;
        const bool ok = m < g.M && n < g.N;
        const float prev = ok && g.accum ? C[(size_t)m * ldc + n] : 0.f;
        dv[j][e] = ok ? prev + acc[j][e] : 0.f;
      }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < TN; ++j) sum += gv[j][e] * dv[j][e];
      sum = row16_sum(sum);
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int m = m0 + 16 * wave + 4 * gq + e, n = 16 * j + r;
        if (m < g.M && n < g.N) C[(size_t)m * ldc + n] = gv[j][e] * (dv[j][e] - sum);
      }
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = m0 + 16 * wave + 4 * gq + e, n = 16 * j + r;
      if (m < g.M && n < g.N) {
        float* c = C + (size_t)m * ldc + n;
        *c = g.accum ? *c + acc[j][e] : acc[j][e];
      }
    }
}

// C[u][m][n] = sum over the splits, in split order.
__global__ void __launch_bounds__(256) gma_split_sum_kernel(const float* __restrict__ part,
                                                            int ksplit, int M, int N,
                                                            float* __restrict__ C, int ldc,
                                                            int64_t sC) {
  const int u = blockIdx.y;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= M * N) return;
  const float* p = part + (size_t)u * ksplit * M * N + i;
  const size_t st = (size_t)M * N;
  float s = 0.f;
  // eight splits' loads in flight before they are added, in split order
  int k = 0;
  for (; k + 8 <= ksplit; k += 8) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = p[(size_t)(k + j) * st];
#pragma unroll
    for (int j = 0; j < 8; ++j) s += v[j];
  }
  for (; k < ksplit; ++k) s += p[(size_t)k * st];
  C[(size_t)u * sC + (size_t)(i / N) * ldc + i % N] = s;
}

template <class T>
__device__ __forceinline__ float ldx(const void* p, size_t i) {
  return (float)static_cast<const T*>(p)[i];
}
template <class T>
__device__ __forceinline__ void stx(void* p, size_t i, float v) {
  static_cast<T*>(p)[i] = (T)v;
}

// Per token: X3 = [x | x^2 | 1] for a routing vector, and (values) V1 = [v | 1],
// rows of stride ld (= width + 3; the pad columns after the ones are zero).
// d / 4 threads per row, four elements each, 16-byte stores.
__device__ __forceinline__ f32x4 load4x(const bf16* p) {
  const bf16x4 v = *reinterpret_cast<const bf16x4*>(__builtin_assume_aligned(p, 8));
  return f32x4{from_bf16(v[0]), from_bf16(v[1]), from_bf16(v[2]), from_bf16(v[3])};
}
__device__ __forceinline__ f32x4 load4x(const float* p) { return ld16<f32x4>(p); }

template <class T>
__global__ void __launch_bounds__(256) gma_bwd_prep_kernel(const void* __restrict__ x, int d,
                                                           int squares, int64_t rows, int ld,
                                                           float* __restrict__ out) {
  const int tpr = d / 4, rpb = 256 / tpr;
  const int j = threadIdx.x % tpr;
  for (int64_t row = (int64_t)blockIdx.x * rpb + threadIdx.x / tpr; row < rows;
       row += (int64_t)gridDim.x * rpb) {
    const f32x4 v = load4x(static_cast<const T*>(x) + (size_t)row * d + 4 * j);
    float* o = out + (size_t)row * ld;
    st16(o + 4 * j, v);
    if (squares) st16(o + d + 4 * j, v * v);
    if (j == 0) st16(o + (squares ? 2 * d : d), f32x4{1.f, 0.f, 0.f, 0.f});
  }
}

// Per head: WW = [w | mu w], w = exp(-log sigma^2), as [K][2 d_r].
__global__ void __launch_bounds__(256) gma_bwd_params_kernel(const float* __restrict__ mu,
                                                             const float* __restrict__ ls2,
                                                             int64_t n, int d,
                                                             float* __restrict__ ww) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int64_t row = i / d;
  const int c = (int)(i - row * d);
  const float w = expf(-ls2[i]);
  ww[row * 2 * d + c] = w;
  ww[row * 2 * d + d + c] = mu[i] * w;
}

// One wave per token: dS = G (dG - sum_l G_l dG_l), in place on dG.
__global__ void __launch_bounds__(256) gma_bwd_softmax_kernel(const float* __restrict__ G,
                                                              float* __restrict__ dG, int K,
                                                              int64_t rows) {
  const int lane = threadIdx.x & 63;
  for (int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); row < rows;
       row += (int64_t)gridDim.x * 4) {
  const float* gr = G + (size_t)row * K;
  float* dr = dG + (size_t)row * K;
  float s = 0.f;
  for (int k = lane; k < K; k += 64) s += gr[k] * dr[k];
  s = groups_sum(row16_sum(s));
  for (int k = lane; k < K; k += 64) dr[k] = gr[k] * (dr[k] - s);
  }
}

// The same for K a multiple of 4 (rows 16-byte aligned), K <= 64 M: one
// 16-lane row per token, four tokens per wave, no loop; lane j holds elements
// 4 j + 64 m (m < M) as 16-byte vectors, so every load of a token is issued
// before its sum is formed.
template <int M>
__global__ void __launch_bounds__(256) gma_bwd_softmax16_kernel(const float* __restrict__ G,
                                                                float* __restrict__ dG, int K,
                                                                int64_t rows) {
  const int j = threadIdx.x & 15;
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  if (row >= rows) return;     // whole 16-lane rows leave together
  const float* gr = G + (size_t)row * K;
  float* dr = dG + (size_t)row * K;
  f32x4 g[M], d[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int c = 4 * j + 64 * m;
    if (c < K) {
      g[m] = ld16<f32x4>(gr + c);
      d[m] = ld16<f32x4>(dr + c);
    } else {
      g[m] = f32x4{0.f, 0.f, 0.f, 0.f};
      d[m] = g[m];
    }
  }
  float s = 0.f;
#pragma unroll
  for (int m = 0; m < M; ++m) s += g[m][0] * d[m][0] + g[m][1] * d[m][1] + g[m][2] * d[m][2] + g[m][3] * d[m][3];
  s = row16_sum(s);
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int c = 4 * j + 64 * m;
    if (c < K) st16(dr + c, g[m] * (d[m] - s));
  }
}

// dX = -x P1 + P2 from X3 = [x | x^2 | 1] and P = [P1 | P2].
// Rows are padded to Np per unit (Np = N without padding); row r of unit u
// goes to row u * N + r of the caller's tensor when r < N.  Four consecutive
// elements per thread.
template <class T>
__device__ __forceinline__ void store4x(void* p, size_t i, f32x4 v) {
#pragma unroll
  for (int e = 0; e < 4; ++e) stx<T>(p, i + e, v[e]);
}

template <class T>
__global__ void __launch_bounds__(256) gma_bwd_dx_kernel(const float* __restrict__ x3, int ld,
                                                         const float* __restrict__ P, int d,
                                                         int64_t rows, int64_t Np, int64_t N,
                                                         void* __restrict__ dx) {
  const int q = d / 4;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < rows * q;
       i += (int64_t)gridDim.x * 256) {
    const int64_t row = i / q;
    const int c = 4 * (int)(i - row * q);
    const int64_t u = row / Np, r = row - u * Np;
    if (r >= N) continue;
    const float* p = P + (size_t)row * 2 * d;
    const f32x4 xv = ld16<f32x4>(x3 + (size_t)row * ld + c);
    const f32x4 p1 = ld16<f32x4>(p + c), p2 = ld16<f32x4>(p + d + c);
    store4x<T>(dx, (size_t)(u * N + r) * d + c, p2 - xv * p1);
  }
}

// [U][N][d] -> [U][Np][d], rows N..Np-1 zero.
template <class T>
__global__ void __launch_bounds__(256) gma_bwd_pad_kernel(const void* __restrict__ src, int d,
                                                          int64_t U, int64_t Np, int64_t N,
                                                          void* __restrict__ dst) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < U * Np * d;
       i += (int64_t)gridDim.x * 256) {
    const int64_t row = i / d;
    const int c = (int)(i - row * d);
    const int64_t u = row / Np, r = row - u * Np;
    static_cast<T*>(dst)[i] =
        r < N ? static_cast<const T*>(src)[(size_t)(u * N + r) * d + c] : (T)0.f;
  }
}

// Exclusive scan over the nc chunk records of each unit (reverse: over the
// later chunks), in place; records of n floats.
__global__ void __launch_bounds__(256) gma_bwd_chunk_scan_kernel(float* __restrict__ x, int nc,
                                                                 int n, int reverse) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= n) return;
  float* base = x + (size_t)blockIdx.y * nc * n + e;
  float run = 0.f;
  // eight records read before their exclusive sums overwrite them (each
  // element belongs to this thread alone), summed in scan order
  int i = 0;
  for (; i + 8 <= nc; i += 8) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = reverse ? nc - 1 - (i + j) : i + j;
      v[j] = base[(size_t)c * n];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = reverse ? nc - 1 - (i + j) : i + j;
      base[(size_t)c * n] = run;
      run += v[j];
    }
  }
  for (; i < nc; ++i) {
    const int c = reverse ? nc - 1 - i : i;
    const float v = base[(size_t)c * n];
    base[(size_t)c * n] = run;
    run += v;
  }
}

// Chunk-local masks on [Z][64][64]: lower keeps column <= row (key j <= query
// i), upper keeps column >= row (query i >= key j).
__global__ void __launch_bounds__(256) gma_bwd_mask_kernel(float* __restrict__ m, int64_t n,
                                                           int upper) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * 256) {
    const int r = (int)((i >> 6) & 63), c = (int)(i & 63);
    if (upper ? c < r : c > r) m[i] = 0.f;
  }
}

// Per head: sum R = [R1 | R2 | r0] over batches and over queries and keys,
// then the parameter gradients.
__global__ void __launch_bounds__(256) gma_bwd_param_grad_kernel(
    const float* __restrict__ Rq, const float* __restrict__ Rk, int64_t B, int H, int K, int d,
    int W,
    const float* __restrict__ mu, const float* __restrict__ ls2, float* __restrict__ dmu,
    float* __restrict__ dls2, float* __restrict__ dlpi) {
  const int h = blockIdx.y;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= K * d) return;
  const int k = i / d, c = i - k * d;
  double r1 = 0.0, r2 = 0.0, r0 = 0.0;
  for (int src = 0; src < 2; ++src) {
    const float* R = src ? Rk : Rq;
    for (int64_t b = 0; b < B; ++b) {
      const float* row = R + ((size_t)(b * H + h) * K + k) * W;
      r1 += row[c];
      r2 += row[d + c];
      r0 += row[2 * d];
    }
  }
  const size_t pi = (size_t)h * K * d + i;
  const double m = mu[pi], w = exp(-(double)ls2[pi]);
  dmu[pi] = (float)(w * (r1 - m * r0));
  dls2[pi] = (float)(0.5 * w * (r2 - 2.0 * m * r1 + m * m * r0) - 0.5 * r0);
  if (c == 0) dlpi[(size_t)h * K + k] = (float)r0;
}

// Forward on the product path: O = n / (d + eps) from the [n | d - eps] rows,
// stored at the unpadded position in the output type.
template <class T>
__global__ void __launch_bounds__(256) gma_prod_out_kernel(const float* __restrict__ nd, int dv,
                                                           int ld, float eps, int64_t rows,
                                                           int64_t Np, int64_t N,
                                                           void* __restrict__ out) {
  const int q = dv / 4;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < rows * q;
       i += (int64_t)gridDim.x * 256) {
    const int64_t row = i / q;
    const int c = 4 * (int)(i - row * q);
    const int64_t u = row / Np, r = row - u * Np;
    if (r < N) {
      const float* src = nd + (size_t)row * ld;
      const float inv = 1.f / (src[dv] + eps);
      store4x<T>(out, (size_t)(u * N + r) * dv + c, ld16<f32x4>(src + c) * inv);
    }
  }
}

// [U][Np] int32 -> [U][N].
__global__ void __launch_bounds__(256) gma_prod_assign_kernel(const int32_t* __restrict__ src,
                                                              int64_t U, int64_t Np, int64_t N,
                                                              int32_t* __restrict__ dst) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < U * N;
       i += (int64_t)gridDim.x * 256) {
    const int64_t u = i / N, r = i - u * N;
    dst[i] = src[u * Np + r];
  }
}

}  // namespace

// ---- host ------------------------------------------------------------------
namespace {

size_t r256(size_t x) { return (x + 255) & ~(size_t)255; }
constexpr int kChunk = 64;                  // causal chunk (one product tile)

// The backward runs on rows padded to Np per unit: Np = N (bidirectional) or
// N rounded up to the chunk (causal; zero rows at the end of a sequence affect
// no earlier position, and their dO is zero).  pp is the plan at Np.
struct BwdLayout {
  int64_t Np = 0, nc = 0;
  size_t pads, x3q, x3k, v1, nd, gq, gk, dgq, dgk, p, dv, vtz, dvtz, rq, rk, ww, part;
  size_t pc, qc, total;
  int ks_tok;        // split of the token contractions
};

BwdLayout bwd_layout(const Plan& pp, bool causal, int64_t N) {
  BwdLayout L{};
  L.Np = pp.N;
  L.nc = causal ? pp.N / kChunk : 0;
  const size_t U = (size_t)pp.BH, Np = (size_t)pp.N, K = (size_t)pp.K;
  const size_t dr = pp.DR, dv = pp.DV, es = pp.bf ? 2 : 4;
  int ks = (int)((1024 + U - 1) / U);
  const int maxk = (int)((pp.N + 255) / 256);      // at least 256 tokens per split
  if (ks > maxk) ks = maxk;
  if (ks > 32) ks = 32;
  if ((int64_t)ks * pp.BH > 65535) ks = (int)(65535 / pp.BH);
  if (ks < 1) ks = 1;
  L.ks_tok = ks;
  size_t off = r256(pp.total);
  auto take = [&](size_t bytes) { const size_t o = off; off += r256(bytes); return o; };
  const size_t w3p = 2 * dr + 4, w1p = dv + 4;      // padded row strides
  // causal: padded copies of Q_X, K_X, V_X, dO in the input type
  L.pads = take(causal && (int64_t)Np != N ? U * Np * (2 * dr + 2 * dv) * es : 0);
  L.x3q = take(U * Np * w3p * 4);
  L.x3k = take(U * Np * w3p * 4);
  L.v1 = take(U * Np * w1p * 4);
  L.nd = take(U * Np * w1p * 4);
  L.gq = take(U * Np * K * 4);
  L.gk = take(U * Np * K * 4);
  L.dgq = take(U * Np * K * 4);
  L.dgk = take(U * Np * K * 4);
  L.p = take(U * Np * 2 * dr * 4);
  L.dv = take(U * Np * dv * 4);
  // [V~ | Z] and [dV~ | dZ] per unit, or per chunk (causal: the carried prefix
  // and suffix states)
  const size_t recs = causal ? U * (size_t)L.nc : U;
  L.vtz = take(recs * K * w1p * 4);
  L.dvtz = take(recs * K * w1p * 4);
  L.rq = take(U * K * w3p * 4);
  L.rk = take(U * K * w3p * 4);
  L.ww = take((size_t)pp.H * K * 2 * dr * 4);
  const size_t wmax = (2 * dr + 1) > (dv + 1) ? (2 * dr + 1) : (dv + 1);
  L.part = take(U * (size_t)ks * K * wmax * 4);
  L.pc = take(causal ? recs * kChunk * kChunk * 4 : 0);
  L.qc = take(causal ? recs * kChunk * kChunk * 4 : 0);
  L.total = off;
  return L;
}

// wide: 0 (64 x 64 tiles), 4, 8 or 9 (one column tile of 16 wide columns)
template <bool TA, bool TB>
void launch_gemm_kernel(int wide, dim3 grid, const GemmArgs& g, hipStream_t s) {
  if (!wide) hipLaunchKernelGGL((gma_bgemm_kernel<TA, TB>), grid, dim3(256), 0, s, g);
  else if (wide == 4) hipLaunchKernelGGL((gma_bgemm_wide_kernel<TA, TB, 4>), grid, dim3(256), 0, s, g);
  else if (wide == 8) hipLaunchKernelGGL((gma_bgemm_wide_kernel<TA, TB, 8>), grid, dim3(256), 0, s, g);
  else hipLaunchKernelGGL((gma_bgemm_wide_kernel<TA, TB, 9>), grid, dim3(256), 0, s, g);
}

// Whether gemm() can apply the softmax Jacobian of a result of width N in its
// epilogue (one column tile).
bool gemm_jacobian_ok(int N) { return N <= 144; }

// The dX epilogue: P = [P1 | P2] of width N = 2 d in one column tile whose
// halves are whole MFMA tiles (d of 32 or 64).
bool gemm_dx_ok(int N) { return N == 64 || N == 128; }

struct DxOut {
  void* dx = nullptr;
  int bf = 0;
  int64_t N = 0;
  const float* X = nullptr;
  int64_t sX = 0;
  int ldx = 0;
};
// A result stored straight into a caller's [units][N][width] tensor from
// padded rows (Np per unit).
struct StoreOut {
  void* dst = nullptr;
  int bf = 0;
  int64_t N = 0, Np = 0;
};

hipError_t gemm(bool ta, bool tb, const float* A, int lda, int64_t sA, const float* B, int ldb,
                int64_t sB, int bmod, float* C, int ldc, int64_t sC, int M, int N, int K,
                int64_t U, int ksplit, float* part, hipStream_t s, bool accum = false,
                const float* G = nullptr, int64_t sG = 0, int ldg = 0,
                const DxOut* dxo = nullptr, const void* dO = nullptr, int dO_bf = 0,
                float eps = 0.f, const StoreOut* so = nullptr) {
  if (so && (ksplit > 1 || G || dxo || dO || N > 144 || so->Np % M)) return hipErrorInvalidValue;
  if (G && (ksplit > 1 || !gemm_jacobian_ok(N))) return hipErrorInvalidValue;
  if (dxo && (ksplit > 1 || accum || G || !gemm_dx_ok(N))) return hipErrorInvalidValue;
  if (dO && (ksplit > 1 || G || dxo || N > 144)) return hipErrorInvalidValue;
  const int vec = ((lda % 4 == 0 && sA % 4 == 0 && ((uintptr_t)A & 15) == 0) ? 1 : 0) |
                  ((ldb % 4 == 0 && sB % 4 == 0 && ((uintptr_t)B & 15) == 0) ? 2 : 0);
  GemmArgs g{A, B, ksplit > 1 ? part : C, M, N, K, lda, ldb, ldc, sA, sB, sC, bmod, ksplit, vec,
             accum ? 1 : 0, G, sG, ldg};
  g.dO = dO;
  g.dO_bf = dO_bf;
  g.eps = eps;
  if (so) {
    g.so = so->dst;
    g.so_bf = so->bf;
    g.soN = so->N;
    g.soNp = so->Np;
  }
  if (dxo) {
    g.dx = dxo->dx;
    g.dx_bf = dxo->bf;
    g.dxN = dxo->N;
    g.X = dxo->X;
    g.sX = dxo->sX;
    g.ldx = dxo->ldx;
  }
  // 64 < N <= 144: one column tile of 128 (8 MFMA tiles per wave) or 144 (9);
  // with an epilogue that needs whole rows also N <= 64 (4)
  const int wide = N > 128 && N <= 144 ? 9 : (N > kGT && N <= 128 ? 8 : (G || dxo || dO || so ? 4 : 0));
  const dim3 grid(wide ? 1u : (unsigned)((N + kGT - 1) / kGT), (unsigned)((M + kGT - 1) / kGT),
                  (unsigned)(U * ksplit));
  if (!ta && !tb) launch_gemm_kernel<false, false>(wide, grid, g, s);
  else if (!ta && tb) launch_gemm_kernel<false, true>(wide, grid, g, s);
  else if (ta && !tb) launch_gemm_kernel<true, false>(wide, grid, g, s);
  else launch_gemm_kernel<true, true>(wide, grid, g, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ksplit <= 1) return e;
  hipLaunchKernelGGL(gma_split_sum_kernel, dim3((unsigned)((M * N + 255) / 256), (unsigned)U),
                     dim3(256), 0, s, part, ksplit, M, N, C, ldc, sC);
  return hipGetLastError();
}

unsigned blocks(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }
// striding kernels: at most eight workgroups per compute unit
unsigned sblocks(int64_t n, int per) {
  const int64_t b = (n + per - 1) / per;
  return (unsigned)(b < 16384 ? b : 16384);
}

static void launch_bwd_softmax(const float* G, float* dG, int K, int64_t rows, hipStream_t s) {
  if (K % 4 == 0 && K <= 128) {
    const dim3 grid((unsigned)((rows + 15) / 16));
    if (K <= 64)
      hipLaunchKernelGGL(gma_bwd_softmax16_kernel<1>, grid, dim3(256), 0, s, G, dG, K, rows);
    else
      hipLaunchKernelGGL(gma_bwd_softmax16_kernel<2>, grid, dim3(256), 0, s, G, dG, K, rows);
    return;
  }
  hipLaunchKernelGGL(gma_bwd_softmax_kernel, dim3(sblocks(rows, 4)), dim3(256), 0, s, G, dG, K,
                     rows);
}

template <class T>
hipError_t run_backward(const Plan& pp, const Tensors& t0, const BwdTensors& gt, bool causal,
                        int64_t N0, hipStream_t s) {
  const BwdLayout L = bwd_layout(pp, causal, N0);
  Tensors t = t0;
  char* ws = t.ws;
  float* x3q = reinterpret_cast<float*>(ws + L.x3q);
  float* x3k = reinterpret_cast<float*>(ws + L.x3k);
  float* v1 = reinterpret_cast<float*>(ws + L.v1);
  float* nd = reinterpret_cast<float*>(ws + L.nd);
  float* Gq = reinterpret_cast<float*>(ws + L.gq);
  float* Gk = reinterpret_cast<float*>(ws + L.gk);
  float* dGq = reinterpret_cast<float*>(ws + L.dgq);
  float* dGk = reinterpret_cast<float*>(ws + L.dgk);
  float* P = reinterpret_cast<float*>(ws + L.p);
  float* dvf = reinterpret_cast<float*>(ws + L.dv);
  float* vtz = reinterpret_cast<float*>(ws + L.vtz);
  float* dvtz = reinterpret_cast<float*>(ws + L.dvtz);
  float* Rq = reinterpret_cast<float*>(ws + L.rq);
  float* Rk = reinterpret_cast<float*>(ws + L.rk);
  float* WW = reinterpret_cast<float*>(ws + L.ww);
  float* part = reinterpret_cast<float*>(ws + L.part);
  float* pc = reinterpret_cast<float*>(ws + L.pc);
  float* qc = reinterpret_cast<float*>(ws + L.qc);
  const int64_t U = pp.BH, Np = L.Np, rows = U * Np;
  const int K = pp.K, dr = pp.DR, dv = pp.DV, ks = L.ks_tok;
  const int w3 = 2 * dr + 1, w1 = dv + 1;           // logical widths
  const int l3 = 2 * dr + 4, l1 = dv + 4;           // row strides (multiples of 4)
  const void* dO = gt.dO;
  hipError_t e;
#define GMA_CHECK(x) do { e = (x); if (e != hipSuccess) return e; } while (0)
  if (L.pads && Np != N0) {
    // causal with a ragged last chunk: zero-padded copies of the inputs
    T* pq = reinterpret_cast<T*>(ws + L.pads);
    T* pk = pq + (size_t)rows * dr;
    T* pv = pk + (size_t)rows * dr;
    T* pd = pv + (size_t)rows * dv;
    if (g_launch_hook) g_launch_hook("gma_bwd_prep", s, 1);
    hipLaunchKernelGGL(gma_bwd_pad_kernel<T>, dim3(sblocks(rows * dr, 256)), dim3(256), 0, s, t.q,
                       dr, U, Np, N0, (void*)pq);
    hipLaunchKernelGGL(gma_bwd_pad_kernel<T>, dim3(sblocks(rows * dr, 256)), dim3(256), 0, s, t.k,
                       dr, U, Np, N0, (void*)pk);
    hipLaunchKernelGGL(gma_bwd_pad_kernel<T>, dim3(sblocks(rows * dv, 256)), dim3(256), 0, s, t.v,
                       dv, U, Np, N0, (void*)pv);
    hipLaunchKernelGGL(gma_bwd_pad_kernel<T>, dim3(sblocks(rows * dv, 256)), dim3(256), 0, s, dO,
                       dv, U, Np, N0, (void*)pd);
    GMA_CHECK(hipGetLastError());
    if (g_launch_hook) g_launch_hook("gma_bwd_prep", s, 0);
    t.q = pq;
    t.k = pk;
    t.v = pv;
    dO = pd;
  }
  // responsibilities of queries and keys
  Tensors tr = t;
  tr.assign_q = nullptr;
  tr.q = t.q;
  tr.gamma = Gq;
  GMA_CHECK(launch_resp(pp, tr, s));
  tr.q = t.k;
  tr.gamma = Gk;
  GMA_CHECK(launch_resp(pp, tr, s));
  if (g_launch_hook) g_launch_hook("gma_bwd_prep", s, 1);
  hipLaunchKernelGGL(gma_bwd_prep_kernel<T>, dim3(sblocks(rows, 1024 / dr)), dim3(256), 0, s, t.q,
                     dr, 1, rows, l3, x3q);
  hipLaunchKernelGGL(gma_bwd_prep_kernel<T>, dim3(sblocks(rows, 1024 / dr)), dim3(256), 0, s, t.k,
                     dr, 1, rows, l3, x3k);
  hipLaunchKernelGGL(gma_bwd_prep_kernel<T>, dim3(sblocks(rows, 1024 / dv)), dim3(256), 0, s, t.v,
                     dv, 0, rows, l1, v1);
  hipLaunchKernelGGL(gma_bwd_params_kernel, dim3(blocks(pp.H * K * dr, 256)), dim3(256), 0, s,
                     t.mu, t.ls2, pp.H * K * (int64_t)dr, dr, WW);
  GMA_CHECK(hipGetLastError());
  if (g_launch_hook) g_launch_hook("gma_bwd_prep", s, 0);

  const int64_t Z = causal ? U * L.nc : U;      // product batch: units, or chunks
  const int C = kChunk;
  // the softmax Jacobian in the epilogue of the products giving dGq and dGk
  // where one column tile holds a row of K
  const bool jac = gemm_jacobian_ok(K);
  // dV goes to the caller's tensor from the epilogue of its (last) product
  StoreOut dvo;
  dvo.dst = gt.dV;
  dvo.bf = sizeof(T) == 2;
  dvo.N = N0;
  dvo.Np = Np;
  if (!causal) {
    if (g_launch_hook) g_launch_hook("gma_bwd_gemm", s, 1);
    // [V~ | Z] = Gk^T [V | 1]
    GMA_CHECK(gemm(true, false, Gk, K, Np * K, v1, l1, Np * l1, 0, vtz, l1, (int64_t)K * l1, K,
                   w1, (int)Np, U, ks, part, s));
    // [n | d - eps] = Gq [V~ | Z], turned into [a | b] in the epilogue
    GMA_CHECK(gemm(false, false, Gq, K, Np * K, vtz, l1, (int64_t)K * l1, 0, nd, l1, Np * l1,
                   (int)Np, w1, K, U, 1, part, s, false, nullptr, 0, 0, nullptr, dO,
                   sizeof(T) == 2, t.eps));
    if (g_launch_hook) g_launch_hook("gma_bwd_gemm", s, 0);
  } else {
    if (g_launch_hook) g_launch_hook("gma_bwd_gemm", s, 1);
    // per chunk: [V~ | Z] totals, then their exclusive prefix over chunks
    GMA_CHECK(gemm(true, false, Gk, K, (int64_t)C * K, v1, l1, (int64_t)C * l1, 0, vtz, l1,
                   (int64_t)K * l1, K, w1, C, Z, 1, part, s));
    hipLaunchKernelGGL(gma_bwd_chunk_scan_kernel, dim3(blocks((int64_t)K * l1, 256), (unsigned)U),
                       dim3(256), 0, s, vtz, (int)L.nc, K * l1, 0);
    GMA_CHECK(hipGetLastError());
    // in-chunk affinity Gq_c Gk_c^T, keys j <= query i
    GMA_CHECK(gemm(false, true, Gq, K, (int64_t)C * K, Gk, K, (int64_t)C * K, 0, pc, C,
                   (int64_t)C * C, C, C, K, Z, 1, part, s));
    hipLaunchKernelGGL(gma_bwd_mask_kernel, dim3(sblocks(Z * C * C, 256)), dim3(256), 0, s, pc,
                       Z * C * C, 0);
    GMA_CHECK(hipGetLastError());
    // [n | d - eps] = Gq_c [V~ | Z]_prefix + mask(Gq_c Gk_c^T) [V | 1]_c
    GMA_CHECK(gemm(false, false, Gq, K, (int64_t)C * K, vtz, l1, (int64_t)K * l1, 0, nd, l1,
                   (int64_t)C * l1, C, w1, K, Z, 1, part, s));
    GMA_CHECK(gemm(false, false, pc, C, (int64_t)C * C, v1, l1, (int64_t)C * l1, 0, nd, l1,
                   (int64_t)C * l1, C, w1, C, Z, 1, part, s, true, nullptr, 0, 0, nullptr, dO,
                   sizeof(T) == 2, t.eps));
    if (g_launch_hook) g_launch_hook("gma_bwd_gemm", s, 0);
  }
  // [a | b] = [dO / d | -(dO . o) / d] was formed in the epilogue of the last
  // product giving [n | d - eps] (d_v + 1 <= 129 columns: one column tile)
  if (g_launch_hook) g_launch_hook("gma_bwd_gemm", s, 1);
  if (!causal) {
    // dGq = [a | b] [V~ | Z]^T, then dSq = Gq (dGq - rowsum(Gq dGq)) in the
    // product's epilogue where one column tile holds a row
    GMA_CHECK(gemm(false, true, nd, l1, Np * l1, vtz, l1, (int64_t)K * l1, 0, dGq, K, Np * K,
                   (int)Np, K, w1, U, 1, part, s, false, jac ? Gq : nullptr, Np * K, K));
    // [dV~ | dZ] = Gq^T [a | b]
    GMA_CHECK(gemm(true, false, Gq, K, Np * K, nd, l1, Np * l1, 0, dvtz, l1, (int64_t)K * l1, K,
                   w1, (int)Np, U, ks, part, s));
    // dV = Gk dV~, stored into the caller's dV by the epilogue
    GMA_CHECK(gemm(false, false, Gk, K, Np * K, dvtz, l1, (int64_t)K * l1, 0, dvf, dv, Np * dv,
                   (int)Np, dv, K, U, 1, part, s, false, nullptr, 0, 0, nullptr, nullptr, 0, 0.f,
                   &dvo));
    // dGk = [V | 1] [dV~ | dZ]^T (and dSk)
    GMA_CHECK(gemm(false, true, v1, l1, Np * l1, dvtz, l1, (int64_t)K * l1, 0, dGk, K, Np * K,
                   (int)Np, K, w1, U, 1, part, s, false, jac ? Gk : nullptr, Np * K, K));
  } else {
    // dGq_c = [a | b]_c [V~ | Z]_prefix^T + mask([a | b]_c [V | 1]_c^T) Gk_c
    GMA_CHECK(gemm(false, true, nd, l1, (int64_t)C * l1, vtz, l1, (int64_t)K * l1, 0, dGq, K,
                   (int64_t)C * K, C, K, w1, Z, 1, part, s));
    GMA_CHECK(gemm(false, true, nd, l1, (int64_t)C * l1, v1, l1, (int64_t)C * l1, 0, qc, C,
                   (int64_t)C * C, C, C, w1, Z, 1, part, s));
    hipLaunchKernelGGL(gma_bwd_mask_kernel, dim3(sblocks(Z * C * C, 256)), dim3(256), 0, s, qc,
                       Z * C * C, 0);
    GMA_CHECK(hipGetLastError());
    GMA_CHECK(gemm(false, false, qc, C, (int64_t)C * C, Gk, K, (int64_t)C * K, 0, dGq, K,
                   (int64_t)C * K, C, K, C, Z, 1, part, s, true, jac ? Gq : nullptr,
                   (int64_t)C * K, K));
    // per chunk: Gq_c^T [a | b]_c, then the exclusive suffix over later chunks
    GMA_CHECK(gemm(true, false, Gq, K, (int64_t)C * K, nd, l1, (int64_t)C * l1, 0, dvtz, l1,
                   (int64_t)K * l1, K, w1, C, Z, 1, part, s));
    hipLaunchKernelGGL(gma_bwd_chunk_scan_kernel, dim3(blocks((int64_t)K * l1, 256), (unsigned)U),
                       dim3(256), 0, s, dvtz, (int)L.nc, K * l1, 1);
    GMA_CHECK(hipGetLastError());
    // dGk_c = [V | 1]_c [dV~ | dZ]_suffix^T + mask([V | 1]_c [a | b]_c^T) Gq_c
    GMA_CHECK(gemm(false, true, v1, l1, (int64_t)C * l1, dvtz, l1, (int64_t)K * l1, 0, dGk, K,
                   (int64_t)C * K, C, K, w1, Z, 1, part, s));
    GMA_CHECK(gemm(false, true, v1, l1, (int64_t)C * l1, nd, l1, (int64_t)C * l1, 0, qc, C,
                   (int64_t)C * C, C, C, w1, Z, 1, part, s));
    hipLaunchKernelGGL(gma_bwd_mask_kernel, dim3(sblocks(Z * C * C, 256)), dim3(256), 0, s, qc,
                       Z * C * C, 1);
    GMA_CHECK(hipGetLastError());
    GMA_CHECK(gemm(false, false, qc, C, (int64_t)C * C, Gq, K, (int64_t)C * K, 0, dGk, K,
                   (int64_t)C * K, C, K, C, Z, 1, part, s, true, jac ? Gk : nullptr,
                   (int64_t)C * K, K));
    // dV_c = Gk_c dV~_suffix + mask(Gq_c Gk_c^T)^T a_c
    GMA_CHECK(gemm(false, false, Gk, K, (int64_t)C * K, dvtz, l1, (int64_t)K * l1, 0, dvf, dv,
                   (int64_t)C * dv, C, dv, K, Z, 1, part, s));
    GMA_CHECK(gemm(true, false, pc, C, (int64_t)C * C, nd, l1, (int64_t)C * l1, 0, dvf, dv,
                   (int64_t)C * dv, C, dv, C, Z, 1, part, s, true, nullptr, 0, 0, nullptr,
                   nullptr, 0, 0.f, &dvo));
  }
  if (g_launch_hook) g_launch_hook("gma_bwd_gemm", s, 0);
  if (!jac) {
    if (g_launch_hook) g_launch_hook("gma_bwd_rows", s, 1);
    launch_bwd_softmax(Gq, dGq, K, rows, s);
    launch_bwd_softmax(Gk, dGk, K, rows, s);
    GMA_CHECK(hipGetLastError());
    if (g_launch_hook) g_launch_hook("gma_bwd_rows", s, 0);
  }

  for (int side = 0; side < 2; ++side) {
    float* dS = side ? dGk : dGq;
    float* x3 = side ? x3k : x3q;
    if (g_launch_hook) g_launch_hook("gma_bwd_gemm", s, 1);
    // [P1 | P2] = dS [w | mu w] (the head's table); where its halves are
    // whole MFMA tiles the epilogue forms dX = -x P1 + P2 itself
    const bool fdx = gemm_dx_ok(2 * dr);
    DxOut dxo;
    dxo.dx = side ? gt.dK : gt.dQ;
    dxo.bf = sizeof(T) == 2;
    dxo.N = N0;
    dxo.X = x3;
    dxo.sX = Np * l3;
    dxo.ldx = l3;
    GMA_CHECK(gemm(false, false, dS, K, Np * K, WW, 2 * dr, (int64_t)K * 2 * dr, (int)pp.H, P,
                   2 * dr, Np * 2 * dr, (int)Np, 2 * dr, K, U, 1, part, s, false, nullptr, 0, 0,
                   fdx ? &dxo : nullptr));
    // [R1 | R2 | r0] = dS^T [x | x^2 | 1]
    GMA_CHECK(gemm(true, false, dS, K, Np * K, x3, l3, Np * l3, 0, side ? Rk : Rq, l3,
                   (int64_t)K * l3, K, w3, (int)Np, U, ks, part, s));
    if (g_launch_hook) g_launch_hook("gma_bwd_gemm", s, 0);
    if (!fdx) {
      if (g_launch_hook) g_launch_hook("gma_bwd_rows", s, 1);
      hipLaunchKernelGGL(gma_bwd_dx_kernel<T>, dim3(sblocks(rows * dr / 4, 256)), dim3(256), 0, s,
                         x3, l3, P, dr, rows, Np, N0, side ? gt.dK : gt.dQ);
      GMA_CHECK(hipGetLastError());
      if (g_launch_hook) g_launch_hook("gma_bwd_rows", s, 0);
    }
  }
  if (g_launch_hook) g_launch_hook("gma_bwd_params", s, 1);
  hipLaunchKernelGGL(gma_bwd_param_grad_kernel, dim3(blocks((int64_t)K * dr, 256), (unsigned)pp.H),
                     dim3(256), 0, s, Rq, Rk, pp.B, (int)pp.H, K, dr, l3, t.mu, t.ls2, gt.dmu,
                     gt.dls2, gt.dlpi);
  if (g_launch_hook) g_launch_hook("gma_bwd_params", s, 0);
#undef GMA_CHECK
  return hipGetLastError();
}

// ---- the forward as a chain of products --------------------------------------
// For shapes whose fused scan kernel does not fit (the causal form at large
// K x d_v): the responsibilities of queries and keys are stored in fp32 and the
// forward runs on the same batched products as the backward's first part:
//   [V~ | Z] = Gk^T [V | 1],  [n | d - eps] = Gq [V~ | Z]      (Eqs. 5-7)
// or, causal ("Causal GMA", Eq. 8b), per 64-token chunk c:
//   [n | d - eps]_c = Gq_c [V~ | Z]_prefix(c) + mask(Gq_c Gk_c^T) [V | 1]_c,
// then O = n / (d + eps).
struct ProdLayout {
  int64_t Np = 0, nc = 0;
  size_t pads, v1, nd, gq, gk, vtz, part, pc, asg, total;
  int ks_tok;
};

ProdLayout prod_layout(const Plan& pp, bool causal, int64_t N, size_t in_size) {
  ProdLayout L{};
  L.Np = pp.N;
  L.nc = causal ? pp.N / kChunk : 0;
  const size_t U = (size_t)pp.BH, Np = (size_t)pp.N, K = (size_t)pp.K;
  const size_t dr = pp.DR, dv = pp.DV;
  int ks = (int)((1024 + U - 1) / U);
  const int maxk = (int)((pp.N + 255) / 256);
  if (ks > maxk) ks = maxk;
  if (ks > 32) ks = 32;
  if ((int64_t)ks * pp.BH > 65535) ks = (int)(65535 / pp.BH);
  if (ks < 1) ks = 1;
  L.ks_tok = ks;
  size_t off = r256(pp.total);
  auto take = [&](size_t bytes) { const size_t o = off; off += r256(bytes); return o; };
  const size_t w1p = dv + 4;
  L.pads = take(causal && (int64_t)Np != N ? U * Np * (2 * dr + dv) * in_size : 0);
  L.v1 = take(U * Np * w1p * 4);
  L.nd = take(U * Np * w1p * 4);
  L.gq = take(U * Np * K * 4);
  L.gk = take(U * Np * K * 4);
  const size_t recs = causal ? U * (size_t)L.nc : U;
  L.vtz = take(recs * K * w1p * 4);
  L.part = take(causal ? 0 : U * (size_t)ks * K * w1p * 4);
  L.pc = take(causal ? recs * kChunk * kChunk * 4 : 0);
  L.asg = take(2 * U * Np * 4);
  L.total = off;
  return L;
}

template <class TI, class TO>
hipError_t run_prod_forward(const Plan& pp, const Tensors& t0, bool causal, int64_t N0,
                            hipStream_t s) {
  const ProdLayout L = prod_layout(pp, causal, N0, sizeof(TI));
  Tensors t = t0;
  char* ws = t.ws;
  float* v1 = reinterpret_cast<float*>(ws + L.v1);
  float* nd = reinterpret_cast<float*>(ws + L.nd);
  float* Gq = reinterpret_cast<float*>(ws + L.gq);
  float* Gk = reinterpret_cast<float*>(ws + L.gk);
  float* vtz = reinterpret_cast<float*>(ws + L.vtz);
  float* part = reinterpret_cast<float*>(ws + L.part);
  float* pc = reinterpret_cast<float*>(ws + L.pc);
  int32_t* aq = reinterpret_cast<int32_t*>(ws + L.asg);
  int32_t* ak = aq + (size_t)pp.BH * L.Np;
  const int64_t U = pp.BH, Np = L.Np, rows = U * Np;
  const int K = pp.K, dr = pp.DR, dv = pp.DV;
  const int w1 = dv + 1, l1 = dv + 4;
  hipError_t e;
#define GMA_CHECK(x) do { e = (x); if (e != hipSuccess) return e; } while (0)
  if (g_launch_hook) g_launch_hook("gma_prod_prep", s, 1);
  if (L.pads && Np != N0) {
    TI* pq = reinterpret_cast<TI*>(ws + L.pads);
    TI* pk = pq + (size_t)rows * dr;
    TI* pv = pk + (size_t)rows * dr;
    hipLaunchKernelGGL(gma_bwd_pad_kernel<TI>, dim3(sblocks(rows * dr, 256)), dim3(256), 0, s,
                       t.q, dr, U, Np, N0, (void*)pq);
    hipLaunchKernelGGL(gma_bwd_pad_kernel<TI>, dim3(sblocks(rows * dr, 256)), dim3(256), 0, s,
                       t.k, dr, U, Np, N0, (void*)pk);
    hipLaunchKernelGGL(gma_bwd_pad_kernel<TI>, dim3(sblocks(rows * dv, 256)), dim3(256), 0, s,
                       t.v, dv, U, Np, N0, (void*)pv);
    GMA_CHECK(hipGetLastError());
    t.q = pq;
    t.k = pk;
    t.v = pv;
  }
  hipLaunchKernelGGL(gma_bwd_prep_kernel<TI>, dim3(sblocks(rows, 1024 / dv)), dim3(256), 0, s,
                     t.v, dv, 0, rows, l1, v1);
  GMA_CHECK(hipGetLastError());
  if (g_launch_hook) g_launch_hook("gma_prod_prep", s, 0);
  // responsibilities (and assignments) of queries and keys, fp32 [U][Np][K]
  Tensors tr = t;
  tr.q = t.q;
  tr.gamma = Gq;
  tr.assign_q = t0.assign_q ? aq : nullptr;
  GMA_CHECK(launch_resp(pp, tr, s));
  tr.q = t.k;
  tr.gamma = Gk;
  tr.assign_q = t0.assign_k ? ak : nullptr;
  GMA_CHECK(launch_resp(pp, tr, s));

  const int64_t Z = causal ? U * L.nc : U;
  const int C = kChunk;
  if (g_launch_hook) g_launch_hook("gma_prod_gemm", s, 1);
  if (!causal) {
    GMA_CHECK(gemm(true, false, Gk, K, Np * K, v1, l1, Np * l1, 0, vtz, l1, (int64_t)K * l1, K,
                   w1, (int)Np, U, L.ks_tok, part, s));
    GMA_CHECK(gemm(false, false, Gq, K, Np * K, vtz, l1, (int64_t)K * l1, 0, nd, l1, Np * l1,
                   (int)Np, w1, K, U, 1, part, s));
  } else {
    GMA_CHECK(gemm(true, false, Gk, K, (int64_t)C * K, v1, l1, (int64_t)C * l1, 0, vtz, l1,
                   (int64_t)K * l1, K, w1, C, Z, 1, part, s));
    hipLaunchKernelGGL(gma_bwd_chunk_scan_kernel, dim3(blocks((int64_t)K * l1, 256), (unsigned)U),
                       dim3(256), 0, s, vtz, (int)L.nc, K * l1, 0);
    GMA_CHECK(hipGetLastError());
    GMA_CHECK(gemm(false, true, Gq, K, (int64_t)C * K, Gk, K, (int64_t)C * K, 0, pc, C,
                   (int64_t)C * C, C, C, K, Z, 1, part, s));
    hipLaunchKernelGGL(gma_bwd_mask_kernel, dim3(sblocks(Z * C * C, 256)), dim3(256), 0, s, pc,
                       Z * C * C, 0);
    GMA_CHECK(hipGetLastError());
    GMA_CHECK(gemm(false, false, Gq, K, (int64_t)C * K, vtz, l1, (int64_t)K * l1, 0, nd, l1,
                   (int64_t)C * l1, C, w1, K, Z, 1, part, s));
    GMA_CHECK(gemm(false, false, pc, C, (int64_t)C * C, v1, l1, (int64_t)C * l1, 0, nd, l1,
                   (int64_t)C * l1, C, w1, C, Z, 1, part, s, true));
  }
  if (g_launch_hook) g_launch_hook("gma_prod_gemm", s, 0);
  if (g_launch_hook) g_launch_hook("gma_prod_out", s, 1);
  hipLaunchKernelGGL(gma_prod_out_kernel<TO>, dim3(sblocks(rows * dv / 4, 256)), dim3(256), 0, s,
                     nd, dv, l1, t.eps, rows, Np, N0, t0.out);
  GMA_CHECK(hipGetLastError());
  if (t0.assign_q)
    hipLaunchKernelGGL(gma_prod_assign_kernel, dim3(sblocks(U * N0, 256)), dim3(256), 0, s, aq, U,
                       Np, N0, t0.assign_q);
  if (t0.assign_k)
    hipLaunchKernelGGL(gma_prod_assign_kernel, dim3(sblocks(U * N0, 256)), dim3(256), 0, s, ak, U,
                       Np, N0, t0.assign_k);
  if (g_launch_hook) g_launch_hook("gma_prod_out", s, 0);
#undef GMA_CHECK
  return hipGetLastError();
}

}  // namespace

size_t backward_workspace_bytes(const Plan& pp, bool causal, int64_t N) {
  return bwd_layout(pp, causal, N).total;
}

hipError_t launch_backward(const Plan& pp, const Tensors& t, const BwdTensors& gt, bool causal,
                           int64_t N, hipStream_t s) {
  const hipError_t e = launch_prologue(pp, t, s);
  if (e != hipSuccess) return e;
  return pp.out_bf ? run_backward<bf16>(pp, t, gt, causal, N, s)
                   : run_backward<float>(pp, t, gt, causal, N, s);
}

}  // namespace gma

namespace gma {

size_t prod_forward_workspace_bytes(const Plan& pp, bool causal, int64_t N) {
  return prod_layout(pp, causal, N, pp.bf ? 2 : 4).total;
}

hipError_t launch_prod_forward(const Plan& pp, const Tensors& t, bool causal, int64_t N,
                               bool out_bf, hipStream_t s) {
  const hipError_t e = launch_prologue(pp, t, s);
  if (e != hipSuccess) return e;
  if (pp.bf) return run_prod_forward<bf16, bf16>(pp, t, causal, N, s);
  return out_bf ? run_prod_forward<float, bf16>(pp, t, causal, N, s)
                : run_prod_forward<float, float>(pp, t, causal, N, s);
}

}  // namespace gma
