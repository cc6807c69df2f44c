// Bidirectional GMA forward on gfx950: parameter prologue, latent write,
// partial reduction and the fused responsibility + read kernel.
//
// Paper: "Gaussian Mixture Attention: Linear-Time Sequence Mixing via
// Probabilistic Latent Routing".
//  - Scores (Eqs. 2-3 and Eq. 16): s_ik = log pi_k + log N(x_i; mu_k, diag sigma^2_k).
//    Expanded as s_ik = c_k + sum_d A_kd x_d^2 + sum_d B_kd x_d with
//    A = -w/2, B = mu*w, c = log pi - 1/2 sum_d (mu^2 w + log sigma^2),
//    w = exp(-log sigma^2); the -(d_r/2) log 2pi term is dropped because the
//    posterior is a softmax over k.  A, B and c carry a factor log2(e) so the
//    exponentials are exp2.  Both contractions run on MFMA.  The fp32 path
//    contracts A with (x^2 - 1) and adds c + sum_d A_kd afterwards: the same
//    value in exact arithmetic, with a far smaller fp32 accumulator.
//  - gamma_ik = exp(s_ik - m_i) / sum_l exp(s_il - m_i) with m_i = max_k s_ik.
//  - Write (Eqs. 5-6): V~ = Gamma^K^T V_X, Z = Gamma^K^T 1, split over N with
//    deterministic partial sums.
//  - Read (Eq. 7 and its footnote): O_i = gamma^Q_i V~ / (gamma^Q_i Z + eps),
//    fused with the query responsibilities so Gamma^Q never reaches HBM.
//
// Workgroup = 4 waves on a 64-token tile.  The K_pad = 16*CT components are
// split into NG groups; wave w owns component group w % NG (CPW 16-wide tiles,
// its A/B coefficients held in VGPRs for the whole kernel) and token group
// w / NG (NG of the four 16-token MFMA tiles).  Per-token max / sum over
// components is finished across the NG waves through LDS.
#include "gma_tiles.h"

namespace gma {

// ============================================================================
// Parameter prologue: per head, A, B (bf16 hi/lo pairs or fp32) and c.
// Layout per head: NARR arrays [Kp][DRP] (A_hi, A_lo, B_hi, B_lo or A, B)
// followed by c[Kp] fp32.  Padded components get A = B = 0, c = -inf
// (gamma exactly 0); padded routing columns get A = B = 0.
// ============================================================================
template <bool BF>
__global__ void __launch_bounds__(256) gma_prologue_kernel(
    const float* __restrict__ mu, const float* __restrict__ ls2, const float* __restrict__ lpi,
    int H, int K, int Kp, int DR, int DRP, char* __restrict__ params, size_t head_bytes) {
  // one wave per (head, component) row; lanes stride the routing columns
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (row >= H * Kp) return;
  const int h = row / Kp, k = row - h * Kp;
  const int n = Kp * DRP;
  char* base = params + (size_t)h * head_bytes;
  // fp32 path: the kernels contract A with (x^2 - 1) instead of x^2 (keeping the
  // fp32 accumulator near zero for unit-scale routing vectors) and add
  // c' = c + sum_d A_kd once at the end; bf16 path: c seeds the accumulator.
  double acc = 0.0, asum = 0.0;
  for (int d = lane; d < DRP; d += 64) {
    double a = 0.0, b = 0.0;
    if (k < K && d < DR) {
      const size_t off = ((size_t)h * K + k) * DR + d;
      const double l = ls2[off], m = mu[off];
      const double w = (double)expf(-ls2[off]);
      a = -0.5 * w * kLog2eD;
      b = m * w * kLog2eD;
      acc += m * m * w + l;
      asum += -0.5 * w;
    }
    const int idx = k * DRP + d;
    if constexpr (BF) {
      bf16* Ahi = reinterpret_cast<bf16*>(base);
      const bf16 ah = to_bf16((float)a), bh = to_bf16((float)b);
      Ahi[idx] = ah;
      Ahi[n + idx] = to_bf16((float)(a - (double)from_bf16(ah)));
      Ahi[2 * n + idx] = bh;
      Ahi[3 * n + idx] = to_bf16((float)(b - (double)from_bf16(bh)));
    } else {
      float* A = reinterpret_cast<float*>(base);
      A[idx] = (float)a;
      A[n + idx] = (float)b;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    acc += __shfl_xor(acc, off);
    asum += __shfl_xor(asum, off);
  }
  if (lane == 0) {
    float* c = reinterpret_cast<float*>(base + (size_t)8 * n);
    if (k < K) {
      const double ck = (double)lpi[(size_t)h * K + k] - 0.5 * acc + (BF ? 0.0 : asum);
      c[k] = (float)(kLog2eD * ck);
    } else {
      c[k] = -INFINITY;
    }
  }
}

// Sum the partials of each sequence in a fixed order: V~ [BH][Kp][DV], Z [BH][Kp].
__global__ void __launch_bounds__(256) gma_reduce_kernel(const float* __restrict__ partial,
                                                         const float* __restrict__ partial_z,
                                                         int PS, int Kp, int DV,
                                                         float* __restrict__ vt,
                                                         float* __restrict__ z) {
  const int64_t bh = blockIdx.y;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  const int nv = Kp * DV;
  if (idx < nv) {
    const float* p = partial + (size_t)bh * PS * nv + idx;
    float s = 0.f;
    for (int q = 0; q < PS; ++q) s += p[(size_t)q * nv];
    vt[(size_t)bh * nv + idx] = s;
  } else if (idx < nv + Kp) {
    const int k = idx - nv;
    const float* p = partial_z + (size_t)bh * PS * Kp + k;
    float s = 0.f;
    for (int q = 0; q < PS; ++q) s += p[(size_t)q * Kp];
    z[(size_t)bh * Kp + k] = s;
  }
}

// ============================================================================
// Fused query responsibilities + read-out (MODE 0), or responsibilities only
// (MODE 1: gamma and assignment written to HBM, for testing).
// ============================================================================
template <class C, int MODE>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(C::kWPERead))) gma_read_kernel(BidirArgs a) {
  using in_t = typename C::in_t;
  using op_t = typename C::op_t;
  using chunk_t = typename C::chunk_t;
  __shared__ __attribute__((aligned(16))) op_t F[C::NF * C::FAS];
  __shared__ __attribute__((aligned(16))) op_t G[MODE == 0 ? C::GAS : 1];
  __shared__ __attribute__((aligned(16))) f32x4 stats[C::NG * kTile];
  __shared__ __attribute__((aligned(16))) float fac[C::NG * kTile];
  __shared__ __attribute__((aligned(16))) float rinv[kTile];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int cgi = wave % C::NG, tg = wave / C::NG;
  const int gt0 = tg * C::TTW;
  const int64_t bh = blockIdx.y;
  const int h = (int)(bh % a.H);
  const int split = blockIdx.x;
  const int64_t t_begin = (int64_t)split * a.tiles_per_split * kTile;
  const int64_t t_end = min(a.N, t_begin + (int64_t)a.tiles_per_split * kTile);
  const bool want_assign = a.assign != nullptr;

  for (int i = threadIdx.x; i < C::NF * C::FAS; i += kThreads) F[i] = (op_t)0;
  if constexpr (MODE == 0)
    for (int i = threadIdx.x; i < C::GAS; i += kThreads) G[i] = (op_t)0;

  const char* pbase = a.params + (size_t)h * a.head_bytes;
  chunk_t W[C::CPW][C::NKS][C::NARR];
  load_w<C>(pbase, cgi * C::CPW, W);
  const float* cvec = reinterpret_cast<const float*>(pbase + (size_t)8 * C::Kp * C::DRP);
  f32x4 cv4[C::CPW], z4[C::CPW];
#pragma unroll
  for (int ct = 0; ct < C::CPW; ++ct) {
    const int comp = (cgi * C::CPW + ct) * 16 + 4 * g;
    cv4[ct] = ld16<f32x4>(cvec + comp);
    if constexpr (MODE == 0) z4[ct] = ld16<f32x4>(a.z + (size_t)bh * C::Kp + comp);
    else z4[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // V~ slice as the B operand of the read-out contraction (components x d_v)
  chunk_t Vr[MODE == 0 ? C::DPW : 1][C::KSO];
  if constexpr (MODE == 0) {
#pragma unroll
    for (int j = 0; j < C::DPW; ++j) {
      const int dt = C::DVT >= C::NG ? cgi * C::DPW + j : cgi % C::DVT;
      const float* vtb = a.vt + (size_t)bh * C::Kp * C::DV + dt * 16 + c;
#pragma unroll
      for (int s = 0; s < C::KSO; ++s)
#pragma unroll
        for (int e = 0; e < C::E; ++e) {
          const int comp = s * C::CS + g * C::E + e;
          const float val = comp < C::Kp ? vtb[(size_t)comp * C::DV] : 0.f;
          Vr[j][s][e] = (op_t)val;
        }
    }
  }

  const in_t* xs = reinterpret_cast<const in_t*>(a.x) + (size_t)bh * a.N * C::DR;
  FeatureTile<C> xreg;
  if (t_begin < t_end) xreg.load(xs, t_begin, (int)min((int64_t)kTile, t_end - t_begin));

  for (int64_t tile0 = t_begin; tile0 < t_end; tile0 += kTile) {
    const int nvalid = (int)min((int64_t)kTile, t_end - tile0);
    lds_barrier();
    xreg.store(F);
    lds_barrier();
    if (tile0 + kTile < t_end)
      xreg.load(xs, tile0 + kTile, (int)min((int64_t)kTile, t_end - tile0 - kTile));

    f32x4 S[C::TTW][C::CPW];
#pragma unroll
    for (int tt = 0; tt < C::TTW; ++tt)
#pragma unroll
      for (int ct = 0; ct < C::CPW; ++ct) S[tt][ct] = score_seed<C>(cv4[ct]);
    score_tiles<C, true>(F, gt0, W, S);
#pragma unroll
    for (int tt = 0; tt < C::TTW; ++tt)
#pragma unroll
      for (int ct = 0; ct < C::CPW; ++ct) finish_scores<C>(S[tt][ct], cv4[ct]);

    // lane (c, g) holds token tile_token(gt, c) and components 16*ctile + 4g + i
    float m[C::TTW], l[C::TTW], dn[C::TTW];
    int am[C::TTW];
#pragma unroll
    for (int tt = 0; tt < C::TTW; ++tt) {
      float v = S[tt][0][0];
#pragma unroll
      for (int ct = 0; ct < C::CPW; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) v = fmaxf(v, S[tt][ct][i]);
      m[tt] = groups_max(v);
      am[tt] = 0;
      if (want_assign) {
        float bv = S[tt][0][0];
        int bi = (cgi * C::CPW) * 16 + 4 * g;
#pragma unroll
        for (int ct = 0; ct < C::CPW; ++ct)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            argmax_merge(bv, bi, S[tt][ct][i], (cgi * C::CPW + ct) * 16 + 4 * g + i);
        groups_argmax(bv, bi);
        am[tt] = bi;
      }
      const float mu_ = m[tt] == -INFINITY ? 0.f : m[tt];
      float sum = 0.f, den = 0.f;
#pragma unroll
      for (int ct = 0; ct < C::CPW; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = exp2_fast(S[tt][ct][i] - mu_);
          S[tt][ct][i] = e;
          sum += e;
          den += e * z4[ct][i];
        }
      l[tt] = groups_sum(sum);
      dn[tt] = groups_sum(den);
    }

    float f[C::TTW];
    if constexpr (C::NG > 1) {
      if (g == 0) {
#pragma unroll
        for (int tt = 0; tt < C::TTW; ++tt)
          stats[cgi * kTile + tile_token(gt0 + tt, c)] =
              f32x4{m[tt], l[tt], dn[tt], __int_as_float(am[tt])};
      }
      lds_barrier();
      if (threadIdx.x < kTile) {
        const int t = threadIdx.x;
        f32x4 st[C::NG];
        float M = -INFINITY;
#pragma unroll
        for (int q = 0; q < C::NG; ++q) {
          st[q] = stats[q * kTile + t];
          M = fmaxf(M, st[q][0]);
        }
        float L = 0.f, D = 0.f, fq[C::NG];
        int arg = 0;
        bool found = false;
#pragma unroll
        for (int q = 0; q < C::NG; ++q) {
          fq[q] = st[q][0] == -INFINITY ? 0.f : exp2_fast(st[q][0] - M);
          L += fq[q] * st[q][1];
          D += fq[q] * st[q][2];
          if (!found && st[q][0] == M) { arg = __float_as_int(st[q][3]); found = true; }
        }
        if constexpr (MODE == 0) {
#pragma unroll
          for (int q = 0; q < C::NG; ++q) fac[q * kTile + t] = fq[q];
          rinv[t] = 1.f / (D + a.eps * L);
        } else {
          const float invL = 1.f / L;
#pragma unroll
          for (int q = 0; q < C::NG; ++q) fac[q * kTile + t] = fq[q] * invL;
        }
        if (want_assign && t < nvalid) a.assign[(size_t)bh * a.N + tile0 + t] = arg;
      }
      lds_barrier();
#pragma unroll
      for (int tt = 0; tt < C::TTW; ++tt) f[tt] = fac[cgi * kTile + tile_token(gt0 + tt, c)];
    } else {
#pragma unroll
      for (int tt = 0; tt < C::TTW; ++tt) {
        const int tok = tile_token(gt0 + tt, c);
        if constexpr (MODE == 0) {
          f[tt] = 1.f;
          if (g == 0) rinv[tok] = 1.f / (dn[tt] + a.eps * l[tt]);
        } else {
          f[tt] = 1.f / l[tt];
        }
        if (want_assign && g == 0 && tok < nvalid) a.assign[(size_t)bh * a.N + tile0 + tok] = am[tt];
      }
    }

    if constexpr (MODE == 1) {
      if (a.gamma != nullptr) {
#pragma unroll
        for (int tt = 0; tt < C::TTW; ++tt) {
          const int tok = tile_token(gt0 + tt, c);
          if (tok < nvalid) {
            float* gr = a.gamma + ((size_t)bh * a.N + tile0 + tok) * a.K;
#pragma unroll
            for (int ct = 0; ct < C::CPW; ++ct)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int comp = (cgi * C::CPW + ct) * 16 + 4 * g + i;
                if (comp < a.K) gr[comp] = S[tt][ct][i] * f[tt];
              }
          }
        }
      }
      continue;
    } else {
      // Gamma' (unnormalised responsibilities relative to the tile maximum) -> LDS [token][component]
#pragma unroll
      for (int tt = 0; tt < C::TTW; ++tt) {
        const int tok = tile_token(gt0 + tt, c);
#pragma unroll
        for (int ct = 0; ct < C::CPW; ++ct) {
          op_t* dst = &G[C::grow(tok) + (cgi * C::CPW + ct) * 16 + 4 * g];
          if constexpr (C::kBF) {
            bf16x4 v4;
#pragma unroll
            for (int i = 0; i < 4; ++i) v4[i] = to_bf16(S[tt][ct][i] * f[tt]);
            *reinterpret_cast<bf16x4*>(dst) = v4;
          } else {
            st16(dst, S[tt][ct] * f[tt]);
          }
        }
      }
      lds_barrier();

      // O^T = V~^T Gamma'^T for this wave's (token tile, d tile) share: lane column =
      // token, rows = four consecutive d, so each lane scales by one normaliser and
      // writes 8 (bf16) or 16 (fp32) contiguous bytes
#pragma unroll
      for (int jt = 0; jt < C::TPW; ++jt) {
        const int tt = C::DVT >= C::NG ? jt : cgi / C::DVT + (C::NG / C::DVT) * jt;
        const int gt = gt0 + tt;
        f32x4 acc[C::DPW];
#pragma unroll
        for (int j = 0; j < C::DPW; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int rtok = tile_token(gt, c);
#pragma unroll
        for (int s = 0; s < C::KSO; ++s) {
          const chunk_t Bg = ld16<chunk_t>(&G[C::grow(rtok) + s * C::CS + g * C::E]);
#pragma unroll
          for (int j = 0; j < C::DPW; ++j) acc[j] = mma(Vr[j][s], Bg, acc[j]);
        }
        const float rv = rinv[rtok];
        if (rtok < nvalid) {
#pragma unroll
          for (int j = 0; j < C::DPW; ++j) {
            const int dt = C::DVT >= C::NG ? cgi * C::DPW + j : cgi % C::DVT;
            const size_t off = ((size_t)bh * a.N + tile0 + rtok) * C::DV + dt * 16 + 4 * g;
            const f32x4 o = acc[j] * rv;
            if (a.out_bf) {
              bf16x4 o4;
#pragma unroll
              for (int i = 0; i < 4; ++i) o4[i] = to_bf16(o[i]);
              *reinterpret_cast<bf16x4*>(reinterpret_cast<bf16*>(a.out) + off) = o4;
            } else {
              st16(reinterpret_cast<float*>(a.out) + off, o);
            }
          }
        }
      }
    }
  }
}

// ============================================================================
// Host-side dispatch.
// ============================================================================
template <class C>
static hipError_t run_bidir(const Plan& p, const Tensors& t, hipStream_t s) {
  BidirArgs a{};
  a.params = t.ws + p.off_params;
  a.head_bytes = p.head_bytes;
  a.partial = reinterpret_cast<float*>(t.ws + p.off_partial);
  a.partial_z = reinterpret_cast<float*>(t.ws + p.off_partial_z);
  a.vt = reinterpret_cast<const float*>(t.ws + p.off_vt);
  a.z = reinterpret_cast<const float*>(t.ws + p.off_z);
  a.N = p.N;
  a.H = (int)p.H;
  a.K = p.K;
  a.S = p.S;
  a.tiles_per_split = p.tiles_per_split;
  a.eps = t.eps;
  a.out_bf = p.out_bf ? 1 : 0;
  const dim3 grid(p.S, (unsigned)p.BH);

  a.x = t.k;
  a.v = t.v;
  a.assign = t.assign_k;
  if (g_launch_hook) g_launch_hook("gma_write", s, 1);
  if constexpr (C::kBF) hipLaunchKernelGGL(gma_write_bf16_kernel<C>, grid, dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL(gma_write_kernel<C>, grid, dim3(kThreads), 0, s, a);
  if (g_launch_hook) g_launch_hook("gma_write", s, 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int PS = C::kBF ? p.S : p.S * C::TG;    // partial slots per sequence
  const int nred = C::Kp * C::DV + C::Kp;
  if (g_launch_hook) g_launch_hook("gma_reduce", s, 1);
  hipLaunchKernelGGL(gma_reduce_kernel, dim3((nred + 255) / 256, (unsigned)p.BH), dim3(256), 0, s,
                     a.partial, a.partial_z, PS, C::Kp, C::DV,
                     reinterpret_cast<float*>(t.ws + p.off_vt),
                     reinterpret_cast<float*>(t.ws + p.off_z));
  if (g_launch_hook) g_launch_hook("gma_reduce", s, 0);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  a.x = t.q;
  a.v = nullptr;
  a.out = t.out;
  a.assign = t.assign_q;
  if (g_launch_hook) g_launch_hook("gma_read", s, 1);
  hipLaunchKernelGGL((gma_read_kernel<C, 0>), grid, dim3(kThreads), 0, s, a);
  if (g_launch_hook) g_launch_hook("gma_read", s, 0);
  return hipGetLastError();
}

template <class C>
static hipError_t run_resp(const Plan& p, const Tensors& t, hipStream_t s) {
  BidirArgs a{};
  a.params = t.ws + p.off_params;
  a.head_bytes = p.head_bytes;
  a.N = p.N;
  a.H = (int)p.H;
  a.K = p.K;
  a.S = p.S;
  a.tiles_per_split = p.tiles_per_split;
  a.x = t.q;
  a.assign = t.assign_q;
  a.gamma = t.gamma;
  if (g_launch_hook) g_launch_hook("gma_resp", s, 1);
  hipLaunchKernelGGL((gma_read_kernel<C, 1>), dim3(p.S, (unsigned)p.BH), dim3(kThreads), 0, s, a);
  if (g_launch_hook) g_launch_hook("gma_resp", s, 0);
  return hipGetLastError();
}

hipError_t launch_prologue(const Plan& p, const Tensors& t, hipStream_t s) {
  if (g_launch_hook) g_launch_hook("gma_prologue", s, 1);
  const int64_t rows = p.H * (int64_t)p.Kp;          // one wave per (head, component)
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (p.bf)
    hipLaunchKernelGGL(gma_prologue_kernel<true>, grid, dim3(256), 0, s, t.mu, t.ls2, t.lpi,
                       (int)p.H, p.K, p.Kp, p.DR, p.DRP, t.ws + p.off_params, p.head_bytes);
  else
    hipLaunchKernelGGL(gma_prologue_kernel<false>, grid, dim3(256), 0, s, t.mu, t.ls2, t.lpi,
                       (int)p.H, p.K, p.Kp, p.DR, p.DRP, t.ws + p.off_params, p.head_bytes);
  if (g_launch_hook) g_launch_hook("gma_prologue", s, 0);
  return hipGetLastError();
}

// (BF, CPW, NG) x DR x DV dispatch.
#define GMA_DV_CASES(FN, BF, CPW, NG, DR)                                   \
  switch (p.DV) {                                                           \
    case 16: return FN<Cfg<BF, CPW, NG, DR, 16>>(p, t, s);                  \
    case 32: return FN<Cfg<BF, CPW, NG, DR, 32>>(p, t, s);                  \
    case 64: return FN<Cfg<BF, CPW, NG, DR, 64>>(p, t, s);                  \
    case 128: return FN<Cfg<BF, CPW, NG, DR, 128>>(p, t, s);                \
  }                                                                         \
  break;
#define GMA_DR_CASES(FN, BF, CPW, NG)                                       \
  switch (p.DR) {                                                           \
    case 16: GMA_DV_CASES(FN, BF, CPW, NG, 16)                              \
    case 32: GMA_DV_CASES(FN, BF, CPW, NG, 32)                              \
    case 64: GMA_DV_CASES(FN, BF, CPW, NG, 64)                              \
    case 128: GMA_DV_CASES(FN, BF, CPW, NG, 128)                            \
  }                                                                         \
  break;
#define GMA_GROUP_CASES(FN, BF)                                             \
  switch (p.CT) {                                                           \
    case 1: GMA_DR_CASES(FN, BF, 1, 1)                                      \
    case 2: GMA_DR_CASES(FN, BF, 2, 1)                                      \
    case 4: GMA_DR_CASES(FN, BF, 2, 2)                                      \
    case 8: GMA_DR_CASES(FN, BF, 2, 4)                                      \
  }                                                                         \
  break;

hipError_t launch_bidir(const Plan& p, const Tensors& t, hipStream_t s) {
  if (p.bf) {
    switch (0) { default: GMA_GROUP_CASES(run_bidir, true) }
  } else {
    switch (0) { default: GMA_GROUP_CASES(run_bidir, false) }
  }
  return hipErrorInvalidValue;
}

// Responsibilities do not depend on d_v; fix DV = 16 for the instantiation.
#define GMA_RESP_DR_CASES(BF, CPW, NG)                                      \
  switch (p.DR) {                                                           \
    case 16: return run_resp<Cfg<BF, CPW, NG, 16, 16>>(p, t, s);            \
    case 32: return run_resp<Cfg<BF, CPW, NG, 32, 16>>(p, t, s);            \
    case 64: return run_resp<Cfg<BF, CPW, NG, 64, 16>>(p, t, s);            \
    case 128: return run_resp<Cfg<BF, CPW, NG, 128, 16>>(p, t, s);          \
  }                                                                         \
  break;
#define GMA_RESP_CASES(BF)                                                  \
  switch (p.CT) {                                                           \
    case 1: GMA_RESP_DR_CASES(BF, 1, 1)                                     \
    case 2: GMA_RESP_DR_CASES(BF, 2, 1)                                     \
    case 4: GMA_RESP_DR_CASES(BF, 2, 2)                                     \
    case 8: GMA_RESP_DR_CASES(BF, 2, 4)                                     \
  }                                                                         \
  break;

hipError_t launch_resp(const Plan& p, const Tensors& t, hipStream_t s) {
  if (p.bf) {
    switch (0) { default: GMA_RESP_CASES(true) }
  } else {
    switch (0) { default: GMA_RESP_CASES(false) }
  }
  return hipErrorInvalidValue;
}

}  // namespace gma
