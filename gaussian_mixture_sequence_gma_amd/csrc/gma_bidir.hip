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
#include "gma_team.h"

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
    int H, int K, int Kp, int DR, int DRP, char* __restrict__ params, size_t head_bytes,
    const float* __restrict__ omega, const float* __restrict__ alpha, float eps_sigma) {
  // one wave per (head, component) row; lanes stride the routing columns
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (row >= H * Kp) return;
  const int h = row / Kp, k = row - h * Kp;
  // with omega: log sigma^2 and log pi from the unconstrained parameters, by
  // the reparameterisation kernel's own arithmetic
  const float lse = omega ? wave_log_norm(alpha + (size_t)h * K, K) : 0.f;
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
      const float lf = omega ? reparam_log_var(omega[off], eps_sigma) : ls2[off];
      const double l = lf, m = mu[off];
      const double w = (double)expf(-lf);
      a = -0.5 * w * kLog2eD;
      b = m * w * kLog2eD;
      acc += m * m * w + l;
      asum += -0.5 * w;
    }
    const int idx = k * DRP + d;
    if constexpr (BF) {
      bf16* Ahi = reinterpret_cast<bf16*>(base);
      const bf16 ah = to_bf16((float)a), bh = to_bf16((float)b);
      const bf16 v4[4] = {ah, to_bf16((float)(a - (double)from_bf16(ah))), bh,
                          to_bf16((float)(b - (double)from_bf16(bh)))};
#pragma unroll
      for (int ar = 0; ar < 4; ++ar) Ahi[ar * n + idx] = v4[ar];
      if (Kp % 32 == 0) {
        // operand order: chunk (tile, routing step, array), lane (row, d group), element
        bf16* T = reinterpret_cast<bf16*>(base + head_bytes / 2);
        const int ct = pair_tile(k), r = pair_rowof(k), st = d >> 5, gg = (d & 31) >> 3;
#pragma unroll
        for (int ar = 0; ar < 4; ++ar)
          T[((((ct * (DRP / 32) + st) * 4 + ar) * 64) + r + 16 * gg) * 8 + (d & 7)] = v4[ar];
      }
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
    float cv = -INFINITY;
    if (k < K) {
      const float lp = omega ? alpha[(size_t)h * K + k] - lse : lpi[(size_t)h * K + k];
      const double ck = (double)lp - 0.5 * acc + (BF ? 0.0 : asum);
      cv = (float)(kLog2eD * ck);
    }
    c[k] = cv;
    if (BF && Kp % 32 == 0) {
      float* cp = reinterpret_cast<float*>(base + head_bytes / 2 + (size_t)8 * n);
      cp[pair_tile(k) * 16 + pair_rowof(k)] = cv;
    }
  }
}

// Sum the partials of each sequence in a fixed order: V~ [BH][Kp][DV], Z [BH][Kp].
// With st_v / st_z the first K rows are also written unpadded, [BH][K][DV] and
// [BH][K]: the carried state of a prefix for the decode step.
// With vtab (bf16 path, K_pad a multiple of 32) the sums are also written as
// the read-out's MFMA operand table: block dt (d tile, paired rows as in
// pair_row when d_v >= 32), step p (32 components), lane (row, component
// group), element; block d_v/16 holds rows Z_hi, Z_lo, 1 and zeros.
// Thread j < DV * Kp / 8 sums column d = j % DV of the eight components
// 8 (j / DV) .. + 7 (one 16-byte operand chunk); the next Kp threads sum Z.
__global__ void __launch_bounds__(256) gma_reduce_kernel(const float* __restrict__ partial,
                                                         const float* __restrict__ partial_z,
                                                         int PS, int Kp, int DV,
                                                         float* __restrict__ vt,
                                                         float* __restrict__ z,
                                                         bf16* __restrict__ vtab,
                                                         float* __restrict__ st_v,
                                                         float* __restrict__ st_z, int K) {
  const int64_t bh = blockIdx.y;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  const int nv = Kp * DV, nv8 = nv / 8;
  const int DVT = DV / 16, KS = Kp / 32;
  bf16* vb = vtab ? vtab + (size_t)bh * (DVT + 1) * KS * 512 : nullptr;
  if (idx < nv8) {
    const int d = idx % DV, k0 = 8 * (idx / DV);
    const float* p = partial + (size_t)bh * PS * nv + (size_t)k0 * DV + d;
    float sum[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) sum[e] = 0.f;
    // four partial slots' loads in flight before they are added, in slot order
    int q = 0;
    for (; q + 4 <= PS; q += 4) {
      float v[4][8];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) v[u][e] = p[(size_t)(q + u) * nv + e * DV];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) sum[e] += v[u][e];
    }
    for (; q < PS; ++q)
#pragma unroll
      for (int e = 0; e < 8; ++e) sum[e] += p[(size_t)q * nv + e * DV];
    bf16x8 pk;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int k = k0 + e;
      vt[(size_t)bh * nv + (size_t)k * DV + d] = sum[e];
      if (st_v && k < K) st_v[((size_t)bh * K + k) * DV + d] = sum[e];
      pk[e] = to_bf16(sum[e]);
    }
    if (vb) {
      const int t = DVT >= 2 ? pair_tile(d) : 0, r = DVT >= 2 ? pair_rowof(d) : d;
      st16(vb + ((t * KS + (k0 >> 5)) * 64 + r + 16 * ((k0 & 31) >> 3)) * 8, pk);
    }
  } else if (idx < nv8 + Kp) {
    const int k = idx - nv8;
    const float* p = partial_z + (size_t)bh * PS * Kp + k;
    float s = 0.f;
    int q = 0;
    for (; q + 8 <= PS; q += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = p[(size_t)(q + u) * Kp];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; q < PS; ++q) s += p[(size_t)q * Kp];
    z[(size_t)bh * Kp + k] = s;
    if (st_z && k < K) st_z[(size_t)bh * K + k] = s;
    if (vb) {
      const bf16 zh = to_bf16(s);
      const bf16 zl = to_bf16(s - from_bf16(zh));
      bf16* col = vb + ((DVT * KS + (k >> 5)) * 64 + 16 * ((k & 31) >> 3)) * 8 + (k & 7);
#pragma unroll
      for (int r = 0; r < 16; ++r)
        col[r * 8] = r == 0 ? zh : (r == 1 ? zl : (r == 2 ? (bf16)1.0f : (bf16)0.0f));
    }
  }
}

// ============================================================================
// Fused query responsibilities + read-out (MODE 0), or responsibilities only
// (MODE 1: gamma and assignment written to HBM, for testing), or usage
// statistics of the responsibilities (MODE 2: per workgroup, for each
// component the sum of gamma, the number of tokens with gamma above a.thr and
// the number of tokens assigned to it, and the sum of gamma ln gamma over all
// tokens and components, written to a.diag; nothing per token).
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
  // usage statistics: per token group the gamma sums and threshold counts of
  // every component, then the four waves' gamma ln gamma sums; assignments
  __shared__ float dred[MODE == 2 ? 2 * C::TG * C::Kp + kWaves : 1];
  __shared__ int hist[MODE == 2 ? C::Kp : 1];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int cgi = wave % C::NG, tg = wave / C::NG;
  const int gt0 = tg * C::TTW;
  const int64_t bh = blockIdx.y;
  const int h = (int)(bh % a.H);
  const int split = blockIdx.x;
  const int64_t t_begin = (int64_t)split * a.tiles_per_split * kTile;
  const int64_t t_end = min(a.N, t_begin + (int64_t)a.tiles_per_split * kTile);
  const bool want_assign = a.assign != nullptr || MODE == 2;
  float dsum[C::CPW][4], dcnt[C::CPW][4], dent = 0.f;
#pragma unroll
  for (int ct = 0; ct < C::CPW; ++ct)
#pragma unroll
    for (int i = 0; i < 4; ++i) dsum[ct][i] = dcnt[ct][i] = 0.f;
  if constexpr (MODE == 2)
    for (int i = threadIdx.x; i < C::Kp; i += kThreads) hist[i] = 0;

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
  const op_t* fb[C::TTW];
#pragma unroll
  for (int tt = 0; tt < C::TTW; ++tt) fb[tt] = F + C::frow(tile_token(gt0 + tt, c)) + g * C::E;
  FeatureTile<C> xreg;
  auto tile_n = [&](int64_t t0) { return (int)min((int64_t)kTile, t_end - t0); };
  if (t_begin < t_end) {
    xreg.load(xs, t_begin, tile_n(t_begin));
    lds_barrier();                         // F zero-fill done before the first stage
    xreg.store(F);
    if (t_begin + kTile < t_end) xreg.load(xs, t_begin + kTile, tile_n(t_begin + kTile));
    lds_barrier();
  }

  // Per tile three barriers: B1 after the per-group statistics (every wave is
  // also done reading F), B2 after the combine and the staging of the next
  // tile's features, B3 after Gamma' is in LDS.
  for (int64_t tile0 = t_begin; tile0 < t_end; tile0 += kTile) {
    const int nvalid = tile_n(tile0);
    const bool has_next = tile0 + kTile < t_end;

    f32x4 S[C::TTW][C::CPW];
#pragma unroll
    for (int tt = 0; tt < C::TTW; ++tt)
#pragma unroll
      for (int ct = 0; ct < C::CPW; ++ct) S[tt][ct] = score_seed<C>(cv4[ct]);
    if constexpr (C::kBF) {
      // MFMA order with independent accumulators back to back, half a tile of
      // feature operands in flight at a time
      score_range_T<C, 0, C::TTW / 2>(fb, W, S);
      score_range_T<C, C::TTW / 2, C::TTW>(fb, W, S);
    } else {
      score_tiles<C, true>(F, gt0, W, S);
    }
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
          if constexpr (MODE == 0) den += e * z4[ct][i];
        }
      l[tt] = groups_sum(sum);
      dn[tt] = MODE == 0 ? groups_sum(den) : 0.f;
    }
    if (C::NG > 1 && g == 0) {
#pragma unroll
      for (int tt = 0; tt < C::TTW; ++tt)
        stats[cgi * kTile + tile_token(gt0 + tt, c)] =
            f32x4{m[tt], l[tt], dn[tt], __int_as_float(am[tt])};
    }
    lds_barrier();                                                    // B1

    if constexpr (C::NG > 1) {
      // Combine the NG groups of every token: thread (token, q) with the NG
      // threads of a token adjacent, reduced with in-quad DPP exchanges.  The
      // factor for group q folds in the normaliser: fq / (D + eps L) for the
      // read-out, fq / L for the responsibilities.
      if (threadIdx.x < kTile * C::NG) {
        const int t = threadIdx.x / C::NG, q = threadIdx.x % C::NG;
        const f32x4 st = stats[q * kTile + t];
        float M = st[0];
        M = fmaxf(M, dpp<0xB1>(M));
        if constexpr (C::NG == 4) M = fmaxf(M, dpp<0x4E>(M));
        const float fq = st[0] == -INFINITY ? 0.f : exp2_fast(st[0] - M);
        float L = fq * st[1], D = fq * st[2];
        L += dpp<0xB1>(L);
        D += dpp<0xB1>(D);
        if constexpr (C::NG == 4) {
          L += dpp<0x4E>(L);
          D += dpp<0x4E>(D);
        }
        fac[q * kTile + t] = MODE == 0 ? fq * fast_rcp(D + a.eps * L) : fq * fast_rcp(L);
        if (want_assign) {
          // groups cover increasing component ranges: the smallest index among
          // the groups attaining the maximum is the lowest-index argmax
          int key = st[0] == M ? __float_as_int(st[3]) : 0x7fffffff;
          key = min(key, dpp_i<0xB1>(key));
          if constexpr (C::NG == 4) key = min(key, dpp_i<0x4E>(key));
          if (q == 0 && t < nvalid) {
            if constexpr (MODE == 2) {
              if ((unsigned)key < (unsigned)C::Kp) atomicAdd(&hist[key], 1);
            } else {
              a.assign[(size_t)bh * a.N + tile0 + t] = key;
            }
          }
        }
      }
    }
    if (has_next) {
      xreg.store(F);
      if (tile0 + 2 * kTile < t_end) xreg.load(xs, tile0 + 2 * kTile, tile_n(tile0 + 2 * kTile));
    }
    lds_barrier();                                                    // B2

    float f[C::TTW];
    if constexpr (C::NG > 1) {
#pragma unroll
      for (int tt = 0; tt < C::TTW; ++tt) f[tt] = fac[cgi * kTile + tile_token(gt0 + tt, c)];
    } else {
#pragma unroll
      for (int tt = 0; tt < C::TTW; ++tt) {
        const int tok = tile_token(gt0 + tt, c);
        f[tt] = MODE == 0 ? fast_rcp(dn[tt] + a.eps * l[tt]) : fast_rcp(l[tt]);
        if (want_assign && g == 0 && tok < nvalid) {
          if constexpr (MODE == 2) {
            if ((unsigned)am[tt] < (unsigned)C::Kp) atomicAdd(&hist[am[tt]], 1);
          } else {
            a.assign[(size_t)bh * a.N + tile0 + tok] = am[tt];
          }
        }
      }
    }

    if constexpr (MODE == 2) {
#pragma unroll
      for (int tt = 0; tt < C::TTW; ++tt) {
        if (tile_token(gt0 + tt, c) < nvalid) {
#pragma unroll
          for (int ct = 0; ct < C::CPW; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float gm = S[tt][ct][i] * f[tt];      // exactly 0 for padded components
              dsum[ct][i] += gm;
              dcnt[ct][i] += gm > a.thr ? 1.f : 0.f;
              dent += gm > 0.f ? gm * __logf(gm) : 0.f;
            }
        }
      }
    } else if constexpr (MODE == 1) {
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
    } else {
      // Gamma'' = responsibilities already divided by the read-out denominator,
      // -> LDS [token][component]
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
      lds_barrier();                                                  // B3

      // O^T = V~^T Gamma''^T for this wave's (token tile, d tile) share: lane
      // column = token, rows = four consecutive d, written as 8 (bf16) or 16
      // (fp32) contiguous bytes
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
        if (rtok < nvalid) {
#pragma unroll
          for (int j = 0; j < C::DPW; ++j) {
            const int dt = C::DVT >= C::NG ? cgi * C::DPW + j : cgi % C::DVT;
            const size_t off = ((size_t)bh * a.N + tile0 + rtok) * C::DV + dt * 16 + 4 * g;
            if (a.out_bf) {
              bf16x4 o4;
#pragma unroll
              for (int i = 0; i < 4; ++i) o4[i] = to_bf16(acc[j][i]);
              *reinterpret_cast<bf16x4*>(reinterpret_cast<bf16*>(a.out) + off) = o4;
            } else {
              st16(reinterpret_cast<float*>(a.out) + off, acc[j]);
            }
          }
        }
      }
    }
  }

  if constexpr (MODE == 2) {
    // over the 16 token columns of a lane row (DPP), then over the token
    // groups in a fixed order; counts are exact in fp32 (< 2^24 per workgroup)
#pragma unroll
    for (int ct = 0; ct < C::CPW; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float s1 = row16_sum(dsum[ct][i]), s2 = row16_sum(dcnt[ct][i]);
        const int comp = (cgi * C::CPW + ct) * 16 + 4 * g + i;
        if (c == 0) {
          dred[(2 * tg) * C::Kp + comp] = s1;
          dred[(2 * tg + 1) * C::Kp + comp] = s2;
        }
      }
    const float e = groups_sum(row16_sum(dent));
    if (lane == 0) dred[2 * C::TG * C::Kp + wave] = e;
    lds_barrier();
    float* out = a.diag + ((size_t)bh * gridDim.x + split) * (3 * C::Kp + 4);
    for (int k = threadIdx.x; k < C::Kp; k += kThreads) {
      float s1 = 0.f, s2 = 0.f;
#pragma unroll
      for (int q = 0; q < C::TG; ++q) {
        s1 += dred[(2 * q) * C::Kp + k];
        s2 += dred[(2 * q + 1) * C::Kp + k];
      }
      out[k] = s1;
      out[C::Kp + k] = s2;
      out[2 * C::Kp + k] = (float)hist[k];
    }
    if (threadIdx.x == 0) {
      float e4 = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) e4 += dred[2 * C::TG * C::Kp + w];
      out[3 * C::Kp] = e4;
    }
  }
}

// ============================================================================
// Read-out, bf16 inputs, token-owner form.  Every wave owns 32 queries at a
// time and all K_pad components, so the per-query softmax and the read-out
// normaliser stay inside the wave: the main loop has no barrier and no LDS
// write.  The workgroup (8 waves) keeps two read-only tables in LDS:
//   coef  -- the score coefficients (A_hi, A_lo, B_hi, B_lo) as ready-made MFMA
//            A operands, component rows in the order pi below;
//   vtab  -- V~^T as MFMA A operands (bf16) plus one extra 16-row block holding
//            Z_hi, Z_lo and ones, so the same MFMAs that form Gamma V~ also form
//            the denominator sum_k e_k Z_k and the mass sum_k e_k.
// Scores use D[component][query].  Component row r of score tile ct is
// pi(ct, r) = 32 (ct / 2) + 8 (r / 4) + 4 (ct % 2) + r % 4, which puts the
// eight consecutive components 32p + 8g .. 32p + 8g + 7 of tiles 2p, 2p+1 in
// lane group g: exactly the B operand chunk of O^T = V~^T Gamma^T for
// contraction step p, so e = exp2(s - m) feeds the read-out straight from
// registers.  Likewise output row r of d tile dt is d = sigma(dt, r) (same
// pairing), so a lane holds eight consecutive outputs of one query: one
// 16-byte store per pair of d tiles.
// ============================================================================
template <class C>
struct Read2 {
  static constexpr int KP = C::Kp;                       // a multiple of 32 (a pair of tiles)
  static constexpr int CT = KP / 16;
  static constexpr int KS = KP / 32;
  static constexpr int NKS = C::DRP / 32;
  static constexpr int DVT = C::DV / 16;
  static constexpr int OT = DVT + 1;                     // + (Z_hi, Z_lo, 1) block
  static constexpr int COEF = CT * NKS * 4;              // 1 KB operand chunks
  static constexpr int VCH = OT * KS;
  static constexpr int LDS = (COEF + VCH) * 1024 + KP * 4;
  static_assert(LDS == read2_lds_bytes(C::DRP, C::DV, KP), "read-out LDS sizing");
  static constexpr bool kOK = C::kBF && C::Kp % 32 == 0 && C::DRP <= 64 && LDS <= kRead2MaxLds;
};
// Waves per SIMD of the read-out (one workgroup of 4 * WPE waves per compute
// unit): three where the registers allow (plain routing vectors), two for
// split ones (their features take more registers) and for the second half of
// a split K (it also holds the first half's partials).
template <bool XS, int HM = 0> constexpr int kRead2WPE = XS || HM == 2 ? 2 : 3;

// HM = 0: all components.  HM = 1, 2: the components koff .. koff + C::Kp - 1
// of the tables laid out for CF (K_pad = 2 C::Kp); the first half (HM = 1)
// leaves each query's numerator, denominator and maximum in qpart / qpart2,
// the second (HM = 2) rescales both halves to the larger maximum and writes O.
// AS: query assignments are written (a.assign non-null); a separate variant, so
// that the plain read-out carries none of the argmax code.
template <class C, bool XS, int HM = 0, class CF = C, bool AS = false>
__global__ void __launch_bounds__(256 * (kRead2WPE<XS, HM>), 1)
__attribute__((amdgpu_waves_per_eu((kRead2WPE<XS, HM>), (kRead2WPE<XS, HM>))))
gma_read2_kernel(BidirArgs a) {
  using R = Read2<C>;
  static_assert(HM == 0 || (!XS && CF::Kp == 2 * C::Kp && CF::DRP == C::DRP && R::DVT >= 2),
                "half read-out");
  constexpr int NW = 4 * kRead2WPE<XS, HM>;
  __shared__ __attribute__((aligned(16))) bf16x8 coef[R::COEF * 64];
  __shared__ __attribute__((aligned(16))) bf16x8 vtab[R::VCH * 64];
  __shared__ __attribute__((aligned(16))) float cperm[R::KP];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int64_t bh = blockIdx.y;
  const int h = (int)(bh % a.H);
  constexpr bool want_assign = AS;
  const int koff = HM ? a.koff : 0;

  // ---- tables: copies of what the prologue and the reduction wrote (a half:
  // its component tiles of the coefficients, its contraction steps of each
  // V~ block) ----
  {
    constexpr int KSF = CF::Kp / 32;                 // contraction steps of the stored table
    const char* tb = a.params + (size_t)h * a.head_bytes + a.head_bytes / 2;
    const bf16x8* src = reinterpret_cast<const bf16x8*>(tb) + (size_t)(koff / 16) * R::NKS * 4 * 64;
    for (int idx = threadIdx.x; idx < R::COEF * 64; idx += NW * 64) coef[idx] = src[idx];
    const float* cp = reinterpret_cast<const float*>(tb + (size_t)8 * CF::Kp * CF::DRP) + koff;
    for (int j = threadIdx.x; j < R::KP; j += NW * 64) cperm[j] = cp[j];
    const bf16x8* vsrc = a.vtab + (size_t)bh * R::OT * KSF * 64 + (koff / 32) * 64;
    for (int idx = threadIdx.x; idx < R::VCH * 64; idx += NW * 64) {
      const int blk = idx / (R::KS * 64), rem = idx - blk * (R::KS * 64);
      vtab[idx] = vsrc[blk * KSF * 64 + rem];
    }
  }
  __syncthreads();

  // ---- queries: groups of 32, wave w takes groups w, w + 8, ... of this split ----
  const int64_t G32 = (a.N + 31) / 32;
  const int64_t gpw = (G32 + gridDim.x - 1) / gridDim.x;
  const int64_t gb = (int64_t)blockIdx.x * gpw;
  const int64_t ge = gb + gpw < G32 ? gb + gpw : G32;
  const bf16* xs = reinterpret_cast<const bf16*>(a.x) + (size_t)bh * a.N * C::DR;
  bf16* out = reinterpret_cast<bf16*>(a.out) + (size_t)bh * a.N * C::DV;

  // lane (c, g) of query tile tt holds query tok0 + 16 tt + c, routing columns
  // 32 s + 8 g .. + 7
  const bf16* xls = XS ? reinterpret_cast<const bf16*>(a.x_lo) + (size_t)bh * a.N * C::DR : xs;
  bf16x8 xr[2][R::NKS], xl[2][R::NKS];
  auto load_x = [&](int64_t grp) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int64_t tok = grp * 32 + 16 * tt + c;
#pragma unroll
      for (int s = 0; s < R::NKS; ++s) {
        const int col = 32 * s + 8 * g;
        if (tok < a.N && col < C::DR) {
          xr[tt][s] = ld16<bf16x8>(xs + (size_t)tok * C::DR + col);
          if constexpr (XS) xl[tt][s] = ld16<bf16x8>(xls + (size_t)tok * C::DR + col);
        } else {
          xr[tt][s] = bf16x8{};
          if constexpr (XS) xl[tt][s] = bf16x8{};
        }
      }
    }
  };
  int64_t grp = gb + wave;
  if (grp < ge) load_x(grp);
  for (; grp < ge; grp += NW) {
    // the tables are loop-invariant: keep the compiler from hoisting all of
    // their reads (far more registers than a wave has) out of the loop
    asm volatile("" ::: "memory");
    // scores, two component tiles at a time (four independent accumulators)
    f32x4 S[2][R::CT];
#pragma unroll
    for (int ct = 0; ct < R::CT; ++ct) {
      const f32x4 cs = *reinterpret_cast<const f32x4*>(&cperm[ct * 16 + 4 * g]);
      S[0][ct] = cs;
      S[1][ct] = cs;
    }
    // steps j = (routing chunk s outer, tile pair inner): the features of one
    // routing chunk are live at a time.  With three waves per SIMD the other
    // waves cover the LDS latency of each step's operands; with two, the
    // operands of step j + 1 are read while the MFMAs of step j run.
    constexpr int NCP = R::CT / 2;
    constexpr int NSTEP = NCP * R::NKS;
    constexpr int NBUF = kRead2WPE<XS, HM> >= 3 ? 1 : 2;
    auto load_w = [&](int j, bf16x8 (&w)[2][4]) {
      const int cp = 2 * (j % NCP), s = j / NCP;
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int ar = 0; ar < 4; ++ar) w[u][ar] = coef[(((cp + u) * R::NKS + s) * 4 + ar) * 64 + lane];
    };
    bf16x8 wbuf[NBUF][2][4];
    bf16x8 f[2][NFX<XS>];
    if constexpr (NBUF == 2) load_w(0, wbuf[0]);
#pragma unroll
    for (int j = 0; j < NSTEP; ++j) {
      const int cp = 2 * (j % NCP), s = j / NCP;
      if (j % NCP == 0) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) make_features<XS>(xr[tt][s], xl[tt][s], f[tt]);
        if (s == R::NKS - 1 && grp + NW < ge) load_x(grp + NW);
      }
      if constexpr (NBUF == 2) {
        if (j + 1 < NSTEP) load_w(j + 1, wbuf[(j + 1) & 1]);
        // keep the prefetch one full step ahead of its use
        __builtin_amdgcn_sched_barrier(0);
      } else {
        load_w(j, wbuf[0]);
      }
      bf16x8 (&w)[2][4] = wbuf[NBUF == 2 ? (j & 1) : 0];
#pragma unroll
      for (int q = 0; q < NQX<XS>; ++q)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int u = 0; u < 2; ++u)
            S[tt][cp + u] = mma(w[u][kWI[q]], f[tt][kFI[q]], S[tt][cp + u]);
      if constexpr (NBUF == 2) __builtin_amdgcn_sched_barrier(0);
    }

    // per query: max over components (in-lane, then across the four lane
    // groups), e = exp2(s - m) packed as the read-out operand
    bf16x8 E[2][R::KS];
    int am[2] = {0, 0};
    float mx[2], bvs[2] = {0.f, 0.f};
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      float v = S[tt][0][0];
#pragma unroll
      for (int ct = 0; ct < R::CT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) v = fmaxf(v, S[tt][ct][i]);
      const float m = groups_max(v);
      mx[tt] = m;
      if (want_assign) {
        // the lowest component index whose score equals the maximum m (m is
        // one of the scores: the maxima select, they do not round)
        int bi = 0x7fffffff;
#pragma unroll
        for (int ct = 0; ct < R::CT; ++ct)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            bi = min(bi, S[tt][ct][i] == m ? koff + pair_row(ct, 4 * g + i) : 0x7fffffff);
        am[tt] = groups_min_i(bi);
        bvs[tt] = m;
      }
#pragma unroll
      for (int p = 0; p < R::KS; ++p)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          E[tt][p][i] = to_bf16(exp2_fast(S[tt][2 * p][i] - m));
          E[tt][p][4 + i] = to_bf16(exp2_fast(S[tt][2 * p + 1][i] - m));
        }
    }

    // second half: the first half's partials of this lane's queries, in flight
    // during the contraction below
    f32x4 pnum[2][HM == 2 ? R::DVT : 1];
    f32x4 pq[2] = {f32x4{1.f, 0.f, 0.f, 0.f}, f32x4{1.f, 0.f, 0.f, 0.f}};
    if constexpr (HM == 2) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int64_t tok = grp * 32 + 16 * tt + c;
#pragma unroll
        for (int dt = 0; dt < R::DVT; ++dt) pnum[tt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (tok < a.N) {
          const size_t qt = (size_t)bh * a.N + tok;
          const float* prow = a.qpart + qt * C::DV + 8 * g;
#pragma unroll
          for (int qd = 0; qd < R::DVT / 2; ++qd) {
            pnum[tt][2 * qd] = *reinterpret_cast<const f32x4*>(prow + 32 * qd);
            pnum[tt][2 * qd + 1] = *reinterpret_cast<const f32x4*>(prow + 32 * qd + 4);
          }
          pq[tt] = *reinterpret_cast<const f32x4*>(a.qpart2 + qt);
        }
      }
    }

    // O^T (and the denominator block) = V~^T E^T
    f32x4 O[2][R::OT];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int dt = 0; dt < R::OT; ++dt) O[tt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // contraction step p outermost: consecutive MFMAs update different blocks
    constexpr int NV = R::OT * R::KS;
    auto vidx = [&](int j) { return ((j % R::OT) * R::KS + j / R::OT) * 64 + lane; };
    bf16x8 vb[4];
#pragma unroll
    for (int j = 0; j < 3 && j < NV; ++j) vb[j] = vtab[vidx(j)];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      if (j + 3 < NV) vb[(j + 3) & 3] = vtab[vidx(j + 3)];
      __builtin_amdgcn_sched_barrier(0);
      const int dt = j % R::OT, p = j / R::OT;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) O[tt][dt] = mma(vb[j & 3], E[tt][p], O[tt][dt]);
      __builtin_amdgcn_sched_barrier(0);
    }

    // O_i = num_i / (D_i + eps L_i); rows 0..2 of the last block (lane group 0)
    // hold Z_hi . e, Z_lo . e and sum e
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const f32x4 dz = O[tt][R::DVT];
      float den = dz[0] + dz[1] + a.eps * dz[2];
      float r0, r1;
      pair_xor16(den, r0, r1);
      pair_xor32(r0, den, r1);        // every lane: the value of lane group 0
      const int64_t tok = grp * 32 + 16 * tt + c;
      if constexpr (HM == 1) {
        if (tok < a.N) {
          const size_t qt = (size_t)bh * a.N + tok;
          float* prow = a.qpart + qt * C::DV + 8 * g;
#pragma unroll
          for (int qd = 0; qd < R::DVT / 2; ++qd) {
            *reinterpret_cast<f32x4*>(prow + 32 * qd) = O[tt][2 * qd];
            *reinterpret_cast<f32x4*>(prow + 32 * qd + 4) = O[tt][2 * qd + 1];
          }
          if (g == 0) a.qpart2[qt] = float4{den, mx[tt], bvs[tt], __int_as_float(am[tt])};
        }
      } else {
        // second half: both halves rescaled to the larger maximum
        float s0 = 0.f, s1 = 1.f;
        if constexpr (HM == 2) {
          const float M = fmaxf(mx[tt], pq[tt][1]);
          s0 = exp2_fast(pq[tt][1] - M);
          s1 = exp2_fast(mx[tt] - M);
          den = s0 * pq[tt][0] + s1 * den;
        }
        const float r = fast_rcp(den);
        s0 *= r;
        s1 *= r;
        if (tok < a.N) {
          bf16* orow = out + (size_t)tok * C::DV;
          if constexpr (R::DVT >= 2) {
#pragma unroll
            for (int qd = 0; qd < R::DVT / 2; ++qd) {
              bf16x8 o8;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                if constexpr (HM == 2) {
                  o8[i] = to_bf16(O[tt][2 * qd][i] * s1 + pnum[tt][2 * qd][i] * s0);
                  o8[4 + i] = to_bf16(O[tt][2 * qd + 1][i] * s1 + pnum[tt][2 * qd + 1][i] * s0);
                } else {
                  o8[i] = to_bf16(O[tt][2 * qd][i] * s1);
                  o8[4 + i] = to_bf16(O[tt][2 * qd + 1][i] * s1);
                }
              }
              st16(orow + 32 * qd + 8 * g, o8);
            }
          } else {
            bf16x4 o4;
#pragma unroll
            for (int i = 0; i < 4; ++i) o4[i] = to_bf16(O[tt][0][i] * s1);
            *reinterpret_cast<bf16x4*>(orow + 4 * g) = o4;
          }
          // the lowest component at the overall maximum: the first half's on a tie
          if (want_assign && g == 0)
            a.assign[(size_t)bh * a.N + tok] =
                HM == 2 && !(bvs[tt] > pq[tt][2]) ? __float_as_int(pq[tt][3]) : am[tt];
        }
      }
    }
  }
}

// ============================================================================
// Latent write, bf16 inputs, component-owner form with responsibilities kept
// in registers.  Wave (cgi, tg) holds the coefficients of component group cgi
// (CPW tiles) and scores the tokens of its token group in the layout
// D[token][component], rows in tile_token order: lane group g of key tiles 2P,
// 2P + 1 then holds keys 32P + 8g .. 32P + 8g + 7 of one component, which is
// the A operand of V~ += Gamma^T V with no transpose.  Per-token statistics
// over the wave's components (16-lane row reductions) are combined across the
// NG groups through LDS by all threads; V tiles are copied HBM -> LDS directly
// into a double buffer.  Two barriers per 64-token tile; small enough in
// registers and LDS for two workgroups per compute unit.
// ============================================================================
template <class C>
struct Write3 {
  static constexpr int VROWCH = C::DV / 8;
  static constexpr int VROUNDS = kTile * VROWCH / 64;           // 1 KB wave copies per V tile
  static constexpr int VRPW = (VROUNDS + kWaves - 1) / kWaves;
  static constexpr bool kOK = C::kBF && C::NG >= 2 && C::TTW % 2 == 0 && C::DV >= 32;
};

template <class C>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
gma_write3_kernel(BidirArgs a) {
  using R = Write3<C>;
  constexpr int TTW = C::TTW, CPW = C::CPW, NG = C::NG;
  __shared__ __attribute__((aligned(16))) bf16 F[3 * C::FAS];
  __shared__ __attribute__((aligned(16))) bf16 Vr[2][kTile * C::DV];
  __shared__ __attribute__((aligned(16))) f32x4 stats[NG * kTile];
  __shared__ __attribute__((aligned(16))) float fac[NG * kTile];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int cgi = wave % NG, tg = wave / NG;
  const int gt0 = tg * TTW;
  const int64_t bh = blockIdx.y;
  const int h = (int)(bh % a.H);
  const int64_t t_begin = (int64_t)blockIdx.x * a.tiles_per_split * kTile;
  const int64_t t_end = a.N < t_begin + (int64_t)a.tiles_per_split * kTile
                            ? a.N : t_begin + (int64_t)a.tiles_per_split * kTile;
  const int ntiles = t_end > t_begin ? (int)((t_end - t_begin + kTile - 1) / kTile) : 0;
  const bool want_assign = a.assign != nullptr;

  const char* pbase = a.params + (size_t)h * a.head_bytes;
  bf16x8 W[CPW][C::NKS][4];
  load_w<C>(pbase, cgi * CPW, W);
  float cv[CPW];
  {
    const float* cvec = reinterpret_cast<const float*>(pbase + (size_t)8 * C::Kp * C::DRP);
#pragma unroll
    for (int ct = 0; ct < CPW; ++ct) cv[ct] = cvec[(cgi * CPW + ct) * 16 + c];
  }
  const bf16* fb[TTW];
#pragma unroll
  for (int tt = 0; tt < TTW; ++tt) fb[tt] = F + C::frow(tile_token(gt0 + tt, c)) + g * 8;

  const bf16* xs = reinterpret_cast<const bf16*>(a.x) + (size_t)bh * a.N * C::DR;
  const bf16* vs = reinterpret_cast<const bf16*>(a.v) + (size_t)bh * a.N * C::DV;
  auto tile_start = [&](int k) { return t_begin + (int64_t)k * kTile; };
  auto tile_valid = [&](int k) {
    const int64_t r = t_end - tile_start(k);
    return (int)(r < kTile ? r : kTile);
  };
  auto load_v = [&](int k, int buf) {
    const int64_t t0 = tile_start(k);
    const int nv = tile_valid(k);
#pragma unroll
    for (int j = 0; j < R::VRPW; ++j) {
      const int round = wave * R::VRPW + j;
      if (round < R::VROUNDS) {
        const int P = round * 64 + lane;
        const int r = P / R::VROWCH, pc = P - r * R::VROWCH;
        const int lc = pc ^ ((2 * r) & (R::VROWCH - 2));
        const int rr = r < nv ? r : nv - 1;                 // tail rows repeat a valid row
        global_to_lds16(vs + (size_t)(t0 + rr) * C::DV + lc * 8, &Vr[buf][round * 512]);
      }
    }
  };

  f32x4 vacc[CPW][C::DVT], vz[CPW];
#pragma unroll
  for (int ct = 0; ct < CPW; ++ct) {
    vz[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < C::DVT; ++dt) vacc[ct][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (bf16)1.0f;

  FeatureTile<C> kreg;
  if (ntiles > 0) {
    kreg.load(xs, tile_start(0), tile_valid(0));
    load_v(0, 0);
    kreg.store(F);
    if (ntiles > 1) kreg.load(xs, tile_start(1), tile_valid(1));
    lds_barrier();
  }

  for (int k = 0; k < ntiles; ++k) {
    const int64_t tile0 = tile_start(k);
    const int nvalid = tile_valid(k);
    const int buf = k & 1;

    // scores D[token][component], independent accumulators back to back
    f32x4 S[TTW][CPW];
#pragma unroll
    for (int tt = 0; tt < TTW; ++tt)
#pragma unroll
      for (int ct = 0; ct < CPW; ++ct) S[tt][ct] = f32x4{cv[ct], cv[ct], cv[ct], cv[ct]};
    {
      constexpr int WI[5] = {0, 0, 1, 2, 3};
      constexpr int FI[5] = {0, 1, 0, 2, 2};
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        constexpr int NT = TTW / 2;
        bf16x8 f[C::NKS][NT][3];
#pragma unroll
        for (int s = 0; s < C::NKS; ++s)
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const bf16* fp = fb[h2 * NT + t] + s * C::CS;
            f[s][t][0] = ld16<bf16x8>(fp);
            f[s][t][1] = ld16<bf16x8>(fp + C::FAS);
            f[s][t][2] = ld16<bf16x8>(fp + 2 * C::FAS);
          }
#pragma unroll
        for (int s = 0; s < C::NKS; ++s)
#pragma unroll
          for (int q = 0; q < 5; ++q)
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
              for (int ct = 0; ct < CPW; ++ct)
                S[h2 * NT + t][ct] = mma(f[s][t][FI[q]], W[ct][s][WI[q]], S[h2 * NT + t][ct]);
      }
    }

    // per token (row 4g + i of tile tt): max and sum over this wave's components
#pragma unroll
    for (int tt = 0; tt < TTW; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float m = S[tt][0][i];
#pragma unroll
        for (int ct = 1; ct < CPW; ++ct) m = fmaxf(m, S[tt][ct][i]);
        m = row16_max(m);
        int am = 0;
        if (want_assign) {
          float bv = S[tt][0][i];
          am = (cgi * CPW) * 16 + c;
#pragma unroll
          for (int ct = 1; ct < CPW; ++ct) argmax_merge(bv, am, S[tt][ct][i], (cgi * CPW + ct) * 16 + c);
          row16_argmax(bv, am);
        }
        const float mref = m == -INFINITY ? 0.f : m;      // all-padding group: every e is 0
        float l = 0.f;
#pragma unroll
        for (int ct = 0; ct < CPW; ++ct) {
          const float e = exp2_fast(S[tt][ct][i] - mref);
          S[tt][ct][i] = e;
          l += e;
        }
        l = row16_sum(l);
        if (c == 0) stats[cgi * kTile + tile_token(gt0 + tt, 4 * g + i)] = f32x4{m, l, 0.f, __int_as_float(am)};
      }
    lds_barrier();                                                    // B1

    // combine the NG groups of every token (thread (token, q), quad exchanges)
    if (threadIdx.x < kTile * NG) {
      const int t = threadIdx.x / NG, q = threadIdx.x % NG;
      const f32x4 st = stats[q * kTile + t];
      float M = st[0];
      M = fmaxf(M, dpp<0xB1>(M));
      if constexpr (NG == 4) M = fmaxf(M, dpp<0x4E>(M));
      const float fq = st[0] == -INFINITY ? 0.f : exp2_fast(st[0] - M);
      float L = fq * st[1];
      L += dpp<0xB1>(L);
      if constexpr (NG == 4) L += dpp<0x4E>(L);
      fac[q * kTile + t] = t < nvalid ? fq * fast_rcp(L) : 0.f;
      if (want_assign) {
        int key = st[0] == M ? __float_as_int(st[3]) : 0x7fffffff;
        key = min(key, dpp_i<0xB1>(key));
        if constexpr (NG == 4) key = min(key, dpp_i<0x4E>(key));
        if (q == 0 && t < nvalid) a.assign[(size_t)bh * a.N + tile0 + t] = key;
      }
    }
    if (k + 1 < ntiles) kreg.store(F);
    wait_global_loads();                 // this wave's copies of V(k)
    if (k + 1 < ntiles) load_v(k + 1, buf ^ 1);
    if (k + 2 < ntiles) kreg.load(xs, tile_start(k + 2), tile_valid(k + 2));
    lds_barrier();                                                    // B2

    // Gamma = e * fac (bf16) as the A operand of V~ += Gamma^T V
    bf16x8 A[CPW][TTW / 2];
#pragma unroll
    for (int tt = 0; tt < TTW; ++tt) {
      const f32x4 f4 = *reinterpret_cast<const f32x4*>(&fac[cgi * kTile + tile_token(gt0 + tt, 4 * g)]);
#pragma unroll
      for (int ct = 0; ct < CPW; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) A[ct][tt >> 1][4 * (tt & 1) + i] = to_bf16(S[tt][ct][i] * f4[i]);
    }
#pragma unroll
    for (int P = 0; P < TTW / 2; ++P) {
      const int tok0 = 32 * ((gt0 >> 1) + P);
#pragma unroll
      for (int ct = 0; ct < CPW; ++ct) vz[ct] = mma(A[ct][P], ones, vz[ct]);
#pragma unroll
      for (int dt = 0; dt < C::DVT; ++dt) {
        const bf16x8 Bv = tr_chunk_swz<R::VROWCH>(Vr[buf], tok0, dt * 16);
#pragma unroll
        for (int ct = 0; ct < CPW; ++ct) vacc[ct][dt] = mma(A[ct][P], Bv, vacc[ct][dt]);
      }
    }
  }

  // partial (V~, Z) of this (split, token group)
  const size_t pslot = ((size_t)bh * a.S + blockIdx.x) * C::TG + tg;
  float* pv = a.partial + pslot * C::Kp * C::DV;
  float* pz = a.partial_z + pslot * C::Kp;
#pragma unroll
  for (int ct = 0; ct < CPW; ++ct) {
    const int comp0 = (cgi * CPW + ct) * 16;
#pragma unroll
    for (int dt = 0; dt < C::DVT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) pv[(comp0 + 4 * g + i) * C::DV + dt * 16 + c] = vacc[ct][dt][i];
    if (c == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) pz[comp0 + 4 * g + i] = vz[ct][i];
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
  a.vtab = reinterpret_cast<const bf16x8*>(t.ws + p.off_vtab);
  a.N = p.N;
  a.H = (int)p.H;
  a.K = p.K;
  a.S = p.S;
  a.tiles_per_split = p.tiles_per_split;
  a.eps = t.eps;
  a.out_bf = p.out_bf ? 1 : 0;
  const dim3 grid(p.S, (unsigned)p.BH);

  const bool split = t.k_lo != nullptr;
  a.x = t.k;
  a.x_lo = t.k_lo;
  a.v = t.v;
  a.assign = t.assign_k;
  // token-owner write: about one workgroup per compute unit (two where two
  // waves fit on a SIMD), each at least four 32-key groups; its splits
  // replace the plan's (the partial buffer holds S * TG >= this many slots per
  // sequence).  Split routing vectors (the
  // layer's projections) run only on the token-owner kernels.
  int PS = C::kBF ? p.S : p.S * C::TG;          // partial slots per sequence
  // K_pad = 256 where the read-out's tables exceed LDS: it runs once per half
  // of the components (CH)
  constexpr bool KHR = bidir_khalf(C::kBF, C::DRP, C::DV, C::Kp);
  using CH = Cfg<C::kBF, (C::CPW > 1 ? C::CPW / 2 : 1), C::NG, C::DR, C::DV>;
  static_assert(!KHR || (Read2<CH>::kOK && CH::Kp * 2 == C::Kp), "half read-out");
  if (split && !((WriteTeam<C>::kOK || Write2<C>::kOK) && Read2<C>::kOK))
    return hipErrorNotSupported;
  if (g_launch_hook) g_launch_hook("gma_write", s, 1);
  if constexpr (WriteTeam<C>::kOK) {
    // team write (K_pad 128 or 256): one eight-wave workgroup per compute
    // unit, each team at least two 32-key groups
    const int64_t g32 = (p.N + 31) / 32;
    int64_t s2 = (256 + p.BH - 1) / p.BH;
    const int64_t cap = (g32 + 2 * WriteTeam<C>::NT - 1) / (2 * WriteTeam<C>::NT);
    if (s2 > cap) s2 = cap;
    if (s2 > PS) s2 = PS;
    if (s2 < 1) s2 = 1;
    PS = (int)s2;
    const dim3 g2((unsigned)s2, (unsigned)p.BH);
    if (a.assign) {
      if (split) hipLaunchKernelGGL((gma_write_team_kernel<C, true, true>), g2, dim3(512), 0, s, a);
      else hipLaunchKernelGGL((gma_write_team_kernel<C, false, true>), g2, dim3(512), 0, s, a);
    } else {
      if (split) hipLaunchKernelGGL((gma_write_team_kernel<C, true, false>), g2, dim3(512), 0, s, a);
      else hipLaunchKernelGGL((gma_write_team_kernel<C, false, false>), g2, dim3(512), 0, s, a);
    }
  } else if constexpr (Write2<C>::kOK) {
    const int64_t g32 = (p.N + 31) / 32;
    int64_t s2 = (256 * Write2<C>::WPE + p.BH - 1) / p.BH;
    const int64_t cap = (g32 + 3) / 4;
    if (s2 > cap) s2 = cap;
    if (s2 > PS) s2 = PS;
    if (s2 < 1) s2 = 1;
    PS = (int)s2;
    const dim3 g2((unsigned)s2, (unsigned)p.BH);
    if (split) hipLaunchKernelGGL((gma_write2_kernel<C, true>), g2, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((gma_write2_kernel<C, false>), g2, dim3(256), 0, s, a);
  } else if constexpr (Write3<C>::kOK) {
    PS = p.S * C::TG;
    hipLaunchKernelGGL(gma_write3_kernel<C>, grid, dim3(kThreads), 0, s, a);
  } else if constexpr (C::kBF) {
    hipLaunchKernelGGL(gma_write_bf16_kernel<C>, grid, dim3(kThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL(gma_write_kernel<C>, grid, dim3(kThreads), 0, s, a);
  }
  if (g_launch_hook) g_launch_hook("gma_write", s, 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int nred = C::Kp * C::DV / 8 + C::Kp;
  if (g_launch_hook) g_launch_hook("gma_reduce", s, 1);
  hipLaunchKernelGGL(gma_reduce_kernel, dim3((nred + 255) / 256, (unsigned)p.BH), dim3(256), 0, s,
                     a.partial, a.partial_z, PS, C::Kp, C::DV,
                     reinterpret_cast<float*>(t.ws + p.off_vt),
                     reinterpret_cast<float*>(t.ws + p.off_z),
                     (Read2<C>::kOK || KHR) && !t.state_v
                         ? reinterpret_cast<bf16*>(t.ws + p.off_vtab)
                         : nullptr,
                     t.state_v, t.state_z, p.K);
  if (g_launch_hook) g_launch_hook("gma_reduce", s, 0);
  e = hipGetLastError();
  // a prefix state stops here: V~ and Z are the state after the last key
  if (e != hipSuccess || t.state_v) return e;

  a.x = t.q;
  a.x_lo = t.q_lo;
  a.v = nullptr;
  a.out = t.out;
  a.assign = t.assign_q;
  if (g_launch_hook) g_launch_hook("gma_read", s, 1);
  if constexpr (KHR) {
    // the first half leaves its partials, the second combines them; grids as
    // below
    const int64_t g32 = (p.N + 31) / 32;
    int64_t s2 = (256 + p.BH - 1) / p.BH;
    const int64_t cap = (g32 + 7) / 8;
    if (s2 > cap) s2 = cap;
    if (s2 < 1) s2 = 1;
    a.qpart = reinterpret_cast<float*>(t.ws + p.off_qpart);
    a.qpart2 = reinterpret_cast<float4*>(t.ws + p.off_qpart2);
    const dim3 gr((unsigned)s2, (unsigned)p.BH);
    a.koff = 0;
    if (a.assign)
      hipLaunchKernelGGL((gma_read2_kernel<CH, false, 1, C, true>), gr, dim3(256 * kRead2WPE<false, 1>), 0, s, a);
    else
      hipLaunchKernelGGL((gma_read2_kernel<CH, false, 1, C>), gr, dim3(256 * kRead2WPE<false, 1>), 0, s, a);
    a.koff = CH::Kp;
    if (a.assign)
      hipLaunchKernelGGL((gma_read2_kernel<CH, false, 2, C, true>), gr, dim3(256 * kRead2WPE<false, 2>), 0, s, a);
    else
      hipLaunchKernelGGL((gma_read2_kernel<CH, false, 2, C>), gr, dim3(256 * kRead2WPE<false, 2>), 0, s, a);
  } else if constexpr (Read2<C>::kOK) {
    // about one workgroup per compute unit, at least eight 32-query groups each
    const int64_t g32 = (p.N + 31) / 32;
    int64_t s2 = (256 + p.BH - 1) / p.BH;
    const int64_t cap = (g32 + 7) / 8;
    if (s2 > cap) s2 = cap;
    if (s2 < 1) s2 = 1;
    const dim3 gr((unsigned)s2, (unsigned)p.BH);
    if (split) {
      if (a.assign) hipLaunchKernelGGL((gma_read2_kernel<C, true, 0, C, true>), gr, dim3(256 * kRead2WPE<true>), 0, s, a);
      else hipLaunchKernelGGL((gma_read2_kernel<C, true>), gr, dim3(256 * kRead2WPE<true>), 0, s, a);
    } else {
      if (a.assign) hipLaunchKernelGGL((gma_read2_kernel<C, false, 0, C, true>), gr, dim3(256 * kRead2WPE<false>), 0, s, a);
      else hipLaunchKernelGGL((gma_read2_kernel<C, false>), gr, dim3(256 * kRead2WPE<false>), 0, s, a);
    }
  } else {
    hipLaunchKernelGGL((gma_read_kernel<C, 0>), grid, dim3(kThreads), 0, s, a);
  }
  if (g_launch_hook) g_launch_hook("gma_read", s, 0);
  return hipGetLastError();
}

template <class C>
static void launch_resp_kernel(const Plan& p, const BidirArgs& a, hipStream_t s);

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
  launch_resp_kernel<C>(p, a, s);
  if (g_launch_hook) g_launch_hook("gma_resp", s, 0);
  return hipGetLastError();
}

// ============================================================================
// Usage statistics, token-owner form (bf16 routing vectors, K_pad a multiple of
// 32, d_r <= 64): the latent write's key loop without the values.  Every wave
// owns 32 tokens at a time and all components: scores on MFMA from the
// coefficient table in LDS, the per-token softmax inside the wave, and per
// lane, for the components of its column, the sums of gamma and of gamma >
// thr, per token sum_k gamma ln gamma from the softmax's own sums, and an LDS
// histogram of the assignments.  With
// no V~ in the accumulation registers it runs two waves per SIMD.  One record
// of 3 K_pad + 4 floats per workgroup, as the component-owner statistics pass.
// MODE 1 writes the responsibilities and assignments instead (a.gamma
// [BH][N][K], a.assign [BH][N], either may be null), with no statistics.
// ============================================================================
template <class C>
struct Usage2 {
  static constexpr int KP = C::Kp;
  static constexpr int CT = KP / 16;
  static constexpr int NKS = C::DRP / 32;
  static constexpr int COEF = CT * NKS * 4;
  static constexpr int LDS = COEF * 1024 + KP * 4 + KP * 4 + 4 * (3 * KP + 1) * 4;
  // two workgroups per compute unit where the tables allow, else one (K_pad 256
  // with d_r = 64)
  static constexpr bool kOK = C::kBF && KP % 32 == 0 && C::DRP <= 64 && LDS <= 150 * 1024;
};

template <class C, int MODE>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
gma_usage2_kernel(BidirArgs a) {
  using R = Usage2<C>;
  constexpr int NW = 4;
  __shared__ __attribute__((aligned(16))) char lds[R::LDS];
  bf16x8* coef = reinterpret_cast<bf16x8*>(lds);
  float* cperm = reinterpret_cast<float*>(lds + R::COEF * 1024);
  int* hist = reinterpret_cast<int*>(lds + R::COEF * 1024 + R::KP * 4);
  float* red = reinterpret_cast<float*>(lds + R::COEF * 1024 + 2 * R::KP * 4);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int64_t bh = blockIdx.y;
  const int h = (int)(bh % a.H);
  {
    const char* tb = a.params + (size_t)h * a.head_bytes + a.head_bytes / 2;
    const bf16x8* src = reinterpret_cast<const bf16x8*>(tb);
    for (int idx = threadIdx.x; idx < R::COEF * 64; idx += NW * 64) coef[idx] = src[idx];
    const float* cp = reinterpret_cast<const float*>(tb + (size_t)8 * C::Kp * C::DRP);
    for (int j = threadIdx.x; j < R::KP; j += NW * 64) {
      cperm[j] = cp[j];
      hist[j] = 0;
    }
  }
  __syncthreads();

  const int64_t G32 = (a.N + 31) / 32;
  const int64_t gpw = (G32 + gridDim.x - 1) / gridDim.x;
  const int64_t gb = (int64_t)blockIdx.x * gpw;
  const int64_t ge = gb + gpw < G32 ? gb + gpw : G32;
  const bf16* xs = reinterpret_cast<const bf16*>(a.x) + (size_t)bh * a.N * C::DR;

  bf16x8 xr[2][R::NKS];
  auto load_x = [&](int64_t grp) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int64_t tok = grp * 32 + tile_token(tt, c);
#pragma unroll
      for (int s = 0; s < R::NKS; ++s) {
        const int col = 32 * s + 8 * g;
        const bool ok = tok < a.N && col < C::DR;
        const bf16x8 v = ld16<bf16x8>(xs + (size_t)(ok ? tok : 0) * C::DR + (ok ? col : 0));
        xr[tt][s] = ok ? v : bf16x8{};
      }
    }
  };

  float gsum[R::CT], gcnt[R::CT], gent = 0.f;
#pragma unroll
  for (int ct = 0; ct < R::CT; ++ct) gsum[ct] = gcnt[ct] = 0.f;

  int64_t grp = gb + wave;
  if (grp < ge) load_x(grp);
  for (; grp < ge; grp += NW) {
    bf16x8 f[2][R::NKS][NFX<false>];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int s = 0; s < R::NKS; ++s) make_features<false>(xr[tt][s], xr[tt][s], f[tt][s]);
    if (grp + NW < ge) load_x(grp + NW);

    f32x4 S[2][R::CT];
#pragma unroll
    for (int ct = 0; ct < R::CT; ++ct) {
      const float cv = cperm[ct * 16 + c];
      S[0][ct] = f32x4{cv, cv, cv, cv};
      S[1][ct] = S[0][ct];
    }
    // steps hs = (component tile, routing chunk): the four coefficient operands
    // of step hs + 1 are read from LDS while the MFMAs of step hs run
    constexpr int NH = R::CT * R::NKS;
    bf16x8 wbuf[2][4];
#pragma unroll
    for (int ar = 0; ar < 4; ++ar) wbuf[0][ar] = coef[ar * 64 + lane];
#pragma unroll
    for (int hs = 0; hs < NH; ++hs) {
      if (hs + 1 < NH) {
#pragma unroll
        for (int ar = 0; ar < 4; ++ar) wbuf[(hs + 1) & 1][ar] = coef[((hs + 1) * 4 + ar) * 64 + lane];
      }
      __builtin_amdgcn_sched_barrier(0);
      const int ct = hs / R::NKS, s = hs % R::NKS;
#pragma unroll
      for (int q = 0; q < NQX<false>; ++q)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
          S[tt][ct] = mma(f[tt][s][kFI[q]], wbuf[hs & 1][kWI[q]], S[tt][ct]);
      __builtin_amdgcn_sched_barrier(0);
    }

    // per token (row 4g + i of key tile tt): softmax over the CT columns of
    // this lane and the 16 lanes of its row; lane column c of tile ct is
    // component pair_row(ct, c)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t tok = grp * 32 + 8 * g + 4 * tt + i;
        const bool valid = tok < a.N;
        // the row maximum, then the lowest component index attaining it (in a
        // lane the component index grows with the tile)
        float m = S[tt][0][i];
#pragma unroll
        for (int ct = 1; ct < R::CT; ++ct) m = fmaxf(m, S[tt][ct][i]);
        m = row16_max(m);
        int bi = 0x7fffffff;
        if (MODE == 0 || a.assign != nullptr) {
#pragma unroll
          for (int ct = R::CT - 1; ct >= 0; --ct) bi = S[tt][ct][i] == m ? pair_row(ct, c) : bi;
          bi = min(bi, dpp_i<0xB1>(bi));
          bi = min(bi, dpp_i<0x4E>(bi));
          bi = min(bi, dpp_i<0x141>(bi));
          bi = min(bi, dpp_i<0x140>(bi));
        }
        // scores are in log2 units: with t = s - m, gamma = 2^t / l and
        // sum_k gamma ln gamma = ln 2 * sum_k 2^t t / l - ln l, one log per token
        float l = 0.f, et = 0.f;
#pragma unroll
        for (int ct = 0; ct < R::CT; ++ct) {
          const float tk = S[tt][ct][i] - m;
          const float e = exp2_fast(tk);
          S[tt][ct][i] = e;
          l += e;
          et += e > 0.f ? e * tk : 0.f;
        }
        l = row16_sum(l);
        const float inv = valid ? fast_rcp(l) : 0.f;
        if constexpr (MODE == 0) {
          et = row16_sum(et);
          if (valid && c == 0) gent += 0.69314718f * et * inv - __logf(l);
#pragma unroll
          for (int ct = 0; ct < R::CT; ++ct) {
            const float gm = S[tt][ct][i] * inv;
            gsum[ct] += gm;
            gcnt[ct] += (valid && gm > a.thr) ? 1.f : 0.f;
          }
          if (valid && c == 0 && (unsigned)bi < (unsigned)R::KP) atomicAdd(&hist[bi], 1);
        } else {
          if (valid && a.gamma != nullptr) {
            float* gr = a.gamma + ((size_t)bh * a.N + tok) * a.K;
#pragma unroll
            for (int ct = 0; ct < R::CT; ++ct) {
              const int comp = pair_row(ct, c);
              if (comp < a.K) gr[comp] = S[tt][ct][i] * inv;
            }
          }
          if (valid && c == 0 && a.assign != nullptr) a.assign[(size_t)bh * a.N + tok] = bi;
        }
      }
  }
  if constexpr (MODE == 1) return;

  // lanes of one column c hold different tokens: sum the four lane groups,
  // then the four waves in order
#pragma unroll
  for (int ct = 0; ct < R::CT; ++ct) {
    const float s1 = groups_sum(gsum[ct]), s2 = groups_sum(gcnt[ct]);
    if (g == 0) {
      red[(wave * 3 + 0) * R::KP + pair_row(ct, c)] = s1;
      red[(wave * 3 + 1) * R::KP + pair_row(ct, c)] = s2;
    }
  }
  const float e = groups_sum(row16_sum(gent));
  if (lane == 0) red[NW * 3 * R::KP + wave] = e;
  __syncthreads();
  float* out = a.diag + ((size_t)bh * gridDim.x + blockIdx.x) * (3 * C::Kp + 4);
  for (int k = threadIdx.x; k < R::KP; k += NW * 64) {
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      s1 += red[(w * 3 + 0) * R::KP + k];
      s2 += red[(w * 3 + 1) * R::KP + k];
    }
    out[k] = s1;
    out[C::Kp + k] = s2;
    out[2 * C::Kp + k] = (float)hist[k];
  }
  if (threadIdx.x == 0) {
    float e4 = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) e4 += red[NW * 3 * R::KP + w];
    out[3 * C::Kp] = e4;
  }
}

// Responsibilities and assignments of a.x: the token-owner kernel where it
// applies (about two workgroups per compute unit, at least four 32-token groups
// each), else the component-owner kernel.
template <class C>
static void launch_resp_kernel(const Plan& p, const BidirArgs& a, hipStream_t s) {
  if constexpr (Usage2<C>::kOK) {
    const int64_t g32 = (p.N + 31) / 32;
    int64_t s2 = (512 + p.BH - 1) / p.BH;
    const int64_t cap = (g32 + 3) / 4;
    if (s2 > cap) s2 = cap;
    if (s2 < 1) s2 = 1;
    hipLaunchKernelGGL((gma_usage2_kernel<C, 1>), dim3((unsigned)s2, (unsigned)p.BH), dim3(256), 0,
                       s, a);
  } else {
    hipLaunchKernelGGL((gma_read_kernel<C, 1>), dim3(p.S, (unsigned)p.BH), dim3(kThreads), 0, s, a);
  }
}

template <class C>
static hipError_t run_usage(const Plan& p, const Tensors& t, int& splits, hipStream_t s) {
  BidirArgs a{};
  a.params = t.ws + p.off_params;
  a.head_bytes = p.head_bytes;
  a.N = p.N;
  a.H = (int)p.H;
  a.K = p.K;
  a.S = p.S;
  a.tiles_per_split = p.tiles_per_split;
  a.x = t.q;
  a.diag = t.diag;
  a.thr = t.thr;
  if (g_launch_hook) g_launch_hook("gma_usage", s, 1);
  if constexpr (Usage2<C>::kOK) {
    // about two workgroups per compute unit, at least four 32-token groups each,
    // no more than the partial records the workspace holds (p.S per sequence)
    const int64_t g32 = (p.N + 31) / 32;
    int64_t s2 = (512 + p.BH - 1) / p.BH;
    const int64_t cap = (g32 + 3) / 4;
    if (s2 > cap) s2 = cap;
    if (s2 > p.S) s2 = p.S;
    if (s2 < 1) s2 = 1;
    splits = (int)s2;
    hipLaunchKernelGGL((gma_usage2_kernel<C, 0>), dim3((unsigned)s2, (unsigned)p.BH), dim3(256), 0,
                       s, a);
  } else {
    splits = p.S;
    hipLaunchKernelGGL((gma_read_kernel<C, 2>), dim3(p.S, (unsigned)p.BH), dim3(kThreads), 0, s,
                       a);
  }
  if (g_launch_hook) g_launch_hook("gma_usage", s, 0);
  return hipGetLastError();
}

// Per head: the usage statistics summed over batches and workgroups in a
// fixed order (counts exact), then the per-head figures.  One workgroup per head.
__global__ void __launch_bounds__(256) gma_usage_reduce_kernel(
    const float* __restrict__ diag, int64_t B, int H, int S, int Kp, int K, int64_t ntok,
    int32_t* __restrict__ counts, float* __restrict__ mean_gamma, float* __restrict__ util,
    float* __restrict__ head_stats) {
  __shared__ double r_ent[256];
  __shared__ double r_tok[256];
  __shared__ int r_used[256];
  const int h = blockIdx.x, t = threadIdx.x;
  const int W = 3 * Kp + 4;
  const double inv = 1.0 / (double)ntok;
  double ue = 0.0;
  int used = 0;
  for (int k = t; k < K; k += 256) {
    double gs = 0.0;
    int64_t n = 0, hc = 0;
    for (int64_t b = 0; b < B; ++b) {
      const float* row = diag + (size_t)(b * H + h) * S * W + k;
      // four workgroups' records loaded before they are added, in order
      int sp = 0;
      for (; sp + 4 <= S; sp += 4) {
        float v[4][3];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int c = 0; c < 3; ++c) v[u][c] = row[(size_t)(sp + u) * W + c * Kp];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          gs += v[u][0];
          n += (int64_t)v[u][1];
          hc += (int64_t)v[u][2];
        }
      }
      for (; sp < S; ++sp) {
        const float* base = row + (size_t)sp * W;
        gs += base[0];
        n += (int64_t)base[Kp];
        hc += (int64_t)base[2 * Kp];
      }
    }
    if (counts) counts[(size_t)h * K + k] = (int32_t)hc;
    if (mean_gamma) mean_gamma[(size_t)h * K + k] = (float)(gs * inv);
    if (util) util[(size_t)h * K + k] = (float)((double)n * inv);
    if (hc > 0) {
      const double pk = (double)hc * inv;
      ue -= pk * log(pk);
      ++used;
    }
  }
  // the workgroups' token-entropy sums: thread t takes records t, t + 256, ...
  // in order, then the same fixed-order tree as the other two sums
  double te = 0.0;
  for (int64_t r = t; r < B * S; r += 256) {
    const int64_t b = r / S, sp = r - b * S;
    te += diag[((size_t)(b * H + h) * S + sp) * W + 3 * Kp];
  }
  r_ent[t] = ue;
  r_used[t] = used;
  r_tok[t] = te;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (t < w) {
      r_ent[t] += r_ent[t + w];
      r_used[t] += r_used[t + w];
      r_tok[t] += r_tok[t + w];
    }
    __syncthreads();
  }
  if (t == 0 && head_stats) {
    head_stats[(size_t)h * 3 + 0] = (float)(-r_tok[0] * inv);
    head_stats[(size_t)h * 3 + 1] = K > 1 ? (float)(r_ent[0] / log((double)K)) : 0.f;
    head_stats[(size_t)h * 3 + 2] = (float)r_used[0];
  }
}

hipError_t launch_reduce_table(const float* partial, const float* partial_z, int PS, int64_t BH,
                               int Kp, int DV, float* vt, float* z, bf16* vtab, hipStream_t s) {
  if (DV < 32 || Kp % 32) return hipErrorInvalidValue;
  const int nred = Kp * DV / 8 + Kp;
  hipLaunchKernelGGL(gma_reduce_kernel, dim3((nred + 255) / 256, (unsigned)BH), dim3(256), 0, s,
                     partial, partial_z, PS, Kp, DV, vt, z, vtab, nullptr, nullptr, Kp);
  return hipGetLastError();
}

hipError_t launch_prologue(const Plan& p, const Tensors& t, hipStream_t s) {
  if (g_launch_hook) g_launch_hook("gma_prologue", s, 1);
  const int64_t rows = p.H * (int64_t)p.Kp;          // one wave per (head, component)
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (p.bf)
    hipLaunchKernelGGL(gma_prologue_kernel<true>, grid, dim3(256), 0, s, t.mu, t.ls2, t.lpi,
                       (int)p.H, p.K, p.Kp, p.DR, p.DRP, t.ws + p.off_params, p.head_bytes,
                       t.omega, t.alpha, t.eps_sigma);
  else
    hipLaunchKernelGGL(gma_prologue_kernel<false>, grid, dim3(256), 0, s, t.mu, t.ls2, t.lpi,
                       (int)p.H, p.K, p.Kp, p.DR, p.DRP, t.ws + p.off_params, p.head_bytes,
                       t.omega, t.alpha, t.eps_sigma);
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
    case 16: GMA_DR_CASES(FN, BF, 4, 4)                                     \
  }                                                                         \
  break;

template <class C>
static hipError_t split_query(const Plan&, const Tensors&, hipStream_t) {
  return Read2<C>::kOK && (WriteTeam<C>::kOK || Write2<C>::kOK) ? hipSuccess
                                                                 : hipErrorNotSupported;
}

static hipError_t split_query_all(const Plan& p, const Tensors& t, hipStream_t s) {
  switch (0) { default: GMA_GROUP_CASES(split_query, true) }
  return hipErrorNotSupported;
}

bool bidir_split_ok(const Plan& p) {
  return p.bf && split_query_all(p, Tensors{}, nullptr) == hipSuccess;
}

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
    case 16: GMA_RESP_DR_CASES(BF, 4, 4)                                    \
  }                                                                         \
  break;

#define GMA_USAGE_DR_CASES(BF, CPW, NG)                                     \
  switch (p.DR) {                                                           \
    case 16: e = run_usage<Cfg<BF, CPW, NG, 16, 16>>(p, t, splits, s); break;   \
    case 32: e = run_usage<Cfg<BF, CPW, NG, 32, 16>>(p, t, splits, s); break;   \
    case 64: e = run_usage<Cfg<BF, CPW, NG, 64, 16>>(p, t, splits, s); break;   \
    case 128: e = run_usage<Cfg<BF, CPW, NG, 128, 16>>(p, t, splits, s); break; \
  }                                                                         \
  break;
#define GMA_USAGE_CASES(BF)                                                 \
  switch (p.CT) {                                                           \
    case 1: GMA_USAGE_DR_CASES(BF, 1, 1)                                    \
    case 2: GMA_USAGE_DR_CASES(BF, 2, 1)                                    \
    case 4: GMA_USAGE_DR_CASES(BF, 2, 2)                                    \
    case 8: GMA_USAGE_DR_CASES(BF, 2, 4)                                    \
    case 16: GMA_USAGE_DR_CASES(BF, 4, 4)                                   \
  }                                                                         \
  break;

hipError_t launch_usage(const Plan& p, const Tensors& t, int32_t* counts, float* mean_gamma,
                        float* util, float* head_stats, hipStream_t s) {
  hipError_t e = hipErrorInvalidValue;
  int splits = p.S;
  if (p.bf) {
    switch (0) { default: GMA_USAGE_CASES(true) }
  } else {
    switch (0) { default: GMA_USAGE_CASES(false) }
  }
  if (e != hipSuccess) return e;
  if (g_launch_hook) g_launch_hook("gma_usage_reduce", s, 1);
  hipLaunchKernelGGL(gma_usage_reduce_kernel, dim3((unsigned)p.H), dim3(256), 0, s, t.diag, p.B,
                     (int)p.H, splits, p.Kp, p.K, p.B * p.N, counts, mean_gamma, util, head_stats);
  if (g_launch_hook) g_launch_hook("gma_usage_reduce", s, 0);
  return hipGetLastError();
}

hipError_t launch_resp(const Plan& p, const Tensors& t, hipStream_t s) {
  if (p.bf) {
    switch (0) { default: GMA_RESP_CASES(true) }
  } else {
    switch (0) { default: GMA_RESP_CASES(false) }
  }
  return hipErrorInvalidValue;
}

}  // namespace gma
