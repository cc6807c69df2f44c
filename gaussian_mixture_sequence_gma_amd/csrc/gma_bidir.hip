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
#include "gma_device.h"
#include "gma_internal.h"

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
  const int n = Kp * DRP;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  // one thread per (head, component, routing column): A and B
  if (gid < (int64_t)H * n) {
    const int h = (int)(gid / n), idx = (int)(gid - (int64_t)h * n);
    const int k = idx / DRP, d = idx - k * DRP;
    char* base = params + (size_t)h * head_bytes;
    double a = 0.0, b = 0.0;
    if (k < K && d < DR) {
      const size_t off = ((size_t)h * K + k) * DR + d;
      const double w = (double)expf(-ls2[off]);
      a = -0.5 * w * kLog2eD;
      b = (double)mu[off] * w * kLog2eD;
    }
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
  // one thread per (head, component): c.  fp32 path: the kernels contract A
  // with (x^2 - 1) instead of x^2 (keeping the fp32 accumulator near zero for
  // unit-scale routing vectors) and add c' = c + sum_d A_kd once at the end;
  // bf16 path: c seeds the accumulator.
  if (gid < (int64_t)H * Kp) {
    const int h = (int)(gid / Kp), k = (int)(gid - (int64_t)h * Kp);
    float* c = reinterpret_cast<float*>(params + (size_t)h * head_bytes + (size_t)8 * n);
    if (k < K) {
      double acc = 0.0, asum = 0.0;
      const size_t off = ((size_t)h * K + k) * DR;
      for (int d = 0; d < DR; ++d) {
        const double m = mu[off + d], l = ls2[off + d];
        const double w = (double)expf(-ls2[off + d]);
        acc += m * m * w + l;
        asum += -0.5 * w;
      }
      const double ck = (double)lpi[(size_t)h * K + k] - 0.5 * acc + (BF ? 0.0 : asum);
      c[k] = (float)(kLog2eD * ck);
    } else {
      c[k] = -INFINITY;
    }
  }
}

// ============================================================================
// Compile-time configuration of the tiled kernels.
// ============================================================================
template <bool BF, int CPW_, int NG_, int DR_, int DV_>
struct Cfg {
  using P = Prec<BF>;
  using in_t = typename P::in_t;
  using op_t = typename P::op_t;
  using chunk_t = typename P::chunk_t;
  static constexpr bool kBF = BF;
  static constexpr int CPW = CPW_, NG = NG_, DR = DR_, DV = DV_;
  static constexpr int E = P::E, CS = P::CS, NARR = P::NARR;
  static constexpr int DRP = DR < CS ? CS : DR;
  static constexpr int NKS = DRP / CS;             // feature chunk steps
  static constexpr int TG = kWaves / NG;           // token groups
  static constexpr int TTW = 4 / TG;               // 16-token tiles per wave
  static constexpr int Kp = 16 * CPW * NG;
  static constexpr int KpO = (Kp + CS - 1) / CS * CS;  // component extent of the read contraction
  static constexpr int KSO = KpO / CS;
  static constexpr int DVT = DV / 16;
  static constexpr int NF = BF ? 3 : 2;            // staged feature arrays
  static constexpr int PADE = 16 / sizeof(op_t);
  static constexpr int FLD = DRP + PADE;           // feature row stride (elements)
  static constexpr int VLD = kTile + 16 / sizeof(in_t);
  static constexpr int GLD = KpO + PADE;
  // read-out work split among the NG waves of a token group
  static constexpr int DPW = DVT >= NG ? DVT / NG : 1;
  static constexpr int TPW = DVT >= NG ? TTW : TTW * DVT / NG;
};

struct BidirArgs {
  const void* x;          // K_X (write) or Q_X (read / resp), [BH][N][DR]
  const void* v;          // V_X [BH][N][DV] (write)
  void* out;              // O [BH][N][DV] (read)
  const char* params;     // prologue output
  size_t head_bytes;
  float* partial;         // [BH][S*TG][Kp][DV]
  float* partial_z;       // [BH][S*TG][Kp]
  const float* vt;        // [BH][Kp][DV]
  const float* z;         // [BH][Kp]
  int32_t* assign;        // [BH][N] or null
  float* gamma;           // resp: [BH][N][K] or null
  int64_t N;
  int H;
  int K;
  int S;
  int tiles_per_split;
  float eps;
  int out_bf;
};

template <class C>
__device__ __forceinline__ void load_w(const char* pbase, int ctile0,
                                       typename C::chunk_t (&W)[C::CPW][C::NKS][C::NARR]) {
  using op_t = typename C::op_t;
  using chunk_t = typename C::chunk_t;
  const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
  const int n = C::Kp * C::DRP;
  const op_t* arr = reinterpret_cast<const op_t*>(pbase);
#pragma unroll
  for (int ct = 0; ct < C::CPW; ++ct) {
    const int comp = (ctile0 + ct) * 16 + r;
#pragma unroll
    for (int s = 0; s < C::NKS; ++s)
#pragma unroll
      for (int a = 0; a < C::NARR; ++a)
        W[ct][s][a] = ld16<chunk_t>(arr + (size_t)a * n + comp * C::DRP + s * C::CS + g * C::E);
  }
}

// Stage routing features of one tile: bf16 -> (x^2 hi, x^2 lo, x); fp32 -> (x^2 - 1, x).
template <class C>
__device__ __forceinline__ void stage_features(const typename C::in_t* __restrict__ xg,
                                               int nvalid, typename C::op_t* F) {
  using chunk_t = typename C::chunk_t;
  constexpr int CPR = C::DR / C::E;     // 16-byte chunks per token row
  for (int i = threadIdx.x; i < kTile * CPR; i += kThreads) {
    const int t = i / CPR, part = i - t * CPR;
    chunk_t x;
    if (t < nvalid) {
      x = ld16<chunk_t>(xg + (size_t)t * C::DR + part * C::E);
    } else {
#pragma unroll
      for (int e = 0; e < C::E; ++e) x[e] = 0;
    }
    typename C::op_t* f = F + t * C::FLD + part * C::E;
    if constexpr (C::kBF) {
      bf16x8 hi, lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float xf = from_bf16(x[e]);
        bf16 h, l;
        split_bf16(xf * xf, h, l);
        hi[e] = h;
        lo[e] = l;
      }
      st16(f, hi);
      st16(f + kTile * C::FLD, lo);
      st16(f + 2 * kTile * C::FLD, x);
    } else {
      st16(f, x * x - 1.f);
      st16(f + kTile * C::FLD, x);
    }
  }
}

// Stage V transposed: Vt[d][token].
template <class C>
__device__ __forceinline__ void stage_vt(const typename C::in_t* __restrict__ vg, int nvalid,
                                         typename C::in_t* Vt) {
  using chunk_t = typename C::chunk_t;
  constexpr int CPR = C::DV / C::E;
  for (int i = threadIdx.x; i < kTile * CPR; i += kThreads) {
    const int t = i / CPR, part = i - t * CPR;
    chunk_t v;
    if (t < nvalid) {
      v = ld16<chunk_t>(vg + (size_t)t * C::DV + part * C::E);
    } else {
#pragma unroll
      for (int e = 0; e < C::E; ++e) v[e] = 0;
    }
#pragma unroll
    for (int e = 0; e < C::E; ++e) Vt[(part * C::E + e) * C::VLD + t] = v[e];
  }
}

// Score tiles.  TRANS = false: D[token][component] (features are the A operand);
// TRANS = true: D[component][token].  Accumulators arrive initialised with c
// (bf16 path) or zero (fp32 path, whose c' is added by finish_scores).
template <class C, bool TRANS>
__device__ __forceinline__ void score_tiles(const typename C::op_t* F, int gt0,
                                            const typename C::chunk_t (&W)[C::CPW][C::NKS][C::NARR],
                                            f32x4 (&S)[C::TTW][C::CPW]) {
  using chunk_t = typename C::chunk_t;
  const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int s = 0; s < C::NKS; ++s) {
#pragma unroll
    for (int tt = 0; tt < C::TTW; ++tt) {
      const int tok = tile_token(gt0 + tt, r);
      const typename C::op_t* f = F + tok * C::FLD + s * C::CS + g * C::E;
      const chunk_t f0 = ld16<chunk_t>(f);
      const chunk_t f1 = ld16<chunk_t>(f + kTile * C::FLD);
      if constexpr (C::kBF) {
        const chunk_t f2 = ld16<chunk_t>(f + 2 * kTile * C::FLD);
#pragma unroll
        for (int ct = 0; ct < C::CPW; ++ct) {
          f32x4 acc = S[tt][ct];
          if constexpr (!TRANS) {
            acc = mma(f0, W[ct][s][0], acc);   // x^2_hi * A_hi
            acc = mma(f1, W[ct][s][0], acc);   // x^2_lo * A_hi
            acc = mma(f0, W[ct][s][1], acc);   // x^2_hi * A_lo
            acc = mma(f2, W[ct][s][2], acc);   // x * B_hi
            acc = mma(f2, W[ct][s][3], acc);   // x * B_lo
          } else {
            acc = mma(W[ct][s][0], f0, acc);
            acc = mma(W[ct][s][0], f1, acc);
            acc = mma(W[ct][s][1], f0, acc);
            acc = mma(W[ct][s][2], f2, acc);
            acc = mma(W[ct][s][3], f2, acc);
          }
          S[tt][ct] = acc;
        }
      } else {
#pragma unroll
        for (int ct = 0; ct < C::CPW; ++ct) {
          f32x4 acc = S[tt][ct];
          if constexpr (!TRANS) {
            acc = mma(f0, W[ct][s][0], acc);   // x^2 * A
            acc = mma(f1, W[ct][s][1], acc);   // x * B
          } else {
            acc = mma(W[ct][s][0], f0, acc);
            acc = mma(W[ct][s][1], f1, acc);
          }
          S[tt][ct] = acc;
        }
      }
    }
  }
}

// fp32 path: scores = accumulated (x^2 - 1, x) contraction + c'.
template <class C>
__device__ __forceinline__ f32x4 score_seed(f32x4 cvals) {
  if constexpr (C::kBF) return cvals;
  else return f32x4{0.f, 0.f, 0.f, 0.f};
}
template <class C>
__device__ __forceinline__ void finish_scores(f32x4& s, f32x4 cvals) {
  if constexpr (!C::kBF) s += cvals;
}

// ============================================================================
// Latent write: grid (S, B*H).  Each workgroup covers tiles_per_split tiles of
// one sequence and writes TG partial (V~, Z) blocks.
// ============================================================================
template <class C>
__global__ void __launch_bounds__(kThreads) gma_write_kernel(BidirArgs a) {
  using in_t = typename C::in_t;
  using op_t = typename C::op_t;
  using chunk_t = typename C::chunk_t;
  __shared__ __attribute__((aligned(16))) op_t F[C::NF * kTile * C::FLD];
  __shared__ __attribute__((aligned(16))) in_t Vt[C::DV * C::VLD];
  __shared__ __attribute__((aligned(16))) f32x4 stats[C::NG * kTile];
  __shared__ __attribute__((aligned(16))) float fac[C::NG * kTile];

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

  for (int i = threadIdx.x; i < C::NF * kTile * C::FLD; i += kThreads) F[i] = (op_t)0;

  const char* pbase = a.params + (size_t)h * a.head_bytes;
  chunk_t W[C::CPW][C::NKS][C::NARR];
  load_w<C>(pbase, cgi * C::CPW, W);
  const float* cvec = reinterpret_cast<const float*>(pbase + (size_t)8 * C::Kp * C::DRP);
  float cv[C::CPW];
#pragma unroll
  for (int ct = 0; ct < C::CPW; ++ct) cv[ct] = cvec[(cgi * C::CPW + ct) * 16 + c];

  f32x4 vacc[C::CPW][C::DVT];
  float zacc[C::CPW];
#pragma unroll
  for (int ct = 0; ct < C::CPW; ++ct) {
    zacc[ct] = 0.f;
#pragma unroll
    for (int dt = 0; dt < C::DVT; ++dt) vacc[ct][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const in_t* xs = reinterpret_cast<const in_t*>(a.x) + (size_t)bh * a.N * C::DR;
  const in_t* vs = reinterpret_cast<const in_t*>(a.v) + (size_t)bh * a.N * C::DV;

  for (int64_t tile0 = t_begin; tile0 < t_end; tile0 += kTile) {
    const int nvalid = (int)min((int64_t)kTile, t_end - tile0);
    __syncthreads();
    stage_features<C>(xs + (size_t)tile0 * C::DR, nvalid, F);
    stage_vt<C>(vs + (size_t)tile0 * C::DV, nvalid, Vt);
    __syncthreads();

    f32x4 S[C::TTW][C::CPW];
#pragma unroll
    for (int tt = 0; tt < C::TTW; ++tt)
#pragma unroll
      for (int ct = 0; ct < C::CPW; ++ct) S[tt][ct] = score_seed<C>(f32x4{cv[ct], cv[ct], cv[ct], cv[ct]});
    score_tiles<C, false>(F, gt0, W, S);
#pragma unroll
    for (int tt = 0; tt < C::TTW; ++tt)
#pragma unroll
      for (int ct = 0; ct < C::CPW; ++ct) finish_scores<C>(S[tt][ct], f32x4{cv[ct], cv[ct], cv[ct], cv[ct]});

    // per-token statistics over this wave's components (lanes of a DPP row hold
    // the 16 components of a tile; rows 4g+i are tokens)
    float m[C::TTW][4], l[C::TTW][4];
    int am[C::TTW][4];
#pragma unroll
    for (int tt = 0; tt < C::TTW; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = S[tt][0][i];
#pragma unroll
        for (int ct = 1; ct < C::CPW; ++ct) v = fmaxf(v, S[tt][ct][i]);
        m[tt][i] = row16_max(v);
        am[tt][i] = 0;
      }
    if (want_assign) {
#pragma unroll
      for (int tt = 0; tt < C::TTW; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = S[tt][0][i];
          int idx = (cgi * C::CPW) * 16 + c;
#pragma unroll
          for (int ct = 1; ct < C::CPW; ++ct)
            argmax_merge(v, idx, S[tt][ct][i], (cgi * C::CPW + ct) * 16 + c);
          row16_argmax(v, idx);
          am[tt][i] = idx;
        }
    }
#pragma unroll
    for (int tt = 0; tt < C::TTW; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float mu_ = m[tt][i] == -INFINITY ? 0.f : m[tt][i];
        float sum = 0.f;
#pragma unroll
        for (int ct = 0; ct < C::CPW; ++ct) {
          const float e = exp2_fast(S[tt][ct][i] - mu_);
          S[tt][ct][i] = e;
          sum += e;
        }
        l[tt][i] = row16_sum(sum);
      }

    float f[C::TTW][4];
    if constexpr (C::NG > 1) {
      {
        const int tts = c >> 2, is = c & 3;
        float sm = 0.f, sl = 0.f;
        int sa = 0;
#pragma unroll
        for (int tt = 0; tt < C::TTW; ++tt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (tt == tts && i == is) { sm = m[tt][i]; sl = l[tt][i]; sa = am[tt][i]; }
        if (tts < C::TTW)
          stats[cgi * kTile + tile_token(gt0 + tts, 4 * g + is)] =
              f32x4{sm, sl, __int_as_float(sa), 0.f};
      }
      __syncthreads();
      if (threadIdx.x < kTile) {
        const int t = threadIdx.x;
        f32x4 st[C::NG];
        float M = -INFINITY;
#pragma unroll
        for (int q = 0; q < C::NG; ++q) {
          st[q] = stats[q * kTile + t];
          M = fmaxf(M, st[q][0]);
        }
        float L = 0.f, fq[C::NG];
        int arg = 0;
        bool found = false;
#pragma unroll
        for (int q = 0; q < C::NG; ++q) {
          fq[q] = st[q][0] == -INFINITY ? 0.f : exp2_fast(st[q][0] - M);
          L += fq[q] * st[q][1];
          if (!found && st[q][0] == M) { arg = __float_as_int(st[q][2]); found = true; }
        }
        const float invL = 1.f / L;
#pragma unroll
        for (int q = 0; q < C::NG; ++q) fac[q * kTile + t] = fq[q] * invL;
        if (want_assign && t < nvalid) a.assign[(size_t)bh * a.N + tile0 + t] = arg;
      }
      __syncthreads();
#pragma unroll
      for (int tt = 0; tt < C::TTW; ++tt) {
        const f32x4 fv = ld16<f32x4>(&fac[cgi * kTile + tile_token(gt0 + tt, 4 * g)]);
#pragma unroll
        for (int i = 0; i < 4; ++i) f[tt][i] = fv[i];
      }
    } else {
#pragma unroll
      for (int tt = 0; tt < C::TTW; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) f[tt][i] = 1.f / l[tt][i];
      if (want_assign && c == 0) {
#pragma unroll
        for (int tt = 0; tt < C::TTW; ++tt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int tok = tile_token(gt0 + tt, 4 * g + i);
            if (tok < nvalid) a.assign[(size_t)bh * a.N + tile0 + tok] = am[tt][i];
          }
      }
    }

    // gamma = e * factor, masked to valid tokens; accumulate Z in fp32
#pragma unroll
    for (int tt = 0; tt < C::TTW; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool valid = tile_token(gt0 + tt, 4 * g + i) < nvalid;
        const float fi = valid ? f[tt][i] : 0.f;
#pragma unroll
        for (int ct = 0; ct < C::CPW; ++ct) {
          const float gm = S[tt][ct][i] * fi;
          S[tt][ct][i] = gm;
          zacc[ct] += gm;
        }
      }

    // V~ += Gamma^T V over this wave's tokens
    if constexpr (C::kBF) {
      constexpr int NP = C::TTW >= 2 ? C::TTW / 2 : 1;
#pragma unroll
      for (int pp = 0; pp < NP; ++pp) {
        const int gta = gt0 + 2 * pp;               // first tile of the pair (or the only one)
        const int P = gta >> 1;
        bf16x8 A[C::CPW];
#pragma unroll
        for (int ct = 0; ct < C::CPW; ++ct) {
#pragma unroll
          for (int e = 0; e < 8; ++e) A[ct][e] = (bf16)0.f;
          if constexpr (C::TTW >= 2) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              A[ct][i] = to_bf16(S[2 * pp][ct][i]);
              A[ct][4 + i] = to_bf16(S[2 * pp + 1][ct][i]);
            }
          } else {
            const int hsel = gt0 & 1;
#pragma unroll
            for (int i = 0; i < 4; ++i) A[ct][4 * hsel + i] = to_bf16(S[0][ct][i]);
          }
        }
#pragma unroll
        for (int dt = 0; dt < C::DVT; ++dt) {
          const bf16x8 Bv = ld16<bf16x8>(&Vt[(dt * 16 + c) * C::VLD + 32 * P + 8 * g]);
#pragma unroll
          for (int ct = 0; ct < C::CPW; ++ct) vacc[ct][dt] = mma(A[ct], Bv, vacc[ct][dt]);
        }
      }
    } else {
#pragma unroll
      for (int tt = 0; tt < C::TTW; ++tt) {
        const int gt = gt0 + tt;
        const int base = 32 * (gt >> 1) + 8 * g + 4 * (gt & 1);
#pragma unroll
        for (int dt = 0; dt < C::DVT; ++dt) {
          const f32x4 Bv = ld16<f32x4>(&Vt[(dt * 16 + c) * C::VLD + base]);
#pragma unroll
          for (int ct = 0; ct < C::CPW; ++ct) vacc[ct][dt] = mma(S[tt][ct], Bv, vacc[ct][dt]);
        }
      }
    }
  }

  // partial (V~, Z) for this (split, token group)
  const int PS = a.S * C::TG;
  const size_t pslot = (size_t)bh * PS + (size_t)split * C::TG + tg;
  float* pv = a.partial + pslot * C::Kp * C::DV;
  float* pz = a.partial_z + pslot * C::Kp;
#pragma unroll
  for (int ct = 0; ct < C::CPW; ++ct) {
    const int comp0 = (cgi * C::CPW + ct) * 16;
#pragma unroll
    for (int dt = 0; dt < C::DVT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) pv[(comp0 + 4 * g + i) * C::DV + dt * 16 + c] = vacc[ct][dt][i];
    const float zt = groups_sum(zacc[ct]);
    if (g == 0) pz[comp0 + c] = zt;
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
__global__ void __launch_bounds__(kThreads) gma_read_kernel(BidirArgs a) {
  using in_t = typename C::in_t;
  using op_t = typename C::op_t;
  using chunk_t = typename C::chunk_t;
  __shared__ __attribute__((aligned(16))) op_t F[C::NF * kTile * C::FLD];
  __shared__ __attribute__((aligned(16))) op_t G[MODE == 0 ? kTile * C::GLD : 1];
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

  for (int i = threadIdx.x; i < C::NF * kTile * C::FLD; i += kThreads) F[i] = (op_t)0;
  if constexpr (MODE == 0)
    for (int i = threadIdx.x; i < kTile * C::GLD; i += kThreads) G[i] = (op_t)0;

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

  for (int64_t tile0 = t_begin; tile0 < t_end; tile0 += kTile) {
    const int nvalid = (int)min((int64_t)kTile, t_end - tile0);
    __syncthreads();
    stage_features<C>(xs + (size_t)tile0 * C::DR, nvalid, F);
    __syncthreads();

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
      __syncthreads();
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
      __syncthreads();
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
          op_t* dst = &G[tok * C::GLD + (cgi * C::CPW + ct) * 16 + 4 * g];
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
      __syncthreads();

      // O = diag(rinv) Gamma' V~ for this wave's (token tile, d tile) share
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
          const chunk_t A = ld16<chunk_t>(&G[rtok * C::GLD + s * C::CS + g * C::E]);
#pragma unroll
          for (int j = 0; j < C::DPW; ++j) acc[j] = mma(A, Vr[j][s], acc[j]);
        }
        const int tok0 = tile_token(gt, 4 * g);
        const f32x4 rv = ld16<f32x4>(&rinv[tok0]);
#pragma unroll
        for (int j = 0; j < C::DPW; ++j) {
          const int dt = C::DVT >= C::NG ? cgi * C::DPW + j : cgi % C::DVT;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int tok = tok0 + i;
            if (tok < nvalid) {
              const float o = acc[j][i] * rv[i];
              const size_t off = ((size_t)bh * a.N + tile0 + tok) * C::DV + dt * 16 + c;
              if (a.out_bf) reinterpret_cast<bf16*>(a.out)[off] = to_bf16(o);
              else reinterpret_cast<float*>(a.out)[off] = o;
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
  hipLaunchKernelGGL(gma_write_kernel<C>, grid, dim3(kThreads), 0, s, a);
  if (g_launch_hook) g_launch_hook("gma_write", s, 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int PS = p.S * C::TG;
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
  const int64_t nthreads = p.H * (int64_t)p.Kp * p.DRP;
  const dim3 grid((unsigned)((nthreads + 255) / 256));
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
