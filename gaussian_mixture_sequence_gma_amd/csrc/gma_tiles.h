// Shared tile machinery of the gfx950 GMA kernels: compile-time configuration,
// coefficient loading, feature / value staging, MFMA score tiles and the
// latent-write kernel (used by the bidirectional path and, per span, by the
// causal path).  See gma_bidir.hip for the method summary.
#pragma once

#include "gma_device.h"
#include "gma_internal.h"

namespace gma {

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
  static constexpr int NF = BF ? 3 : 1;            // staged feature arrays (fp32: x only)
  static constexpr int PADE = 16 / sizeof(op_t);
  static constexpr int FLD = DRP + PADE;           // feature row stride (elements)
  // Each block of 16 token rows is shifted by a further 64 bytes: the 16 rows one
  // MFMA operand read touches (tokens r and r+16 of a 32-token pair, see
  // tile_token) then fall on 16 distinct 4-bank groups for every d_r.  Same for
  // the Gamma' rows below.
  static constexpr int SKEW = 64 / (int)sizeof(op_t);
  static constexpr int FAS = kTile * FLD + 3 * SKEW;   // stride between feature arrays
  __host__ __device__ static constexpr int frow(int r) { return r * FLD + SKEW * (r >> 4); }
  static constexpr int VLD = kTile + 16 / sizeof(in_t);
  static constexpr int GLD = KpO + PADE;
  static constexpr int GAS = kTile * GLD + 3 * SKEW;   // Gamma' [token][component] array size
  __host__ __device__ static constexpr int grow(int r) { return r * GLD + SKEW * (r >> 4); }
  // occupancy request (waves per SIMD) for the streaming kernels; set by
  // WavesPerEU below from register-budget measurements
  // read-out work split among the NG waves of a token group
  static constexpr int DPW = DVT >= NG ? DVT / NG : 1;
  static constexpr int TPW = DVT >= NG ? TTW : TTW * DVT / NG;
  // 2 waves/SIMD where the compiler fits the kernel in 256 VGPRs without spills
  static constexpr int kWPEWrite = (NG == 4 || ((DV == 128 || DR == 128) && NG >= 2)) ? 1 : 2;
  static constexpr int kWPERead = (DR == 128 || (!BF && NG == 4 && DV == 128)) ? 1 : 2;
};

// LDS bytes of the causal scan kernel: the staged features of Q and K share
// storage with Gamma^Q, Gamma^K and the carried state (live at different times).
__host__ __device__ constexpr int causal_union_elems(int NF, int FAS, int DV, int GAS, int GLD) {
  return 2 * NF * FAS > 2 * GAS + DV * GLD ? 2 * NF * FAS : 2 * GAS + DV * GLD;
}
__host__ __device__ constexpr int causal_lds_bytes(bool bf, int DR, int DV, int Kp) {
  // mirrors Cfg: element sizes, strides, padding and skews
  return causal_union_elems(bf ? 3 : 1,
                            kTile * ((DR < (bf ? 32 : 16) ? (bf ? 32 : 16) : DR) + (bf ? 8 : 4)) +
                                3 * (bf ? 32 : 16),
                            DV, kTile * (Kp + (bf ? 8 : 4)) + 3 * (bf ? 32 : 16), Kp + (bf ? 8 : 4)) *
             (bf ? 2 : 4) +
         DV * (kTile + (bf ? 8 : 4)) * (bf ? 2 : 4) +       // Vt
         Kp * 4 + 2 * 4 * kTile * 16 + 2 * 4 * kTile * 4 + kTile * 4;
}
constexpr int kMaxLds = 160 * 1024;

// LDS bytes of the bf16 token-owner scan kernel (gma_causal2_kernel), or 0 where
// it does not apply: the coefficient operand table and constants, the Gamma^K
// and V tiles (double-buffered when that fits) and the carried-state operand
// table.  Mirrors Causal2 in gma_causal.hip.
__host__ __device__ constexpr int causal2_lds_bytes_nb(int DRP, int DV, int Kp, int nb) {
  return (Kp / 16) * (DRP / 32) * 4 * 1024 + Kp * 4 +
         nb * Kp * kTile * 2 + nb * kTile * DV * 2 +
         (DV / 16 + 1) * (Kp / 32) * 1024;
}
__host__ __device__ constexpr int causal2_lds_bytes(bool bf, int DRP, int DV, int Kp) {
  return !(bf && Kp % 64 == 0 && DRP <= 64 && DV >= 32)
             ? 0
             : (causal2_lds_bytes_nb(DRP, DV, Kp, 2) <= kMaxLds
                    ? causal2_lds_bytes_nb(DRP, DV, Kp, 2)
                    : (causal2_lds_bytes_nb(DRP, DV, Kp, 1) <= kMaxLds
                           ? causal2_lds_bytes_nb(DRP, DV, Kp, 1)
                           : 0));
}
// LDS bytes of the bf16 token-owner read-out (gma_read2_kernel): the
// coefficient operand table, the V~ operand table with its (Z_hi, Z_lo, 1)
// block, and the constants.  Mirrors Read2 in gma_bidir.hip.
__host__ __device__ constexpr int read2_lds_bytes(int DRP, int DV, int Kp) {
  return ((Kp / 16) * (DRP / 32) * 4 + (DV / 16 + 1) * (Kp / 32)) * 1024 + Kp * 4;
}
constexpr int kRead2MaxLds = 150 * 1024;
// bf16 bidirectional read-out at K_pad = 256 whose tables exceed that bound
// while those of 128 components fit: it runs once per half of the components
__host__ __device__ constexpr bool bidir_khalf(bool bf, int DRP, int DV, int Kp) {
  return bf && Kp == 256 && DRP <= 64 && DV >= 32 && read2_lds_bytes(DRP, DV, Kp) > kRead2MaxLds &&
         read2_lds_bytes(DRP, DV, Kp / 2) <= kRead2MaxLds;
}
// bf16 causal forward at K_pad = 256 whose scan tables exceed LDS while those
// of 128 components fit: the scan runs once per half of the components, each
// on its rows of the keys' responsibilities from the span-totals pass (the team
// write, which needs d_v of 64 or 128 at this K)
__host__ __device__ constexpr bool causal_khalf(bool bf, int DRP, int DV, int Kp) {
  return bf && Kp == 256 && DRP <= 64 && (DV == 64 || DV == 128) &&
         causal2_lds_bytes(true, DRP, DV, Kp) == 0 && causal2_lds_bytes(true, DRP, DV, Kp / 2) > 0;
}

struct BidirArgs {
  const void* x;          // K_X (write) or Q_X (read / resp), [BH][N][DR]
  const void* x_lo;       // split routing vectors: low bf16 parts (x = x + x_lo), or null
  const void* v;          // V_X [BH][N][DV] (write)
  void* out;              // O [BH][N][DV] (read)
  const char* params;     // prologue output
  size_t head_bytes;
  float* partial;         // [BH][S*TG][Kp][DV]
  float* partial_z;       // [BH][S*TG][Kp]
  const float* vt;        // [BH][Kp][DV]
  const bf16x8* vtab;     // [BH][(DV/16 + 1) * Kp/32 * 64] read-out operand table
  const float* z;         // [BH][Kp]
  int32_t* assign;        // [BH][N] or null
  float* gamma;           // resp: [BH][N][K] or null
  float* diag;            // usage statistics: [BH][S][3 Kp + 4] per-workgroup partials
  float thr;              // usage statistics: responsibility threshold of the utilisation
  int64_t N;
  int H;
  int K;
  int S;
  int tiles_per_split;
  int gpw;                // token-owner write: 32-token groups per split (0: derived)
  float eps;
  int out_bf;
  bf16* gt;               // token-owner writes: the keys' responsibilities stored as
                          // Gamma^K^T tiles [BH][ceil(N/64)][Kp][64] bf16 (every
                          // 64-key chunk whole, zeros past N), for the causal scan;
                          // or null
  // read-out over one half of the components (K_pad = 256):
  float* qpart;           // the first half's numerators [BH][N][DV]
  float4* qpart2;         // and (denominator, maximum, best score, its component) [BH][N]
  int koff;               // first component of this half
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

// Stage routing features of one tile: bf16 -> (x^2 hi, x^2 lo, x); fp32 -> x (the
// score loop forms x^2 - 1 in registers).
template <class C>
__device__ __forceinline__ void stage_features(const typename C::in_t* __restrict__ xg,
                                               int nvalid, typename C::op_t* F) {
  using chunk_t = typename C::chunk_t;
  constexpr int CPR = C::DRP / C::E;    // 16-byte chunks per padded token row
  for (int i = threadIdx.x; i < kTile * CPR; i += kThreads) {
    const int t = i / CPR, part = i - t * CPR;
    chunk_t x;
    if (t < nvalid && part * C::E < C::DR) {   // routing columns beyond d_r stay zero
      x = ld16<chunk_t>(xg + (size_t)t * C::DR + part * C::E);
    } else {
#pragma unroll
      for (int e = 0; e < C::E; ++e) x[e] = 0;
    }
    typename C::op_t* f = F + C::frow(t) + part * C::E;
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
      st16(f + C::FAS, lo);
      st16(f + 2 * C::FAS, x);
    } else {
      st16(f, x);
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

// Routing vectors of one 64-token tile held in registers (prefetched while the
// previous tile is processed), then expanded into the staged feature arrays.
template <class C>
struct FeatureTile {
  using chunk_t = typename C::chunk_t;
  static constexpr int CPR = C::DR / C::E;            // 16-byte chunks per token row
  static constexpr int CH = kTile * CPR;
  static constexpr int NC = (CH + kThreads - 1) / kThreads;
  chunk_t r[NC];

  __device__ __forceinline__ void load(const typename C::in_t* __restrict__ xs, int64_t tile0,
                                       int nvalid) {
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int i = threadIdx.x + j * kThreads;
      const int t = i / CPR, part = i - t * CPR;
      if (i < CH && t < nvalid) r[j] = ld16<chunk_t>(xs + (size_t)(tile0 + t) * C::DR + part * C::E);
      else r[j] = chunk_t{};
    }
  }
  // bf16 -> (x^2 hi, x^2 lo, x); fp32 -> x.  Also zeroes routing columns beyond d_r.
  __device__ __forceinline__ void store(typename C::op_t* F) const {
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int i = threadIdx.x + j * kThreads;
      if (i < CH) {
        const int t = i / CPR, part = i - t * CPR;
        typename C::op_t* f = F + C::frow(t) + part * C::E;
        if constexpr (C::kBF) {
          bf16x8 hi, lo;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float xf = from_bf16(r[j][e]);
            bf16 hh, ll;
            split_bf16(xf * xf, hh, ll);
            hi[e] = hh;
            lo[e] = ll;
          }
          st16(f, hi);
          st16(f + C::FAS, lo);
          st16(f + 2 * C::FAS, r[j]);
        } else {
          st16(f, r[j]);
        }
      }
    }
    if constexpr (C::DR < C::DRP) {
      constexpr int PADCH = (C::DRP - C::DR) / C::E;
      for (int i = threadIdx.x; i < C::NF * kTile * PADCH; i += kThreads) {
        const int row = i / PADCH, pc = i - row * PADCH;
        const int arr = row / kTile, t = row - arr * kTile;
        st16(F + arr * C::FAS + C::frow(t) + C::DR + pc * C::E, chunk_t{});
      }
    }
  }
};

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
      const typename C::op_t* f = F + C::frow(tok) + s * C::CS + g * C::E;
      if constexpr (C::kBF) {
        const chunk_t f0 = ld16<chunk_t>(f);
        const chunk_t f1 = ld16<chunk_t>(f + C::FAS);
        const chunk_t f2 = ld16<chunk_t>(f + 2 * C::FAS);
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
        const chunk_t f1 = ld16<chunk_t>(f);     // x
        const chunk_t f0 = f1 * f1 - 1.f;        // x^2 - 1
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
  __shared__ __attribute__((aligned(16))) op_t F[C::NF * C::FAS];
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

  for (int i = threadIdx.x; i < C::NF * C::FAS; i += kThreads) F[i] = (op_t)0;

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
        const float invL = fast_rcp(L);
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
        for (int i = 0; i < 4; ++i) f[tt][i] = fast_rcp(l[tt][i]);
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


// ============================================================================
// Latent write, bf16 inputs, software-pipelined over 64-token tiles.
//
// Scores use the D[component][token] layout (per-token statistics stay inside
// a lane plus two cross-group steps).  Gamma^K goes to LDS row-major
// [token][component] and both operands of V~ += Gamma^T V (and Z += Gamma^T 1,
// also on MFMA) are read with transpose reads; V tiles are copied HBM -> LDS by
// direct loads into a swizzled double buffer.  Iteration k runs the statistics,
// Gamma and latent-write MMA of tile k while the score MFMAs of tile k+1 are
// issued in the same basic blocks, so MFMA work overlaps the VALU / LDS phases
// and the barriers.  Wave w accumulates its own (component, d_v) output tiles
// over all tokens of the split; one partial per workgroup.
// ============================================================================
template <class C, int TT0, int TT1>
__device__ __forceinline__ void score_range_T(const bf16* const (&fb)[C::TTW],
                                              const bf16x8 (&W)[C::CPW][C::NKS][4],
                                              f32x4 (&S)[C::TTW][C::CPW]) {
  // all feature reads of the range first, then the MFMAs ordered so that
  // consecutive instructions update independent accumulators
  constexpr int NT = TT1 - TT0;
  if constexpr (NT > 0) {
    bf16x8 f[C::NKS][NT][3];
#pragma unroll
    for (int s = 0; s < C::NKS; ++s)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const bf16* fp = fb[TT0 + t] + s * C::CS;
        f[s][t][0] = ld16<bf16x8>(fp);
        f[s][t][1] = ld16<bf16x8>(fp + C::FAS);
        f[s][t][2] = ld16<bf16x8>(fp + 2 * C::FAS);
      }
    constexpr int WI[5] = {0, 0, 1, 2, 3};   // A_hi, A_hi, A_lo, B_hi, B_lo
    constexpr int FI[5] = {0, 1, 0, 2, 2};   // x^2_hi, x^2_lo, x^2_hi, x, x
#pragma unroll
    for (int s = 0; s < C::NKS; ++s)
#pragma unroll
      for (int q = 0; q < 5; ++q)
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int ct = 0; ct < C::CPW; ++ct)
            S[TT0 + t][ct] = mma(W[ct][s][WI[q]], f[s][t][FI[q]], S[TT0 + t][ct]);
  }
}

template <class C>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(C::kWPEWrite)))
gma_write_bf16_kernel(BidirArgs a) {
  static_assert(C::kBF, "bf16 kernel");
  constexpr int TTW = C::TTW;
  constexpr int CT = C::CPW * C::NG;
  constexpr int CTW = CT >= 4 ? CT / 4 : 1;                    // output component tiles per wave
  constexpr int DW = CT >= 4 ? C::DVT : (C::DVT * CT + 3) / 4;  // output d tiles per wave
  constexpr int GRLD = C::Kp + 16;                              // Gamma row stride (16 mod 32)
  constexpr int VROWCH = C::DV / 8;                             // 16-byte chunks per V row
  constexpr int VROUNDS = kTile * VROWCH / 64;                  // 1 KB wave loads per V tile
  constexpr int VRPW = (VROUNDS + kWaves - 1) / kWaves;
  constexpr int P1 = (TTW + 1) / 2;                             // next-tile score split over phases
  constexpr int P2 = P1 + (TTW - P1 + 1) / 2;
  __shared__ __attribute__((aligned(16))) bf16 F[3 * C::FAS];
  __shared__ __attribute__((aligned(16))) bf16 G[kTile * GRLD + 16];
  __shared__ __attribute__((aligned(16))) bf16 Vr[2][kTile * C::DV];
  __shared__ __attribute__((aligned(16))) f32x4 stats[C::NG * kTile];
  __shared__ __attribute__((aligned(16))) float fac[C::NG * kTile];
  __shared__ __attribute__((aligned(16))) float cl[C::Kp];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int cgi = wave % C::NG, tg = wave / C::NG;
  const int gt0 = tg * TTW;
  const int64_t bh = blockIdx.y;
  const int h = (int)(bh % a.H);
  const int64_t t_begin = (int64_t)blockIdx.x * a.tiles_per_split * kTile;
  const int64_t t_end = a.N < t_begin + (int64_t)a.tiles_per_split * kTile
                            ? a.N : t_begin + (int64_t)a.tiles_per_split * kTile;
  const int ntiles = t_end > t_begin ? (int)((t_end - t_begin + kTile - 1) / kTile) : 0;
  const bool want_assign = a.assign != nullptr;
  const bool wave_valid = cgi * C::CPW * 16 < a.K;   // some real component in this group

  const char* pbase = a.params + (size_t)h * a.head_bytes;
  bf16x8 W[C::CPW][C::NKS][4];
  load_w<C>(pbase, cgi * C::CPW, W);
  {
    const float* cvec = reinterpret_cast<const float*>(pbase + (size_t)8 * C::Kp * C::DRP);
    for (int k = threadIdx.x; k < C::Kp; k += kThreads) cl[k] = cvec[k];
  }

  // lane-constant LDS offsets
  const bf16* fb[TTW];
  int gw[TTW];
#pragma unroll
  for (int tt = 0; tt < TTW; ++tt) {
    const int tok = tile_token(gt0 + tt, c);
    fb[tt] = F + C::frow(tok) + g * 8;
    gw[tt] = gtr_row(tok, GRLD) + cgi * C::CPW * 16 + 4 * g;
  }
  const int s4 = lane & 15, a4 = s4 & 3, m4 = s4 >> 2;
  const int g_lo = gtr_row(8 * g + m4, GRLD) + 4 * a4;         // rows +4 share the skew
  const int v_lo = (8 * g + m4) * C::DV + 4 * a4;
  const int h_lo = (8 * g + m4) & (VROWCH / 2 - 1);
  const int h_hi = (8 * g + m4 + 4) & (VROWCH / 2 - 1);
  const int oct0 = CT >= 4 ? wave * CTW : wave % CT;
  // this wave's direct-load slots of a V tile (row, chunk within the swizzled tile)
  int vrow[VRPW], voff[VRPW];
#pragma unroll
  for (int j = 0; j < VRPW; ++j) {
    const int round = wave * VRPW + j;
    const int P = round * 64 + lane;
    const int r = P / VROWCH, pc = P - r * VROWCH;
    vrow[j] = r;
    voff[j] = (pc ^ (r & (VROWCH / 2 - 1)) * 2) * 8;
  }
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
    for (int j = 0; j < VRPW; ++j) {
      const int round = wave * VRPW + j;
      if (round < VROUNDS) {
        const int rr = vrow[j] < nv ? vrow[j] : nv - 1;     // tail rows repeat a valid row
        global_to_lds16(vs + (size_t)(t0 + rr) * C::DV + voff[j], &Vr[buf][round * 512]);
      }
    }
  };

  f32x4 vacc[CTW][DW], vz[CTW];
#pragma unroll
  for (int i = 0; i < CTW; ++i) {
    vz[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < DW; ++j) vacc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (bf16)1.0f;

  f32x4 S[TTW][C::CPW], Sn[TTW][C::CPW];
  auto seed = [&](f32x4 (&X)[TTW][C::CPW]) {
#pragma unroll
    for (int tt = 0; tt < TTW; ++tt)
#pragma unroll
      for (int ct = 0; ct < C::CPW; ++ct) X[tt][ct] = ld16<f32x4>(&cl[(cgi * C::CPW + ct) * 16 + 4 * g]);
  };

  FeatureTile<C> kreg;
  if (ntiles > 0) {
    kreg.load(xs, tile_start(0), tile_valid(0));
    load_v(0, 0);
    lds_barrier();                       // cl visible
    kreg.store(F);
    lds_barrier();
    seed(S);
    score_range_T<C, 0, TTW>(fb, W, S);
    if (ntiles > 1) kreg.load(xs, tile_start(1), tile_valid(1));
    lds_barrier();                       // every wave done with the features of tile 0
    if (ntiles > 1) kreg.store(F);
    if (ntiles > 2) kreg.load(xs, tile_start(2), tile_valid(2));
    lds_barrier();
  }

  for (int k = 0; k < ntiles; ++k) {
    const bool has_next = k + 1 < ntiles;
    const int64_t tile0 = tile_start(k);
    const int nvalid = tile_valid(k);
    const int buf = k & 1;

    // ---- phase 1: next-tile scores (part) || statistics of tile k ----------------
    // (branch-free so the scheduler can interleave the two streams; the scores of
    // a tile past the end are computed from stale features and never used)
    seed(Sn);
    score_range_T<C, 0, P1>(fb, W, Sn);
    float m[TTW], l[TTW];
#pragma unroll
    for (int tt = 0; tt < TTW; ++tt) {
      float v = S[tt][0][0];
#pragma unroll
      for (int ct = 0; ct < C::CPW; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) v = fmaxf(v, S[tt][ct][i]);
      v = groups_max(v);
      m[tt] = wave_valid ? v : -INFINITY;
      const float mref = wave_valid ? v : 0.f;      // all-padding group: every e is 0
      float sum = 0.f;
#pragma unroll
      for (int ct = 0; ct < C::CPW; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = exp2_fast(S[tt][ct][i] - mref);
          S[tt][ct][i] = e;
          sum += e;
        }
      l[tt] = groups_sum(sum);
    }
    int am[TTW];
#pragma unroll
    for (int tt = 0; tt < TTW; ++tt) am[tt] = 0;
    if (want_assign) {
      // exp2 is monotone, so the largest e is the largest score (ties: lowest index)
#pragma unroll
      for (int tt = 0; tt < TTW; ++tt) {
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
    }
    if (C::NG > 1 && g == 0) {
#pragma unroll
      for (int tt = 0; tt < TTW; ++tt)
        stats[cgi * kTile + tile_token(gt0 + tt, c)] = f32x4{m[tt], l[tt], 0.f, __int_as_float(am[tt])};
    }
    lds_barrier();

    // ---- phase 2: next-tile scores (part) || combine the component groups -------
    score_range_T<C, P1, P2>(fb, W, Sn);
    if (C::NG > 1 && threadIdx.x < kTile) {
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
        if (!found && st[q][0] == M) { arg = __float_as_int(st[q][3]); found = true; }
      }
      const float invL = fast_rcp(L);
#pragma unroll
      for (int q = 0; q < C::NG; ++q) fac[q * kTile + t] = fq[q] * invL;
      if (want_assign && t < nvalid) a.assign[(size_t)bh * a.N + tile0 + t] = arg;
    }
    lds_barrier();

    // ---- phase 3: next-tile scores (rest) || Gamma (masked) -> LDS ----------------
    score_range_T<C, P2, TTW>(fb, W, Sn);
#pragma unroll
    for (int tt = 0; tt < TTW; ++tt) {
      const int tok = tile_token(gt0 + tt, c);
      float fi;
      if constexpr (C::NG > 1) fi = fac[cgi * kTile + tok];
      else {
        fi = fast_rcp(l[tt]);
        if (want_assign && g == 0 && tok < nvalid) a.assign[(size_t)bh * a.N + tile0 + tok] = am[tt];
      }
      fi = tok < nvalid ? fi : 0.f;
#pragma unroll
      for (int ct = 0; ct < C::CPW; ++ct) {
        bf16x4 v4;
#pragma unroll
        for (int i = 0; i < 4; ++i) v4[i] = to_bf16(S[tt][ct][i] * fi);
        *reinterpret_cast<bf16x4*>(&G[gw[tt] + ct * 16]) = v4;
      }
    }
    wait_global_loads();                 // V(k) and the routing vectors of tile k+2
    lds_barrier();

    // ---- phase 4: V~ += Gamma^T V, Z += Gamma^T 1 || stage tile k+2, fetch ahead ---
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      bf16x8 A[CTW];
#pragma unroll
      for (int i = 0; i < CTW; ++i) {
        const bf16* gp = G + g_lo + 32 * p * GRLD + (oct0 + i) * 16;
        const short4_t lo = lds_read_tr16(gp);
        const short4_t hi = lds_read_tr16(gp + 4 * GRLD);
        typedef short short8_t __attribute__((ext_vector_type(8)));
        A[i] = __builtin_bit_cast(bf16x8, short8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
        vz[i] = mma(A[i], ones, vz[i]);
      }
#pragma unroll
      for (int j = 0; j < DW; ++j) {
        const int dt = CT >= 4 ? j : wave / CT + (4 / CT) * j;
        if (dt < C::DVT) {
          const bf16* vp = Vr[buf] + 32 * p * C::DV;
          const short4_t lo = lds_read_tr16(vp + v_lo + 16 * (dt ^ h_lo));
          const short4_t hi = lds_read_tr16(vp + v_lo + 4 * C::DV + 16 * (dt ^ h_hi));
          typedef short short8_t __attribute__((ext_vector_type(8)));
          const bf16x8 Bv = __builtin_bit_cast(bf16x8, short8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
#pragma unroll
          for (int i = 0; i < CTW; ++i) vacc[i][j] = mma(A[i], Bv, vacc[i][j]);
        }
      }
    }
    if (k + 2 < ntiles) kreg.store(F);
    if (k + 3 < ntiles) kreg.load(xs, tile_start(k + 3), tile_valid(k + 3));
    if (has_next) load_v(k + 1, buf ^ 1);
#pragma unroll
    for (int tt = 0; tt < TTW; ++tt)
#pragma unroll
      for (int ct = 0; ct < C::CPW; ++ct) S[tt][ct] = Sn[tt][ct];
    lds_barrier();
  }

  // ---- partial (V~, Z) of this workgroup ------------------------------------------
  const size_t pslot = (size_t)bh * a.S + blockIdx.x;
  float* pv = a.partial + pslot * C::Kp * C::DV;
  float* pz = a.partial_z + pslot * C::Kp;
#pragma unroll
  for (int i = 0; i < CTW; ++i) {
#pragma unroll
    for (int j = 0; j < DW; ++j) {
      const int dt = CT >= 4 ? j : wave / CT + (4 / CT) * j;
      if (dt < C::DVT) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          pv[((oct0 + i) * 16 + 4 * g + r) * C::DV + dt * 16 + c] = vacc[i][j][r];
      }
    }
    // every column of Gamma^T 1 holds Z; waves sharing a component tile write once
    if (c == 0 && (CT >= 4 || wave / CT == 0)) {
#pragma unroll
      for (int r = 0; r < 4; ++r) pz[(oct0 + i) * 16 + 4 * g + r] = vz[i][r];
    }
  }
}

}  // namespace gma
