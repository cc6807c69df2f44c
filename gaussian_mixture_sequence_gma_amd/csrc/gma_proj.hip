// Projection GEMM of the GMA layer ("Gaussian Mixture Attention", Section
// "Projections", Eq. 4): Q_X = X W_Q, K_X = X W_K, V_X = X W_V with no bias.
// X is [B*N, d_model] bf16, each W is [d_model, H*d] bf16, and head h owns
// columns [h*d, (h+1)*d).  The products are accumulated in fp32 on bf16 MFMA
// and stored head-major [B,H,N,d], the layout the GMA kernels stream, in one
// of two forms: unrounded fp32, or (split) the routing vectors Q_X and K_X as
// bf16 pairs hi + lo carrying 16 significant bits and V_X rounded to bf16 --
// the operands of the bf16 GMA kernels, at 4 + 4 + 2 bytes per element instead
// of 12.
//
// One launch covers all three matrices.  A workgroup of WAF x WAT waves owns
// (16 WF WAF) output features x (16 WT WAT) tokens, each wave 16 WF x 16 WT of
// them, and walks d_model in steps of 64; both operand tiles are copied
// global -> LDS directly (no register staging) into a double buffer, so the
// copy of step k+1 runs under the MFMAs of step k.  The product is formed as
// D^T = W^T X^T: W supplies the MFMA A operand through transpose reads of its
// row-major [k][feature] tile, X supplies the B operand with plain 16-byte
// reads of its row-major [token][k] tile, and each accumulator lane then holds
// four consecutive features of one token.
//
// Fused form (bf16 causal layer, d_r = 64, at most 64 components): a wave's
// 64 features of Q_X or K_X are one whole head, so the epilogue forms the
// routing scores of its 128 tokens from the fp32 accumulators ("Gaussian
// routing components", Eq. 3, on split-bf16 MFMA) and stores, instead of the
// projections, what the scan consumes: per query the exponentials
// exp2(s - max s) of its scores as bf16 [B,H,N,K_c], and per 64-key chunk the
// keys' responsibilities transposed, bf16 [B,H,chunk][K_c][64], with K_c the
// 32 or 64 components formed.  Q_X and K_X never reach HBM; V_X is stored in
// bf16 as in the split form.
#include "gma_device.h"
#include "gma_internal.h"

namespace gma {
namespace {

constexpr int kPK = 64;    // d_model step
constexpr int kBand = 4;   // token tiles per band of the tile order

struct ProjArgs {
  const bf16* X;
  const bf16* W[3];
  void* out[3];
  bf16* lo[2];       // split: low halves of Q_X and K_X
  int split;
  int ncols[3];      // H * d of each matrix (multiple of 16)
  int dh[3];         // d of each matrix
  int ft0[4];        // first feature tile of each matrix; ft0[3] = total feature tiles
  int64_t M, N;      // M = B * N tokens
  int H, Dm;
  int64_t blocks;
  // fused form
  const char* params;     // prologue tables, head_bytes per head
  size_t head_bytes;
  int Kp, DRP;            // table layout: K_pad rows of DRP routing columns
  int kc;                 // components formed and stored (16 KE)
  bf16* eq;               // [B,H,N][kc] query exponentials
  bf16* gt;               // [B,H,ceil(N/64)][kc][64] keys' responsibilities
  int32_t* assign_q;      // optional [B,H,N]
  int32_t* assign_k;
};

// X tile [tokens][64 k]: eight 16-byte chunks per row, chunk c of row r at
// c ^ xswz(r).  Eight consecutive rows, and the eight even (odd) rows of 16
// consecutive ones, read the same logical chunk from distinct banks.
__device__ __forceinline__ int xswz(int r) { return (r ^ (r >> 3)) & 7; }

// Large problems: 256 x 256 workgroup tiles of eight 64 x 128 wave tiles, two
// waves per SIMD (128 accumulators each, so one wave's MFMAs run while the
// other waits on LDS); per 64-deep step a wave reads 12 KB of LDS operands for
// 64 MFMAs.  (32-deep steps through four stage buffers, three steps' copies in
// flight, measured slower: twice the barriers for the same bytes.)  Small
// problems: 64 x 64 tiles of four 32 x 32 wave tiles, for more workgroups.
template <int WF, int WT, int WAF, int WAT>
struct ProjTile {
  static constexpr int NW = WAF * WAT;                // waves per workgroup
  static constexpr int THREADS = 64 * NW;
  static constexpr int BF = 16 * WF * WAF;            // features per workgroup
  static constexpr int BT = 16 * WT * WAT;            // tokens per workgroup
  static constexpr int WROWCH = BF / 8;               // 16-byte chunks per W row
  static constexpr int XSEG = BT / 8;                 // 1 KB copies per X tile (8 rows each)
  static constexpr int WSEG = kPK * BF * 2 / 1024;    // 1 KB copies per W tile
  static constexpr int WROWS = 64 / WROWCH;           // W rows per copy
  static_assert(XSEG % NW == 0 && WSEG % NW == 0, "copies must divide among the waves");
  static_assert(WROWCH >= 2 && WROWCH <= 64, "W tile row of 32..1024 bytes");
};

// Products of the split score contraction on fp32 routing values x = xh + xl:
// features (x^2 hi, x^2 lo, xh, xl), coefficient arrays (A hi, A lo, B hi,
// B lo); x^2_lo A_lo and the products of xl with B_lo and of x^2 with
// nothing smaller fall below 2^-16 of the score terms.
constexpr int kPF[6] = {0, 1, 0, 2, 2, 3};
constexpr int kPW[6] = {0, 0, 1, 2, 3, 2};

// FDH > 0: the fused form for head dimension FDH, forming 16 KE components.
template <int WF, int WT, int WAF, int WAT, int FDH = 0, int KE = 0>
__global__ void __launch_bounds__(64 * WAF * WAT) gma_proj_kernel(ProjArgs a) {
  using T = ProjTile<WF, WT, WAF, WAT>;
  __shared__ __attribute__((aligned(16))) bf16 Xs[2][T::BT * kPK];
  __shared__ __attribute__((aligned(16))) bf16 Ws[2][kPK * T::BF];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int s16 = lane & 15, g = lane >> 4;

  // Workgroups are dealt to the eight XCDs round-robin; give each XCD a
  // contiguous run of logical tiles, ordered in bands of kBand token tiles
  // (feature tile outer, token tile inner), so the workgroups an XCD runs at
  // once share a few X and W tiles in its L2.
  int64_t L = blockIdx.x;
  if ((a.blocks & 7) == 0) L = (L & 7) * (a.blocks >> 3) + (L >> 3);
  const int ftot = a.ft0[3];
  const int64_t mtiles = a.blocks / ftot;
  const int64_t band = L / ((int64_t)kBand * ftot);
  const int64_t bt = (band + 1) * kBand <= mtiles ? kBand : mtiles - band * kBand;
  const int64_t rb = L - band * kBand * ftot;
  const int ft = (int)(rb / bt);
  const int64_t mt = band * kBand + rb % bt;
  const int m = ft >= a.ft0[2] ? 2 : (ft >= a.ft0[1] ? 1 : 0);
  const int f0 = (ft - a.ft0[m]) * T::BF;
  const int ncols = a.ncols[m];
  const int64_t tok0 = mt * T::BT;
  const bf16* __restrict__ X = a.X;
  const bf16* __restrict__ W = a.W[m];

  // Per-lane global sources of the direct copies: wave w fills 1 KB segments
  // w, w + NW, ... of each tile.
  constexpr int XPW = T::XSEG / T::NW, WPW = T::WSEG / T::NW;
  const bf16* xsrc[XPW];
  const bf16* wsrc[WPW];
#pragma unroll
  for (int j = 0; j < XPW; ++j) {
    const int seg = w + T::NW * j;
    const int xr = 8 * seg + (lane >> 3);
    int64_t tok = tok0 + xr;
    if (tok >= a.M) tok = a.M - 1;                        // ragged tail: rows never stored
    const int xc = (lane & 7) ^ xswz(xr);
    xsrc[j] = X + tok * a.Dm + xc * 8;
  }
#pragma unroll
  for (int j = 0; j < WPW; ++j) {
    const int seg = w + T::NW * j;
    const int wr = T::WROWS * seg + lane / T::WROWCH;
    const int pc = lane % T::WROWCH;
    const int wc = pc ^ ((2 * wr) & (T::WROWCH - 2));     // swz_elem<WROWCH> layout
    int col = f0 + wc * 8;
    if (col >= ncols) col = ncols - 8;                     // ragged features: never stored
    wsrc[j] = W + (int64_t)wr * ncols + col;
  }
  auto stage = [&](int kstep, int buf) {
    const int64_t kx = (int64_t)kstep * kPK;
    const int64_t kw = kx * ncols;
#pragma unroll
    for (int j = 0; j < XPW; ++j) global_to_lds16(xsrc[j] + kx, &Xs[buf][(w + T::NW * j) * 512]);
#pragma unroll
    for (int j = 0; j < WPW; ++j) global_to_lds16(wsrc[j] + kw, &Ws[buf][(w + T::NW * j) * 512]);
  };

  const int wf = w % WAF, wt = w / WAF;   // wave owns features wf*16WF.., tokens wt*16WT..
  f32x4 acc[WF][WT];
#pragma unroll
  for (int i = 0; i < WF; ++i)
#pragma unroll
    for (int j = 0; j < WT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = a.Dm / kPK;
  stage(0, 0);
  wait_global_loads();
  lds_barrier();
  for (int it = 0; it < nk; ++it) {
    const int buf = it & 1;
    if (it + 1 < nk) stage(it + 1, buf ^ 1);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8 wa[WF], xb[WT];
#pragma unroll
      for (int fm = 0; fm < WF; ++fm)
        wa[fm] = tr_chunk_swz<T::WROWCH>(Ws[buf], kk * 32, wf * 16 * WF + fm * 16);
#pragma unroll
      for (int tn = 0; tn < WT; ++tn) {
        const int r = wt * 16 * WT + tn * 16 + s16;
        xb[tn] = ld16<bf16x8>(&Xs[buf][r * kPK + (((kk * 4 + g) ^ xswz(r)) << 3)]);
      }
#pragma unroll
      for (int fm = 0; fm < WF; ++fm)
#pragma unroll
        for (int tn = 0; tn < WT; ++tn) acc[fm][tn] = mma(wa[fm], xb[tn], acc[fm][tn]);
    }
    wait_global_loads();
    lds_barrier();
  }

  // Lane (s16, g) of tile (fm, tn) holds features f..f+3, f = 16 fm + 4 g, of
  // token 16 tn + s16; four consecutive features never straddle a head.
  const int dh = a.dh[m], lgd = __builtin_ctz(dh);     // d is a power of two
  void* __restrict__ out = a.out[m];
  bf16* __restrict__ lo = m < 2 ? a.lo[m] : nullptr;
  // (batch, position) of the tile's first token, once per workgroup; a tile of
  // BT tokens crosses at most one batch boundary when N >= BT
  const int64_t b0 = tok0 / a.N, n0 = tok0 - b0 * a.N;
  auto locate = [&](int r, int64_t& b, int64_t& n) {
    b = b0;
    n = n0 + r;
    if (a.N >= T::BT) {
      if (n >= a.N) {
        n -= a.N;
        ++b;
      }
    } else {
      b += n / a.N;
      n -= (n / a.N) * a.N;
    }
  };

  if constexpr (FDH > 0) {
    static_assert(WF == 4 && WT == 8 && 16 * WF * WAF == T::BF && KE >= 1 && KE <= 4,
                  "fused form: 64-feature waves over 128 tokens");
    if (m < 2) {
      constexpr int HPW = 64 / FDH;       // heads per wave
      constexpr int NKH = FDH / 32;       // 32-wide routing chunks per head
      constexpr int NCH = KE * 8;         // operand chunks per wave (chunk, tile, array)
      const int fw = f0 + wf * 16 * WF;   // first feature of this wave
      const size_t nel = (size_t)a.Kp * a.DRP;
      // Coefficient operands of this wave's heads, in the order of the
      // accumulator features: element e of lane (s16, g) in routing chunk jj
      // is column 32 jj + 4 g + e (e < 4) or 32 jj + 16 + 4 g + e - 4 of the
      // wave's 64, so the contraction index needs no exchange between lanes.
      // Chunk q = (jj KE + ct) 4 + array, lane (s16, g): component 16 ct + s16.
      // The two waves sharing these features fill it; the main loop's tiles
      // are dead (every wave passed its last barrier).
      bf16x8* tab = reinterpret_cast<bf16x8*>(wf < 2 ? Xs[wf & 1] : Ws[wf & 1]);
      for (int q = wt; q < NCH; q += WAT) {
        const int ar = q & 3, ct = (q >> 2) % KE, jj = (q >> 2) / KE;
        bf16x8 v = {};
        if (fw + 32 * jj < ncols) {
          const int head = (fw + 32 * jj) / FDH, fb = (32 * jj) % FDH;
          const bf16* src = reinterpret_cast<const bf16*>(a.params + (size_t)head * a.head_bytes) +
                            (size_t)ar * nel + (size_t)(16 * ct + s16) * a.DRP + fb + 4 * g;
          const bf16x4 u0 = *reinterpret_cast<const bf16x4*>(src);
          const bf16x4 u1 = *reinterpret_cast<const bf16x4*>(src + 16);
          v = bf16x8{u0[0], u0[1], u0[2], u0[3], u1[0], u1[1], u1[2], u1[3]};
        }
        tab[q * 64 + lane] = v;
      }
      __syncthreads();

      const bool qside = m == 0;
      const int64_t nch = (a.N + 63) / 64;
      const int kc = a.kc;
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) {
        const int fh = fw + hh * FDH;
        if (fh >= ncols) break;
        const int head = fh / FDH;
        const float* cs = reinterpret_cast<const float*>(a.params + (size_t)head * a.head_bytes +
                                                         (size_t)8 * nel);
        // score seeds c_k: D[component][query] rows 16 ct + 4 g + i for the
        // queries, D[key][component] column 16 ct + s16 for the keys
        f32x4 seed[KE];
#pragma unroll
        for (int ct = 0; ct < KE; ++ct) {
          if (qside) {
            seed[ct] = *reinterpret_cast<const f32x4*>(cs + 16 * ct + 4 * g);
          } else {
            const float cv = cs[16 * ct + s16];
            seed[ct] = f32x4{cv, cv, cv, cv};
          }
        }
        // token tiles in pairs: each coefficient operand read from LDS serves
        // both
        constexpr int TB = 2;
#pragma unroll
        for (int tp = 0; tp < WT; tp += TB) {
          f32x4 SS[TB][KE];
#pragma unroll
          for (int bb = 0; bb < TB; ++bb)
#pragma unroll
            for (int ct = 0; ct < KE; ++ct) SS[bb][ct] = seed[ct];
#pragma unroll
          for (int j = 0; j < NKH; ++j) {
            // features of tokens 16 tn + s16 in routing chunk j, from the fp32
            // accumulators
            const int jj = hh * NKH + j;
            bf16x8 F[TB][4];
#pragma unroll
            for (int bb = 0; bb < TB; ++bb)
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const float x = acc[2 * jj + (e >> 2)][tp + bb][e & 3];
                bf16 h2, l2, h1, l1;
                split_bf16(x * x, h2, l2);
                split_bf16(x, h1, l1);
                F[bb][0][e] = h2;
                F[bb][1][e] = l2;
                F[bb][2][e] = h1;
                F[bb][3][e] = l1;
              }
#pragma unroll
            for (int ct = 0; ct < KE; ++ct) {
              const bf16x8* tq = tab + ((jj * KE + ct) * 4) * 64 + lane;
              const bf16x8 Wv[4] = {tq[0], tq[64], tq[128], tq[192]};
#pragma unroll
              for (int bb = 0; bb < TB; ++bb)
#pragma unroll
                for (int u = 0; u < 6; ++u)
                  SS[bb][ct] = qside ? mma(Wv[kPW[u]], F[bb][kPF[u]], SS[bb][ct])
                                     : mma(F[bb][kPF[u]], Wv[kPW[u]], SS[bb][ct]);
            }
          }
#pragma unroll
          for (int bb = 0; bb < TB; ++bb) {
          const int tn = tp + bb;
          f32x4 (&S)[KE] = SS[bb];
          if (qside) {
            // query 16 tn + s16: exponentials exp2(s - max) (the scan's
            // unnormalised responsibilities) and the lowest component at the
            // maximum score
            float mx = S[0][0];
#pragma unroll
            for (int ct = 0; ct < KE; ++ct)
#pragma unroll
              for (int i = 0; i < 4; ++i) mx = fmaxf(mx, S[ct][i]);
            mx = groups_max(mx);
            int bi = 0x7fffffff;
            if (a.assign_q) {
#pragma unroll
              for (int ct = 0; ct < KE; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                  bi = min(bi, S[ct][i] == mx ? 16 * ct + 4 * g + i : 0x7fffffff);
              bi = groups_min_i(bi);
            }
            const int r = wt * 16 * WT + tn * 16 + s16;
            if (tok0 + r < a.M) {
              int64_t b, n;
              locate(r, b, n);
              const size_t qrow = ((size_t)b * a.H + head) * a.N + n;
              bf16* dst = a.eq + qrow * kc + 4 * g;
#pragma unroll
              for (int ct = 0; ct < KE; ++ct) {
                bf16x4 v;
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = to_bf16(exp2_fast(S[ct][i] - mx));
                *reinterpret_cast<bf16x4*>(dst + 16 * ct) = v;
              }
              if (a.assign_q && g == 0) a.assign_q[qrow] = bi;
            }
          } else {
            // keys 16 tn + 4 g + i: responsibilities (softmax over the
            // components) and the lowest component at the maximum score
            bf16x4 Gv[KE];
            int bk[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float mx = S[0][i];
#pragma unroll
              for (int ct = 1; ct < KE; ++ct) mx = fmaxf(mx, S[ct][i]);
              mx = row16_max(mx);
              bk[i] = 0x7fffffff;
              if (a.assign_k) {
                int bi = 0x7fffffff;
#pragma unroll
                for (int ct = 0; ct < KE; ++ct) bi = min(bi, S[ct][i] == mx ? 16 * ct + s16 : 0x7fffffff);
                bi = min(bi, dpp_i<0xB1>(bi));
                bi = min(bi, dpp_i<0x4E>(bi));
                bi = min(bi, dpp_i<0x141>(bi));
                bi = min(bi, dpp_i<0x140>(bi));
                bk[i] = bi;
              }
              float ev[KE], l = 0.f;
#pragma unroll
              for (int ct = 0; ct < KE; ++ct) {
                ev[ct] = exp2_fast(S[ct][i] - mx);
                l += ev[ct];
              }
              l = row16_sum(l);
              const float inv = fast_rcp(l);
#pragma unroll
              for (int ct = 0; ct < KE; ++ct) Gv[ct][i] = to_bf16(ev[ct] * inv);
            }
            // Gamma^K^T: row 16 ct + s16 of the key's 64-key chunk, its four
            // consecutive keys in one 8-byte store where N is a multiple of 4
            // (they then share a sequence and a chunk)
            const int r0 = wt * 16 * WT + tn * 16 + 4 * g;
            if ((a.N & 3) == 0) {
              if (tok0 + r0 < a.M) {
                int64_t b, n;
                locate(r0, b, n);
                const size_t sq = (size_t)b * a.H + head;
                bf16* dst = a.gt + ((sq * nch + (size_t)(n >> 6)) * kc + s16) * 64 + (n & 63);
#pragma unroll
                for (int ct = 0; ct < KE; ++ct) *reinterpret_cast<bf16x4*>(dst + 16 * ct * 64) = Gv[ct];
                if (a.assign_k && s16 == 0) {
#pragma unroll
                  for (int i = 0; i < 4; ++i) a.assign_k[sq * a.N + n + i] = bk[i];
                }
              }
            } else {
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                if (tok0 + r0 + i >= a.M) continue;
                int64_t b, n;
                locate(r0 + i, b, n);
                const size_t sq = (size_t)b * a.H + head;
                bf16* dst = a.gt + ((sq * nch + (size_t)(n >> 6)) * kc + s16) * 64 + (n & 63);
#pragma unroll
                for (int ct = 0; ct < KE; ++ct) dst[16 * ct * 64] = Gv[ct][i];
                if (a.assign_k && s16 == 0) a.assign_k[sq * a.N + n] = bk[i];
              }
            }
          }
          }
        }
      }
      return;
    }
  }

#pragma unroll
  for (int tn = 0; tn < WT; ++tn) {
    const int r = wt * 16 * WT + tn * 16 + s16;
    if (tok0 + r >= a.M) continue;
    int64_t b, n;
    locate(r, b, n);
#pragma unroll
    for (int fm = 0; fm < WF; ++fm) {
      const int f = f0 + wf * 16 * WF + fm * 16 + 4 * g;
      if (f >= ncols) continue;
      const int h = f >> lgd, j = f & (dh - 1);
      const int64_t e = ((b * a.H + h) * a.N + n) * dh + j;
      if (!a.split) {
        st16(static_cast<float*>(out) + e, acc[fm][tn]);
      } else {
        bf16x4 hi, lw;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          bf16 vh, vl;
          split_bf16(acc[fm][tn][u], vh, vl);
          hi[u] = vh;
          lw[u] = vl;
        }
        *reinterpret_cast<bf16x4*>(static_cast<bf16*>(out) + e) = hi;
        if (lo) *reinterpret_cast<bf16x4*>(lo + e) = lw;
      }
    }
  }
}

template <int WF, int WT, int WAF, int WAT, int FDH = 0, int KE = 0>
hipError_t launch_tiles(ProjArgs& a, hipStream_t s) {
  using T = ProjTile<WF, WT, WAF, WAT>;
  int ft = 0;
  for (int m = 0; m < 3; ++m) {
    a.ft0[m] = ft;
    ft += (a.ncols[m] + T::BF - 1) / T::BF;
  }
  a.ft0[3] = ft;
  const int64_t mtiles = (a.M + T::BT - 1) / T::BT;
  a.blocks = mtiles * ft;
  if (a.blocks > 0x7fffffff) return hipErrorInvalidValue;
  gma_proj_kernel<WF, WT, WAF, WAT, FDH, KE><<<dim3((unsigned)a.blocks), dim3(T::THREADS), 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_proj(const void* X, const void* const W[3], void* const out[3],
                       void* const lo[2], int split, int64_t B, int64_t N, int H, int d_model,
                       int d_r, int d_v, hipStream_t s, const ProjFused* fz) {
  ProjArgs a{};
  a.X = static_cast<const bf16*>(X);
  a.split = split || fz ? 1 : 0;
  if (split && !fz) {
    if (!lo || !lo[0] || !lo[1]) return hipErrorInvalidValue;
    a.lo[0] = static_cast<bf16*>(lo[0]);
    a.lo[1] = static_cast<bf16*>(lo[1]);
  }
  const int d[3] = {d_r, d_r, d_v};
  for (int m = 0; m < 3; ++m) {
    if (d[m] < 4 || (d[m] & (d[m] - 1))) return hipErrorInvalidValue;   // head dims: powers of two
    a.W[m] = static_cast<const bf16*>(W[m]);
    a.out[m] = out[m];
    a.dh[m] = d[m];
    a.ncols[m] = H * d[m];
  }
  a.M = B * N;
  a.N = N;
  a.H = H;
  a.Dm = d_model;
  if (fz) {
    // fused form: heads of 32 or 64 features, 32 or 64 components formed, the
    // coefficient tables holding them
    const int KE = fz->kc / 16;
    if (d_r != 64 || (KE != 2 && KE != 4) || fz->kc > fz->Kp || fz->DRP != d_r ||
        !fz->params || !fz->eq || !fz->gt || !out[2])
      return hipErrorInvalidValue;
    a.params = fz->params;
    a.head_bytes = fz->head_bytes;
    a.Kp = fz->Kp;
    a.DRP = fz->DRP;
    a.kc = fz->kc;
    a.eq = static_cast<bf16*>(fz->eq);
    a.gt = static_cast<bf16*>(fz->gt);
    a.assign_q = fz->assign_q;
    a.assign_k = fz->assign_k;
    if (g_launch_hook) g_launch_hook("gma_proj", s, 1);
    hipError_t e;
    e = KE == 2 ? launch_tiles<4, 8, 4, 2, 64, 2>(a, s) : launch_tiles<4, 8, 4, 2, 64, 4>(a, s);
    if (g_launch_hook) g_launch_hook("gma_proj", s, 0);
    return e;
  }
  if (g_launch_hook) g_launch_hook("gma_proj", s, 1);
  // large problems: 256 x 256 workgroup tiles; small ones keep more workgroups
  const bool big = a.M >= 4096 && a.ncols[0] >= 256 && a.ncols[2] >= 256;
  hipError_t e = big ? launch_tiles<4, 8, 4, 2>(a, s) : launch_tiles<2, 2, 2, 2>(a, s);
  if (g_launch_hook) g_launch_hook("gma_proj", s, 0);
  return e;
}

}  // namespace gma
