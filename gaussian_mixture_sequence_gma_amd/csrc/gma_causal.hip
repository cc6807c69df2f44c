// Causal GMA forward on gfx950: a chunked prefix scan.
//
// Paper: "Gaussian Mixture Attention: Linear-Time Sequence Mixing via
// Probabilistic Latent Routing", Section "Causal GMA" (Eq. 8b and its
// footnote): the memories become inclusive prefix sums
//   V~^(i)_k = sum_{j<=i} gamma^K_jk v_j,  Z^(i)_k = sum_{j<=i} gamma^K_jk,
//   O_i = gamma^Q_i V~^(i) / (gamma^Q_i Z^(i) + eps),
// which the paper computes as cumulative sums along the sequence.
//
// Three launches per call:
//  1. span totals: the latent-write kernel run with one split per span writes
//     sum_{j in span} gamma^K_j (x) v_j and sum gamma^K_j for every span;
//  2. an exclusive scan over spans gives each span its carried-in state;
//  3. the scan kernel walks its span in 64-token chunks.  For chunk c with
//     carried state (S, z) it computes
//        num_i = gamma^Q_i S + sum_{j in c, j<=i} (gamma^Q_i . gamma^K_j) v_j
//        den_i = gamma^Q_i z + sum_{j in c, j<=i} (gamma^Q_i . gamma^K_j) + eps
//     on MFMA (the masked intra-chunk affinity never leaves the CU), then
//     S += Gamma^K_c^T V_c, z += Gamma^K_c^T 1 in registers.
// The scan kernel uses four component groups (K padded to >= 64) so that all
// four waves see every token of a chunk and the running state is split over
// the waves by component.
#include "gma_team.h"

namespace gma {

struct CausalArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  const char* params;
  size_t head_bytes;
  const float* carry;     // [BH][nspan][Kp][DV] exclusive prefix state
  const float* carry_z;   // [BH][nspan][Kp]
  int32_t* assign_q;
  int32_t* assign_k;
  int64_t N;
  int H;
  int nspan;
  int span_tiles;
  float eps;
  int out_bf;
  const void* q_lo;       // split routing vectors: low bf16 parts, or null
  const void* k_lo;
  const float* state;     // token-owner scan: the spans' totals [BH][nspan][Kp][DV]
  const float* state_z;   // and [BH][nspan][Kp] (the carried state is their prefix sum)
  const bf16* gt;         // token-owner scan: the keys' Gamma^K^T tiles from the
                          // span-totals pass, [BH][ceil(N/64)][Kp][64] bf16
  // scan over one half of the components (K_pad = 256):
  float* qpart;           // the first half's numerators [BH][N][DV]
  float4* qpart2;         // and (denominator, maximum, best score, its component) [BH][N]
  int koff;               // first component of this half
  // the fused layer: queries' exponentials exp2(s - max s) [BH][N][kc] bf16 and
  // the keys' Gamma^K^T [BH][ceil(N/64)][kc][64] from the projection epilogue,
  // kc (32 or 64) components formed; the others are zero
  const bf16* eq;
  int kc;
  const bf16* vtab;       // bidirectional read-out: the summed state as an operand table
};

// out[s] = sum_{s' < s} in[s'] over n terms at stride st, summed in order.
// The loads of eight terms are issued before their sums are stored: the trip
// count is a run-time value, so otherwise every add waits for its own load.
__device__ __forceinline__ void exclusive_sum_strided(const float* __restrict__ in,
                                                      float* __restrict__ out, int n,
                                                      size_t st) {
  float acc = 0.f;
  int s = 0;
  for (; s + 8 <= n; s += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = in[(size_t)(s + u) * st];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      out[(size_t)(s + u) * st] = acc;
      acc += v[u];
    }
  }
  for (; s < n; ++s) {
    out[(size_t)s * st] = acc;
    acc += in[(size_t)s * st];
  }
}

// Exclusive prefix over spans, fixed order: carry[s] = sum_{s' < s} state[s'].
__global__ void __launch_bounds__(256) gma_span_scan_kernel(const float* __restrict__ state,
                                                            const float* __restrict__ state_z,
                                                            int nspan, int Kp, int DV,
                                                            float* __restrict__ carry,
                                                            float* __restrict__ carry_z) {
  const int64_t bh = blockIdx.y;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  const int nv = Kp * DV;
  if (idx < nv) {
    const size_t base = (size_t)bh * nspan * nv + idx;
    exclusive_sum_strided(state + base, carry + base, nspan, (size_t)nv);
  } else if (idx < nv + Kp) {
    const size_t base = (size_t)bh * nspan * Kp + (idx - nv);
    exclusive_sum_strided(state_z + base, carry_z + base, nspan, (size_t)Kp);
  }
}

template <class C>
__global__ void __launch_bounds__(kThreads) gma_causal_kernel(CausalArgs a) {
  static_assert(C::NG == 4 && C::TG == 1 && C::TTW == 4, "causal scan needs four component groups");
  using in_t = typename C::in_t;
  using op_t = typename C::op_t;
  using chunk_t = typename C::chunk_t;
  constexpr int FE = C::NF * C::FAS;
  // features (dead once the scores exist) share storage with Gamma^Q, Gamma^K, S
  __shared__ __attribute__((aligned(16))) op_t U[causal_union_elems(C::NF, C::FAS, C::DV, C::GAS, C::GLD)];
  __shared__ __attribute__((aligned(16))) in_t Vt[C::DV * C::VLD];
  op_t* const QF = U;
  op_t* const KF = U + FE;
  op_t* const GQ = U;
  op_t* const GK = U + C::GAS;
  op_t* const ST = U + 2 * C::GAS;
  __shared__ __attribute__((aligned(16))) float zs[C::Kp];
  __shared__ __attribute__((aligned(16))) f32x4 statsK[4 * kTile];
  __shared__ __attribute__((aligned(16))) f32x4 statsQ[4 * kTile];
  __shared__ __attribute__((aligned(16))) float facK[4 * kTile];
  __shared__ __attribute__((aligned(16))) float facQ[4 * kTile];
  __shared__ __attribute__((aligned(16))) float qden[kTile];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int64_t bh = blockIdx.y;
  const int h = (int)(bh % a.H);
  const int span = blockIdx.x;
  const int64_t t_begin = (int64_t)span * a.span_tiles * kTile;
  const int64_t t_end = a.N < t_begin + (int64_t)a.span_tiles * kTile
                            ? a.N : t_begin + (int64_t)a.span_tiles * kTile;


  const char* pbase = a.params + (size_t)h * a.head_bytes;
  chunk_t W[C::CPW][C::NKS][C::NARR];
  load_w<C>(pbase, w * C::CPW, W);
  const float* cvec = reinterpret_cast<const float*>(pbase + (size_t)8 * C::Kp * C::DRP);
  float cv[C::CPW];
  f32x4 cv4[C::CPW];
#pragma unroll
  for (int ct = 0; ct < C::CPW; ++ct) {
    cv[ct] = cvec[(w * C::CPW + ct) * 16 + c];
    cv4[ct] = ld16<f32x4>(cvec + (w * C::CPW + ct) * 16 + 4 * g);
  }

  // running state: S (D layout, lane column d, rows components) and z (per component c)
  const size_t sslot = (size_t)bh * a.nspan + span;
  f32x4 vacc[C::CPW][C::DVT];
  float zst[C::CPW];
#pragma unroll
  for (int ct = 0; ct < C::CPW; ++ct) {
    const int comp0 = (w * C::CPW + ct) * 16;
#pragma unroll
    for (int dt = 0; dt < C::DVT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        vacc[ct][dt][i] = a.carry[(sslot * C::Kp + comp0 + 4 * g + i) * C::DV + dt * 16 + c];
    zst[ct] = a.carry_z[sslot * C::Kp + comp0 + c];
    if (g == 0) zs[comp0 + c] = zst[ct];
  }

  const in_t* qs = reinterpret_cast<const in_t*>(a.q) + (size_t)bh * a.N * C::DR;
  const in_t* ks = reinterpret_cast<const in_t*>(a.k) + (size_t)bh * a.N * C::DR;
  const in_t* vs = reinterpret_cast<const in_t*>(a.v) + (size_t)bh * a.N * C::DV;
  const bool want_aq = a.assign_q != nullptr, want_ak = a.assign_k != nullptr;

  for (int64_t tile0 = t_begin; tile0 < t_end; tile0 += kTile) {
    const int nvalid = (int)((t_end - tile0) < kTile ? (t_end - tile0) : kTile);
    __syncthreads();
    stage_features<C>(qs + (size_t)tile0 * C::DR, nvalid, QF);
    stage_features<C>(ks + (size_t)tile0 * C::DR, nvalid, KF);
    stage_vt<C>(vs + (size_t)tile0 * C::DV, nvalid, Vt);
    __syncthreads();

    // ---- key responsibilities, D[token][component] --------------------------
    f32x4 SK[4][C::CPW];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int ct = 0; ct < C::CPW; ++ct)
        SK[tt][ct] = score_seed<C>(f32x4{cv[ct], cv[ct], cv[ct], cv[ct]});
    score_tiles<C, false>(KF, 0, W, SK);
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int ct = 0; ct < C::CPW; ++ct)
        finish_scores<C>(SK[tt][ct], f32x4{cv[ct], cv[ct], cv[ct], cv[ct]});
    float mk[4][4], lk[4][4];
    int ak[4][4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = SK[tt][0][i];
        int idx = (w * C::CPW) * 16 + c;
#pragma unroll
        for (int ct = 1; ct < C::CPW; ++ct) argmax_merge(v, idx, SK[tt][ct][i], (w * C::CPW + ct) * 16 + c);
        if (want_ak) {
          float vv = v;
          row16_argmax(vv, idx);
        }
        mk[tt][i] = row16_max(v);
        ak[tt][i] = idx;
        const float mu_ = mk[tt][i] == -INFINITY ? 0.f : mk[tt][i];
        float sum = 0.f;
#pragma unroll
        for (int ct = 0; ct < C::CPW; ++ct) {
          const float e = exp2_fast(SK[tt][ct][i] - mu_);
          SK[tt][ct][i] = e;
          sum += e;
        }
        lk[tt][i] = row16_sum(sum);
      }
    {
      const int tts = c >> 2, is = c & 3;
      float sm = 0.f, sl = 0.f;
      int sa = 0;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (tt == tts && i == is) { sm = mk[tt][i]; sl = lk[tt][i]; sa = ak[tt][i]; }
      statsK[w * kTile + tile_token(tts, 4 * g + is)] = f32x4{sm, sl, __int_as_float(sa), 0.f};
    }

    // ---- query responsibilities, D[component][token] ------------------------
    f32x4 SQ[4][C::CPW];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int ct = 0; ct < C::CPW; ++ct) SQ[tt][ct] = score_seed<C>(cv4[ct]);
    score_tiles<C, true>(QF, 0, W, SQ);
    f32x4 z4[C::CPW];
#pragma unroll
    for (int ct = 0; ct < C::CPW; ++ct) z4[ct] = ld16<f32x4>(&zs[(w * C::CPW + ct) * 16 + 4 * g]);
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
      for (int ct = 0; ct < C::CPW; ++ct) finish_scores<C>(SQ[tt][ct], cv4[ct]);
      float v = SQ[tt][0][0];
      int bi = (w * C::CPW) * 16 + 4 * g;
#pragma unroll
      for (int ct = 0; ct < C::CPW; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) argmax_merge(v, bi, SQ[tt][ct][i], (w * C::CPW + ct) * 16 + 4 * g + i);
      if (want_aq) {
        float vv = v;
        groups_argmax(vv, bi);
      }
      const float m = groups_max(v);
      const float mu_ = m == -INFINITY ? 0.f : m;
      float sum = 0.f, den = 0.f;
#pragma unroll
      for (int ct = 0; ct < C::CPW; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = exp2_fast(SQ[tt][ct][i] - mu_);
          SQ[tt][ct][i] = e;
          sum += e;
          den += e * z4[ct][i];
        }
      sum = groups_sum(sum);
      den = groups_sum(den);
      if (g == 0) statsQ[w * kTile + tile_token(tt, c)] = f32x4{m, sum, den, __int_as_float(bi)};
    }
    __syncthreads();

    // ---- combine the four component groups ---------------------------------
    if (threadIdx.x < 2 * kTile) {
      const bool isq = threadIdx.x >= kTile;
      const int t = threadIdx.x & (kTile - 1);
      const f32x4* st = isq ? statsQ : statsK;
      f32x4 s4[4];
      float M = -INFINITY;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        s4[q] = st[q * kTile + t];
        M = fmaxf(M, s4[q][0]);
      }
      float L = 0.f, D = 0.f, fq[4];
      int arg = 0;
      bool found = false;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        fq[q] = s4[q][0] == -INFINITY ? 0.f : exp2_fast(s4[q][0] - M);
        L += fq[q] * s4[q][1];
        D += fq[q] * s4[q][2];
        const int aq_ = __float_as_int(isq ? s4[q][3] : s4[q][2]);
        if (!found && s4[q][0] == M) { arg = aq_; found = true; }
      }
      const float invL = fast_rcp(L);
      float* fac = isq ? facQ : facK;
#pragma unroll
      for (int q = 0; q < 4; ++q) fac[q * kTile + t] = fq[q] * invL;
      if (isq) qden[t] = D * invL;
      if (t < nvalid) {
        if (isq && want_aq) a.assign_q[(size_t)bh * a.N + tile0 + t] = arg;
        if (!isq && want_ak) a.assign_k[(size_t)bh * a.N + tile0 + t] = arg;
      }
    }
    __syncthreads();

    // ---- normalised responsibilities to LDS; carried state to LDS -----------
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const f32x4 fk = ld16<f32x4>(&facK[w * kTile + tile_token(tt, 4 * g)]);
      const float fqv = facQ[w * kTile + tile_token(tt, c)];
      const int qtok = tile_token(tt, c);
#pragma unroll
      for (int ct = 0; ct < C::CPW; ++ct) {
        const int comp0 = (w * C::CPW + ct) * 16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ktok = tile_token(tt, 4 * g + i);
          const float gk = ktok < nvalid ? SK[tt][ct][i] * fk[i] : 0.f;
          SK[tt][ct][i] = gk;
          GK[C::grow(ktok) + comp0 + c] = (op_t)gk;
          SQ[tt][ct][i] *= fqv;
        }
        op_t* dst = &GQ[C::grow(qtok) + comp0 + 4 * g];
        if constexpr (C::kBF) {
          bf16x4 v4;
#pragma unroll
          for (int i = 0; i < 4; ++i) v4[i] = to_bf16(SQ[tt][ct][i]);
          *reinterpret_cast<bf16x4*>(dst) = v4;
        } else {
          st16(dst, SQ[tt][ct]);
        }
      }
    }
#pragma unroll
    for (int ct = 0; ct < C::CPW; ++ct) {
      const int comp0 = (w * C::CPW + ct) * 16;
#pragma unroll
      for (int dt = 0; dt < C::DVT; ++dt) {
        op_t* dst = &ST[(dt * 16 + c) * C::GLD + comp0 + 4 * g];
        if constexpr (C::kBF) {
          bf16x4 v4;
#pragma unroll
          for (int i = 0; i < 4; ++i) v4[i] = to_bf16(vacc[ct][dt][i]);
          *reinterpret_cast<bf16x4*>(dst) = v4;
        } else {
          st16(dst, vacc[ct][dt]);
        }
      }
    }
    __syncthreads();

    // ---- outputs: wave w owns query tile w ----------------------------------
    {
      const int gt = w;
      const int Pi = gt >> 1;
      const int itok_c = tile_token(gt, c);
      f32x4 acc[C::DVT];
#pragma unroll
      for (int dt = 0; dt < C::DVT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      // carried memory: Gamma^Q_c S
#pragma unroll
      for (int s = 0; s < C::KSO; ++s) {
        const chunk_t A = ld16<chunk_t>(&GQ[C::grow(itok_c) + s * C::CS + g * C::E]);
#pragma unroll
        for (int dt = 0; dt < C::DVT; ++dt) {
          const chunk_t Bs = ld16<chunk_t>(&ST[(dt * 16 + c) * C::GLD + s * C::CS + g * C::E]);
          acc[dt] = mma(A, Bs, acc[dt]);
        }
      }
      // intra-chunk: P^T = Gamma^K Gamma^Q^T (rows key tokens, columns query tokens), masked j <= i
      float rowsum = 0.f;
      for (int p = 0; p <= Pi; ++p) {
        f32x4 PT[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int jt = 2 * p + hh;
          f32x4 pt = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < C::KSO; ++s) {
            const chunk_t Ak = ld16<chunk_t>(&GK[C::grow(tile_token(jt, c)) + s * C::CS + g * C::E]);
            const chunk_t Bq = ld16<chunk_t>(&GQ[C::grow(itok_c) + s * C::CS + g * C::E]);
            pt = mma(Ak, Bq, pt);
          }
          if (p == Pi) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (tile_token(jt, 4 * g + i) > itok_c) pt[i] = 0.f;
          }
          rowsum += pt[0] + pt[1] + pt[2] + pt[3];
          PT[hh] = pt;
        }
        if constexpr (C::kBF) {
          bf16x8 Ap;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            Ap[i] = to_bf16(PT[0][i]);
            Ap[4 + i] = to_bf16(PT[1][i]);
          }
#pragma unroll
          for (int dt = 0; dt < C::DVT; ++dt) {
            const bf16x8 Bv = ld16<bf16x8>(&Vt[(dt * 16 + c) * C::VLD + 32 * p + 8 * g]);
            acc[dt] = mma(Ap, Bv, acc[dt]);
          }
        } else {
#pragma unroll
          for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int dt = 0; dt < C::DVT; ++dt) {
              const f32x4 Bv = ld16<f32x4>(&Vt[(dt * 16 + c) * C::VLD + 32 * p + 8 * g + 4 * hh]);
              acc[dt] = mma(PT[hh], Bv, acc[dt]);
            }
        }
      }
      rowsum = groups_sum(rowsum);   // per query token tile_token(gt, c)
      const f32x4 qd = ld16<f32x4>(&qden[tile_token(gt, 4 * g)]);
      float rinv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // row 4g+i of the accumulator is query token tile_token(gt, 4g+i), whose
        // intra-chunk row sum sits in lane column 4g+i
        const float rs = __int_as_float(__builtin_amdgcn_ds_bpermute((4 * g + i) << 2, __float_as_int(rowsum)));
        rinv[i] = fast_rcp(qd[i] + rs + a.eps);
      }
#pragma unroll
      for (int dt = 0; dt < C::DVT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = tile_token(gt, 4 * g + i);
          if (tok < nvalid) {
            const float o = acc[dt][i] * rinv[i];
            const size_t off = ((size_t)bh * a.N + tile0 + tok) * C::DV + dt * 16 + c;
            if (a.out_bf) reinterpret_cast<bf16*>(a.out)[off] = to_bf16(o);
            else reinterpret_cast<float*>(a.out)[off] = o;
          }
        }
    }

    // ---- state update: S += Gamma^K_c^T V_c, z += Gamma^K_c^T 1 ----------------
#pragma unroll
    for (int ct = 0; ct < C::CPW; ++ct) {
      float zp = 0.f;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) zp += SK[tt][ct][i];
      zst[ct] += groups_sum(zp);
    }
    if constexpr (C::kBF) {
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        bf16x8 A[C::CPW];
#pragma unroll
        for (int ct = 0; ct < C::CPW; ++ct)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            A[ct][i] = to_bf16(SK[2 * pp][ct][i]);
            A[ct][4 + i] = to_bf16(SK[2 * pp + 1][ct][i]);
          }
#pragma unroll
        for (int dt = 0; dt < C::DVT; ++dt) {
          const bf16x8 Bv = ld16<bf16x8>(&Vt[(dt * 16 + c) * C::VLD + 32 * pp + 8 * g]);
#pragma unroll
          for (int ct = 0; ct < C::CPW; ++ct) vacc[ct][dt] = mma(A[ct], Bv, vacc[ct][dt]);
        }
      }
    } else {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int base = 32 * (tt >> 1) + 8 * g + 4 * (tt & 1);
#pragma unroll
        for (int dt = 0; dt < C::DVT; ++dt) {
          const f32x4 Bv = ld16<f32x4>(&Vt[(dt * 16 + c) * C::VLD + base]);
#pragma unroll
          for (int ct = 0; ct < C::CPW; ++ct) vacc[ct][dt] = mma(SK[tt][ct], Bv, vacc[ct][dt]);
        }
      }
    }
    // zs is read again only after the next chunk's first barrier
#pragma unroll
    for (int ct = 0; ct < C::CPW; ++ct)
      if (g == 0) zs[(w * C::CPW + ct) * 16 + c] = zst[ct];
  }
}

// ============================================================================
// Causal scan, bf16 inputs, token-owner form.  Wave w owns queries 16w ..
// 16w+15 of every 64-token chunk, with all K_pad components, so the query
// softmax stays inside the wave.  The keys' responsibilities are not formed
// here: the span-totals pass, which scores every key anyway, stores them as
// Gamma^K^T tiles (per 64-key chunk, [component][key] bf16), and the scan
// copies each chunk's tile into LDS beside its values.  After one barrier
// each wave forms, for its 16 queries,
//   num = e^Q S + sum_{j <= i in chunk} (e^Q . Gamma^K_j) v_j,
//   den = e^Q z + sum_{j <= i} (e^Q . Gamma^K_j) + eps * sum_k e^Q_k
// (e^Q = exp2(s - max), unnormalised: the ratio is the same), all on MFMA: the
// carried state S, z is an LDS operand table (S^T in bf16 with rows Z_hi, Z_lo
// and ones appended, as the bidirectional read-out uses V~), and the intra-
// chunk affinity P = Gamma^K e^Q^T feeds V^T P straight from registers.  After
// a second barrier each wave adds Gamma^K_c^T V_c to its quarter of S (fp32
// registers) and rewrites its part of the table.
// ============================================================================
template <class C>
struct Causal2 {
  static constexpr int KP = C::Kp;
  static constexpr int CT = KP / 16;
  static constexpr int KS = KP / 32;
  static constexpr int NKS = C::DRP / 32;
  static constexpr int DVT = C::DV / 16;
  static constexpr int OT = DVT + 1;
  static constexpr int CTW = CT / 4;                       // state component tiles per wave
  static constexpr int COEF = CT * NKS * 4;
  static constexpr int VROWCH = C::DV / 8;
  static constexpr int VROUNDS = kTile * VROWCH / 64;      // 1 KB wave copies per V tile
  static constexpr int VRPW = (VROUNDS + kWaves - 1) / kWaves;
  static constexpr int GROUNDS = KP * kTile * 2 / 1024;    // 1 KB wave copies per Gamma^K^T tile
  static constexpr int GRPW = GROUNDS / kWaves;
  static constexpr int STCH = OT * KS;
  static constexpr int lds_bytes(int nb) {
    return COEF * 1024 + KP * 4 + nb * KP * kTile * 2 + nb * kTile * C::DV * 2 + STCH * 1024;
  }
  // Gamma^K^T and V tiles double-buffered when they fit (two barriers per
  // chunk), else single-buffered with a third barrier after the state update
  static constexpr int NB = lds_bytes(2) <= 160 * 1024 ? 2 : 1;
  static constexpr bool kOK = C::kBF && KP % 64 == 0 && C::DRP <= 64 && C::DV >= 32 &&
                              lds_bytes(NB) <= 160 * 1024;
  static_assert(!kOK || causal2_lds_bytes(true, C::DRP, C::DV, KP) == lds_bytes(NB),
                "span sizing mirrors this LDS budget");
  static_assert(!kOK || GROUNDS % kWaves == 0, "Gamma^K^T copies divide among the waves");
};

// HM = 0: all components.  HM = 1, 2: the components koff .. koff + C::Kp - 1
// of the tables laid out for CF (K_pad = 2 C::Kp); the first half (HM = 1)
// leaves each query's numerator, denominator and maximum in qpart / qpart2,
// the second (HM = 2) rescales both halves to the larger maximum and writes O.
// QG: the fused layer's scan, the queries' exponentials and the keys'
// Gamma^K^T (a.kc rows) given; no routing scores are formed.  BI (with QG):
// the bidirectional read-out, O_i = gamma^Q_i V~ / (gamma^Q_i Z + eps) with
// the memories of all keys ("Normalized broadcasting", Eq. 7): the state is
// the operand table of every span's totals summed (a.vtab) and no chunk is
// scanned, so a workgroup's span is any run of chunks.
template <class C, bool XS, int HM = 0, class CF = C, bool QG = false, bool BI = false>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
gma_causal2_kernel(CausalArgs a) {
  using R = Causal2<C>;
  static_assert(HM == 0 || (!XS && CF::Kp == 2 * C::Kp && CF::DRP == C::DRP), "half scan");
  static_assert(!QG || (HM == 0 && !XS), "given responsibilities: one pass");
  static_assert(!BI || QG, "read-out on given responsibilities");
  __shared__ __attribute__((aligned(16))) bf16x8 coef[QG ? 1 : R::COEF * 64];
  __shared__ __attribute__((aligned(16))) float cperm[QG ? 1 : R::KP];
  // Gamma^K^T: KP rows of 64 keys, swizzled as swz_elem<8> (unpadded, filled
  // by 1 KB direct copies)
  __shared__ __attribute__((aligned(16))) bf16 G[R::NB][R::KP * kTile];
  __shared__ __attribute__((aligned(16))) bf16 Vb[R::NB][kTile * C::DV];
  __shared__ __attribute__((aligned(16))) bf16 ST[R::STCH * 512];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int64_t bh = blockIdx.y;
  const int h = (int)(bh % a.H);
  const int span = blockIdx.x;
  const int64_t t_begin = (int64_t)span * a.span_tiles * kTile;
  const int64_t t_end = a.N < t_begin + (int64_t)a.span_tiles * kTile
                            ? a.N : t_begin + (int64_t)a.span_tiles * kTile;
  const int nchunks = t_end > t_begin ? (int)((t_end - t_begin + kTile - 1) / kTile) : 0;
  const bool want_aq = a.assign_q != nullptr;
  const int koff = HM ? a.koff : 0;

  // ---- tables, carried state -------------------------------------------------
  {
    if constexpr (!QG) {
      const char* tb = a.params + (size_t)h * a.head_bytes + a.head_bytes / 2;
      const bf16x8* src = reinterpret_cast<const bf16x8*>(tb) + (size_t)(koff / 16) * R::NKS * 4 * 64;
      for (int idx = threadIdx.x; idx < R::COEF * 64; idx += kThreads) coef[idx] = src[idx];
      const float* cp = reinterpret_cast<const float*>(tb + (size_t)8 * CF::Kp * CF::DRP) + koff;
      for (int j = threadIdx.x; j < R::KP; j += kThreads) cperm[j] = cp[j];
    } else {
      // the Gamma^K^T rows past kc are never copied: zero in both buffers
      for (int idx = a.kc * kTile / 8 + threadIdx.x; idx < R::KP * kTile / 8; idx += kThreads)
#pragma unroll
        for (int bb = 0; bb < R::NB; ++bb) reinterpret_cast<bf16x8*>(G[bb])[idx] = bf16x8{};
    }
    // the (Z_hi, Z_lo, 1) block: the ones row and the zero rows are constant
    // (rows 0 and 1 belong to write_st, which runs concurrently)
    for (int idx = threadIdx.x; idx < (BI ? 0 : R::KS * 64); idx += kThreads) {
      const int r = idx & 15;
      if (r < 2) continue;
      bf16x8 v;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (bf16)(r == 2 ? 1.0f : 0.0f);
      reinterpret_cast<bf16x8*>(ST)[R::DVT * R::KS * 64 + idx] = v;
    }
  }
  // the state entering this span: the earlier spans' totals summed in span
  // order (the order of an exclusive scan over spans), SB spans' loads issued
  // before their adds; a slot past the earlier spans adds zeros
  f32x4 sacc[R::CTW][R::DVT], zacc[R::CTW];
#pragma unroll
  for (int j = 0; j < R::CTW; ++j) {
    zacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < R::DVT; ++dt) sacc[j][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if constexpr (!BI) {
    constexpr int V1 = R::CTW * (R::DVT + 1) * 4;          // values per lane per span
    constexpr int SB = V1 >= 48 ? 1 : 96 / V1;
    for (int s0 = 0; s0 < span; s0 += SB) {
      f32x4 ts[SB][R::CTW][R::DVT], tz[SB][R::CTW];
#pragma unroll
      for (int b = 0; b < SB; ++b) {
        const bool in = s0 + b < span;
        const size_t sl = (size_t)bh * a.nspan + (in ? s0 + b : 0);
#pragma unroll
        for (int j = 0; j < R::CTW; ++j) {
          const int comp0 = koff + (w * R::CTW + j) * 16;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            tz[b][j][i] = in ? a.state_z[sl * CF::Kp + comp0 + 4 * g + i] : 0.f;
#pragma unroll
          for (int dt = 0; dt < R::DVT; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              ts[b][j][dt][i] = in ? a.state[(sl * CF::Kp + comp0 + 4 * g + i) * C::DV + dt * 16 + c] : 0.f;
        }
      }
#pragma unroll
      for (int b = 0; b < SB; ++b)
#pragma unroll
        for (int j = 0; j < R::CTW; ++j) {
#pragma unroll
          for (int i = 0; i < 4; ++i) zacc[j][i] += tz[b][j][i];
#pragma unroll
          for (int dt = 0; dt < R::DVT; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) sacc[j][dt][i] += ts[b][j][dt][i];
        }
    }
  }
  // this wave's rows of the state table: S^T (d rows in pair_row order) and Z.
  // A lane's four components 4g .. 4g+3 of a tile are four consecutive
  // elements of one 16-byte operand chunk: one 8-byte store per (tile, d).
  auto write_st = [&]() {
#pragma unroll
    for (int j = 0; j < R::CTW; ++j) {
      const int comp = (w * R::CTW + j) * 16 + 4 * g;
      const int p = comp >> 5, gg = (comp & 31) >> 3, e = comp & 7;
#pragma unroll
      for (int dt = 0; dt < R::DVT; ++dt) {
        const int d = dt * 16 + c;
        bf16x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = to_bf16(sacc[j][dt][i]);
        *reinterpret_cast<bf16x4*>(&ST[((pair_tile(d) * R::KS + p) * 64 + pair_rowof(d) + 16 * gg) * 8 + e]) = v;
      }
      if (c < 2) {
        bf16x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float zz = zacc[j][i];
          const float zh = from_bf16(to_bf16(zz));
          v[i] = to_bf16(c == 0 ? zz : zz - zh);
        }
        *reinterpret_cast<bf16x4*>(&ST[((R::DVT * R::KS + p) * 64 + c + 16 * gg) * 8 + e]) = v;
      }
    }
  };
  if constexpr (BI) {
    const bf16x8* src = reinterpret_cast<const bf16x8*>(a.vtab) + (size_t)bh * R::STCH * 64;
    for (int idx = threadIdx.x; idx < R::STCH * 64; idx += kThreads)
      reinterpret_cast<bf16x8*>(ST)[idx] = src[idx];
  } else {
    write_st();
  }

  const bf16* qs = reinterpret_cast<const bf16*>(a.q) + (size_t)bh * a.N * C::DR;
  const bf16* vs = reinterpret_cast<const bf16*>(a.v) + (size_t)bh * a.N * C::DV;
  const bf16* qls = XS ? reinterpret_cast<const bf16*>(a.q_lo) + (size_t)bh * a.N * C::DR : qs;
  // Gamma^K^T tiles of this sequence: [chunk][CF::Kp][64] bf16, this half's rows
  // (given responsibilities: [chunk][kc][64])
  const int64_t nch = (a.N + kTile - 1) / kTile;
  const int grows = QG ? a.kc : CF::Kp;
  const bf16* gts = a.gt + (size_t)bh * nch * grows * kTile + (size_t)koff * kTile;
  // routing vectors of a chunk's queries (given responsibilities: their
  // exponentials), loaded two chunks ahead: two register buffers, chunks
  // alternating between them
  constexpr int NX = QG ? R::KS : R::NKS;
  bf16x8 xqA[NX], xqlA[NX];
  bf16x8 xqB[NX], xqlB[NX];
  auto load_x = [&](int k, bf16x8 (&xq)[NX], bf16x8 (&xql)[NX]) {
    const int64_t tok = t_begin + (int64_t)k * kTile + 16 * w + c;
    if constexpr (QG) {
      const bf16* es = a.eq + (size_t)bh * a.N * a.kc;
#pragma unroll
      for (int p = 0; p < R::KS; ++p) {
        const bool ok = tok < t_end && 32 * p < a.kc;
        const size_t off = ok ? (size_t)tok * a.kc + 32 * p + 8 * g : 0;
        const bf16x8 e = ld16_nt<bf16x8>(es + off);
        xq[p] = ok ? e : bf16x8{};
      }
      return;
    }
#pragma unroll
    for (int s = 0; s < R::NKS; ++s) {
      const int col = 32 * s + 8 * g;
      const bool ok = tok < t_end && col < C::DR;
      const size_t off = (size_t)(ok ? tok : t_begin) * C::DR + (ok ? col : 0);
      const bf16x8 q = ld16_nt<bf16x8>(qs + off);
      xq[s] = ok ? q : bf16x8{};
      if constexpr (XS) {
        const bf16x8 ql = ld16_nt<bf16x8>(qls + off);
        xql[s] = ok ? ql : bf16x8{};
      }
    }
  };
  auto load_v = [&](int k, int buf) {
    const int64_t t0 = t_begin + (int64_t)k * kTile;
    const int64_t rem = t_end - t0;
    const int nv = (int)(rem < kTile ? rem : kTile);
#pragma unroll
    for (int j = 0; j < R::VRPW; ++j) {
      const int round = w * R::VRPW + j;
      if (round < R::VROUNDS) {
        const int P = round * 64 + lane;
        const int r = P / R::VROWCH, pc = P - r * R::VROWCH;
        const int lc = pc ^ ((2 * r) & (R::VROWCH - 2));
        const int rr = r < nv ? r : nv - 1;
        global_to_lds16_nt(vs + (size_t)(t0 + rr) * C::DV + lc * 8, &Vb[buf][round * 512]);
      }
    }
  };
  // Gamma^K^T tile of chunk k: lane l of copy j fills component row 8 j + l / 8,
  // physical chunk l % 8 (logical chunk of keys (l % 8) ^ (2 row mod 8))
  auto load_g = [&](int k, int buf) {
    const bf16* src = gts + (size_t)(t_begin / kTile + k) * grows * kTile;
#pragma unroll
    for (int j = 0; j < R::GRPW; ++j) {
      const int round = w * R::GRPW + j;
      if (QG && round * 8 >= a.kc) continue;
      const int row = round * 8 + (lane >> 3), pc = lane & 7;
      const int lc = pc ^ ((2 * row) & 6);
      global_to_lds16_nt(src + (size_t)row * kTile + lc * 8, &G[buf][round * 512]);
    }
  };
  bf16x8 ones, ones_r3;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    ones[e] = (bf16)1.0f;
    ones_r3[e] = (bf16)(c == 3 ? 1.0f : 0.0f);          // A operand: row 3 = 1
  }
  if (nchunks > 0) {
    load_x(0, xqA, xqlA);
    if constexpr (!BI) {
      load_v(0, 0);
      load_g(0, 0);
    }
  }
  if (nchunks > 1) load_x(1, xqB, xqlB);
  __syncthreads();                       // coefficient table and seeds visible to every wave

  // one chunk; xq, xql hold its routing vectors and afterwards receive those of
  // chunk k + 2
  auto chunk = [&](int k, bf16x8 (&xq)[NX], bf16x8 (&xql)[NX]) {
    const int buf = R::NB == 2 ? (k & 1) : 0;
    const int64_t tile0 = t_begin + (int64_t)k * kTile;
    const int64_t rem = t_end - tile0;
    const int nvalid = (int)(rem < kTile ? rem : kTile);
    asm volatile("" ::: "memory");
    const int qi = 16 * w + c;                      // this lane's query in the chunk
    const size_t qtok = (size_t)bh * a.N + (size_t)(tile0 + qi);
    // second half: the first half's partials of this lane's query (they arrive
    // while the scores are formed)
    f32x4 pnum[HM == 2 ? R::DVT : 1];
    f32x4 pq{1.f, 0.f, 0.f, 0.f};
    if constexpr (HM == 2) {
#pragma unroll
      for (int dt = 0; dt < R::DVT; ++dt) pnum[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (qi < nvalid) {
        const float* prow = a.qpart + qtok * C::DV + 8 * g;
#pragma unroll
        for (int qd = 0; qd < R::DVT / 2; ++qd) {
          pnum[2 * qd] = *reinterpret_cast<const f32x4*>(prow + 32 * qd);
          pnum[2 * qd + 1] = *reinterpret_cast<const f32x4*>(prow + 32 * qd + 4);
        }
        pq = *reinterpret_cast<const f32x4*>(a.qpart2 + qtok);
      }
    }
    // e = exp2(s - max), packed as the B operand of the contractions over
    // components
    bf16x8 Eq[R::KS];
    float mq = 0.f, qbv = 0.f;
    int qbi = 0;
    if constexpr (QG) {
#pragma unroll
      for (int p = 0; p < R::KS; ++p) Eq[p] = xq[p];
    } else {
      // features of this wave's 16 queries
      bf16x8 fq[R::NKS][NFX<XS>];
#pragma unroll
      for (int s = 0; s < R::NKS; ++s) make_features<XS>(xq[s], xql[s], fq[s]);
      // scores D[component][query]
      f32x4 SQ[R::CT];
#pragma unroll
      for (int ct = 0; ct < R::CT; ++ct) SQ[ct] = *reinterpret_cast<const f32x4*>(&cperm[ct * 16 + 4 * g]);
      {
        // half-steps h = (component tile, routing chunk): the four operands of
        // half-step h + 1 are read from LDS while the MFMAs of h run
        constexpr int NH = R::CT * R::NKS;
        auto load_w = [&](int hs, bf16x8 (&wv)[4]) {
          const int ct = hs / R::NKS, s = hs % R::NKS;
#pragma unroll
          for (int ar = 0; ar < 4; ++ar) wv[ar] = coef[((ct * R::NKS + s) * 4 + ar) * 64 + lane];
        };
        bf16x8 wbuf[2][4];
        load_w(0, wbuf[0]);
#pragma unroll
        for (int hs = 0; hs < NH; ++hs) {
          if (hs + 1 < NH) load_w(hs + 1, wbuf[(hs + 1) & 1]);
          __builtin_amdgcn_sched_barrier(0);
          const int ct = hs / R::NKS, s = hs % R::NKS;
#pragma unroll
          for (int q = 0; q < NQX<XS>; ++q) SQ[ct] = mma(wbuf[hs & 1][kWI[q]], fq[s][kFI[q]], SQ[ct]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }

      {
        float v = SQ[0][0];
#pragma unroll
        for (int ct = 0; ct < R::CT; ++ct)
#pragma unroll
          for (int i = 0; i < 4; ++i) v = fmaxf(v, SQ[ct][i]);
        const float m = groups_max(v);
        mq = m;
#pragma unroll
        for (int p = 0; p < R::KS; ++p)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            Eq[p][i] = to_bf16(exp2_fast(SQ[2 * p][i] - m));
            Eq[p][4 + i] = to_bf16(exp2_fast(SQ[2 * p + 1][i] - m));
          }
        if (want_aq) {
          // the lowest component index whose score equals the maximum m (one of
          // the scores: the maxima select, they do not round)
          int bi = 0x7fffffff;
#pragma unroll
          for (int ct = 0; ct < R::CT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              bi = min(bi, SQ[ct][i] == m ? koff + pair_row(ct, 4 * g + i) : 0x7fffffff);
          bi = groups_min_i(bi);
          qbv = m;
          qbi = bi;
          if (HM == 0 && g == 0 && qi < nvalid) a.assign_q[qtok] = bi;
        }
      }
    }
    if constexpr (!BI) {
      wait_global_loads();               // V(k), Gamma^K^T(k) and this wave's loads
      lds_barrier();                                                  // B1
    }
    if constexpr (R::NB == 2 && !BI) {
      if (k + 1 < nchunks) {
        load_v(k + 1, buf ^ 1);
        load_g(k + 1, buf ^ 1);
      }
    }
    if (k + 2 < nchunks) load_x(k + 2, xq, xql);

    // ---- outputs of this wave's 16 queries ------------------------------------
    f32x4 acc[R::OT];
#pragma unroll
    for (int dt = 0; dt < R::OT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // given responsibilities: the 32-component steps past kc are zero
    const int ksn = QG ? (a.kc + 31) / 32 : R::KS;
#pragma unroll
    for (int p = 0; p < R::KS; ++p) {
      if (QG && p >= ksn) break;
#pragma unroll
      for (int dt = 0; dt < R::OT; ++dt)
        acc[dt] = mma(reinterpret_cast<const bf16x8*>(ST)[(dt * R::KS + p) * 64 + lane], Eq[p], acc[dt]);
    }
    // intra-chunk: key pairs (32 keys; rows of key tile jt in tile_token order,
    // so a pair covers keys 32pp .. 32pp + 31) up to the one holding this wave's
    // queries, which is masked to keys <= query.  The A operand (key rows,
    // components 32p + 8g ..) is a transpose read of Gamma^K^T: source lane s
    // reads the four keys 8 (s % 4) + 4 jt .. of its component row.
    for (int pp = 0; pp <= (BI ? -1 : (w >> 1)); ++pp) {
      f32x4 P[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int jt = 2 * pp + b;
        P[b] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int blk = 32 * pp + 8 * (lane & 3) + 4 * b;
#pragma unroll
        for (int p = 0; p < R::KS; ++p) {
          if (QG && p >= ksn) break;
          P[b] = mma(tr_chunk_swz_blk<8>(G[buf], 32 * p, blk), Eq[p], P[b]);
        }
        if (pp == (w >> 1)) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (tile_token(jt, 4 * g + i) > qi) P[b][i] = 0.f;
        }
      }
      bf16x8 Pc;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        Pc[i] = to_bf16(P[0][i]);
        Pc[4 + i] = to_bf16(P[1][i]);
      }
      // V^T chunk with rows in pair_row order: source lane s reads block
      // pair_row(dt, 4 (s % 4))
      const int a4 = lane & 3;
#pragma unroll
      for (int dt = 0; dt < R::DVT; ++dt) {
        const bf16x8 Av = tr_chunk_swz_blk<R::VROWCH>(Vb[buf], 32 * pp, pair_row(dt, 4 * a4));
        acc[dt] = mma(Av, Pc, acc[dt]);
      }
      acc[R::DVT] = mma(ones_r3, Pc, acc[R::DVT]);
    }
    {
      // denominator: rows 0..3 of the last block (lane group 0), then every lane
      // takes the value of lane group 0
      const f32x4 dz = acc[R::DVT];
      float den = dz[0] + dz[1] + dz[3] + a.eps * dz[2];
      float r0, r1;
      pair_xor16(den, r0, r1);
      pair_xor32(r0, den, r1);
      if constexpr (HM == 1) {
        if (qi < nvalid) {
          float* prow = a.qpart + qtok * C::DV + 8 * g;
#pragma unroll
          for (int qd = 0; qd < R::DVT / 2; ++qd) {
            *reinterpret_cast<f32x4*>(prow + 32 * qd) = acc[2 * qd];
            *reinterpret_cast<f32x4*>(prow + 32 * qd + 4) = acc[2 * qd + 1];
          }
          if (g == 0) a.qpart2[qtok] = float4{den, mq, qbv, __int_as_float(qbi)};
        }
      } else {
        // second half: both halves rescaled to the larger maximum
        float s0 = 0.f, s1 = 1.f;
        if constexpr (HM == 2) {
          const float M = fmaxf(mq, pq[1]);
          s0 = exp2_fast(pq[1] - M);
          s1 = exp2_fast(mq - M);
          den = s0 * pq[0] + s1 * den;
        }
        const float r = fast_rcp(den);
        s0 *= r;
        s1 *= r;
        if (qi < nvalid) {
          bf16* orow = reinterpret_cast<bf16*>(a.out) + qtok * C::DV;
#pragma unroll
          for (int qd = 0; qd < R::DVT / 2; ++qd) {
            bf16x8 o8;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              if constexpr (HM == 2) {
                o8[i] = to_bf16(acc[2 * qd][i] * s1 + pnum[2 * qd][i] * s0);
                o8[4 + i] = to_bf16(acc[2 * qd + 1][i] * s1 + pnum[2 * qd + 1][i] * s0);
              } else {
                o8[i] = to_bf16(acc[2 * qd][i] * s1);
                o8[4 + i] = to_bf16(acc[2 * qd + 1][i] * s1);
              }
            }
            st16(orow + 32 * qd + 8 * g, o8);
          }
          // the lowest component at the overall maximum: the first half's on a tie
          if (HM == 2 && want_aq && g == 0)
            a.assign_q[qtok] = qbv > pq[2] ? qbi : __float_as_int(pq[3]);
        }
      }
    }
    if constexpr (BI) return;
    lds_barrier();                                                    // B2

    // ---- state update on this wave's components: S += Gamma^K^T V, z += Gamma^K^T 1
    // (keys past the end of the sequence, in its last chunk, are cleared)
#pragma unroll
    for (int P2 = 0; P2 < 2; ++P2) {
#pragma unroll
      for (int j = 0; j < R::CTW; ++j) {
        if (QG && (w * R::CTW + j) * 16 >= a.kc) continue;      // rows past kc: zero
        const int comp = (w * R::CTW + j) * 16 + c;
        bf16x8 Ag = *reinterpret_cast<const bf16x8*>(&G[buf][swz_elem<8>(comp, 32 * P2 + 8 * g)]);
        if (nvalid < kTile) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (32 * P2 + 8 * g + e >= nvalid) Ag[e] = (bf16)0.f;
        }
        zacc[j] = mma(Ag, ones, zacc[j]);
#pragma unroll
        for (int dt = 0; dt < R::DVT; ++dt)
          sacc[j][dt] = mma(Ag, tr_chunk_swz<R::VROWCH>(Vb[buf], 32 * P2, dt * 16), sacc[j][dt]);
      }
    }
    write_st();
    if constexpr (R::NB == 1) {
      lds_barrier();                                                  // B3: G, V free
      if (k + 1 < nchunks) {
        load_v(k + 1, 0);
        load_g(k + 1, 0);
      }
    }
  };
  for (int k = 0; k < nchunks; k += 2) {
    chunk(k, xqA, xqlA);
    if (k + 1 < nchunks) chunk(k + 1, xqB, xqlB);
  }
}

// Span totals of the fused layer from the keys' given responsibilities:
// S_span = sum over the span's chunks c of Gamma^K_c^T V_c and z_span =
// Gamma^K_c^T 1 (the memories of "Causal GMA", Eq. 8b, summed over one span),
// each wave on its component tiles as in the scan's state update.  A ring of
// four tile buffers filled by direct global -> LDS copies keeps three chunks
// in flight.
template <class C, int KC>
__global__ void __launch_bounds__(kThreads) gma_gt_totals_kernel(CausalArgs a, float* state,
                                                                 float* state_z) {
  using R = Causal2<C>;
  constexpr int NBUF = 4;
  constexpr int GRW = KC * kTile * 2 / 1024 / kWaves;      // 1 KB copies per wave and chunk
  constexpr int VRW = R::VROUNDS / kWaves;
  constexpr int L = GRW + VRW;
  static_assert(KC * kTile * 2 / 1024 % kWaves == 0 && R::VROUNDS % kWaves == 0 && KC <= R::KP,
                "copies divide among the waves");
  __shared__ __attribute__((aligned(16))) bf16 G[NBUF][KC * kTile];
  __shared__ __attribute__((aligned(16))) bf16 Vb[NBUF][kTile * C::DV];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int64_t bh = blockIdx.y;
  const int span = blockIdx.x;
  const int64_t t_begin = (int64_t)span * a.span_tiles * kTile;
  const int64_t t_end = a.N < t_begin + (int64_t)a.span_tiles * kTile
                            ? a.N : t_begin + (int64_t)a.span_tiles * kTile;
  const int nchunks = t_end > t_begin ? (int)((t_end - t_begin + kTile - 1) / kTile) : 0;
  const bf16* vs = reinterpret_cast<const bf16*>(a.v) + (size_t)bh * a.N * C::DV;
  const int64_t nch = (a.N + kTile - 1) / kTile;
  const bf16* gts = a.gt + (size_t)bh * nch * KC * kTile;

  auto load = [&](int k, int buf) {
    const int64_t t0 = t_begin + (int64_t)k * kTile;
    const int64_t rem = t_end - t0;
    const int nv = (int)(rem < kTile ? rem : kTile);
#pragma unroll
    for (int j = 0; j < VRW; ++j) {
      const int round = w * VRW + j;
      const int P = round * 64 + lane;
      const int r = P / R::VROWCH, pc = P - r * R::VROWCH;
      const int lc = pc ^ ((2 * r) & (R::VROWCH - 2));
      const int rr = r < nv ? r : nv - 1;
      global_to_lds16_nt(vs + (size_t)(t0 + rr) * C::DV + lc * 8, &Vb[buf][round * 512]);
    }
    const bf16* src = gts + (size_t)(t_begin / kTile + k) * KC * kTile;
#pragma unroll
    for (int j = 0; j < GRW; ++j) {
      const int round = w * GRW + j;
      const int row = round * 8 + (lane >> 3), pc = lane & 7;
      const int lc = pc ^ ((2 * row) & 6);
      global_to_lds16_nt(src + (size_t)row * kTile + lc * 8, &G[buf][round * 512]);
    }
  };

  f32x4 sacc[R::CTW][R::DVT], zacc[R::CTW];
#pragma unroll
  for (int j = 0; j < R::CTW; ++j) {
    zacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < R::DVT; ++dt) sacc[j][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (bf16)1.0f;

  for (int k = 0; k < NBUF - 1 && k < nchunks; ++k) load(k, k);
  for (int k = 0; k < nchunks; ++k) {
    const int buf = k % NBUF;
    // chunk k's copies are complete once at most those of the chunks issued
    // after it (k + 1 .. k + NBUF - 2) are outstanding
    const int later = (nchunks - 1 < k + NBUF - 2 ? nchunks - 1 : k + NBUF - 2) - k;
    if (later >= 2) wait_vmcnt<2 * L>();
    else if (later == 1) wait_vmcnt<L>();
    else wait_global_loads();
    lds_barrier();                       // every wave's copies of chunk k; chunk k - 1 read
    if (k + NBUF - 1 < nchunks) load(k + NBUF - 1, (k + NBUF - 1) % NBUF);
    const int64_t rem = t_end - (t_begin + (int64_t)k * kTile);
    const int nvalid = (int)(rem < kTile ? rem : kTile);
#pragma unroll
    for (int P2 = 0; P2 < 2; ++P2) {
#pragma unroll
      for (int j = 0; j < R::CTW; ++j) {
        if ((w * R::CTW + j) * 16 >= KC) continue;
        const int comp = (w * R::CTW + j) * 16 + c;
        bf16x8 Ag = *reinterpret_cast<const bf16x8*>(&G[buf][swz_elem<8>(comp, 32 * P2 + 8 * g)]);
        if (nvalid < kTile) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (32 * P2 + 8 * g + e >= nvalid) Ag[e] = (bf16)0.f;
        }
        zacc[j] = mma(Ag, ones, zacc[j]);
#pragma unroll
        for (int dt = 0; dt < R::DVT; ++dt)
          sacc[j][dt] = mma(Ag, tr_chunk_swz<R::VROWCH>(Vb[buf], 32 * P2, dt * 16), sacc[j][dt]);
      }
    }
  }
  // this span's totals, [BH][nspan][K_pad][d_v] and [BH][nspan][K_pad]
  const size_t sl = (size_t)bh * a.nspan + span;
#pragma unroll
  for (int j = 0; j < R::CTW; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int comp = (w * R::CTW + j) * 16 + 4 * g + i;
      if (c == 0) state_z[sl * R::KP + comp] = zacc[j][i];
#pragma unroll
      for (int dt = 0; dt < R::DVT; ++dt) state[(sl * R::KP + comp) * C::DV + dt * 16 + c] = sacc[j][dt][i];
    }
}

// The fused layer's forward after the projection epilogue: span totals from
// the keys' responsibilities, then the scan (causal) or the read-out over all
// spans' totals (bidirectional) on the given responsibilities.
template <class C>
static hipError_t run_causal_fused(const Plan& p, const Tensors& t, bool causal, hipStream_t s) {
  if constexpr (!(C::kBF && Causal2<C>::kOK)) {
    return hipErrorNotSupported;
  } else {
    if (t.kc != 32 && t.kc != 64) return hipErrorInvalidValue;
    CausalArgs ca{};
    ca.v = t.v;
    ca.out = t.out;
    ca.N = p.N;
    ca.H = (int)p.H;
    ca.nspan = p.nspan;
    ca.span_tiles = p.span_tiles;
    ca.eps = t.eps;
    ca.out_bf = p.out_bf ? 1 : 0;
    ca.gt = reinterpret_cast<const bf16*>(t.ws + p.off_gt);
    ca.eq = static_cast<const bf16*>(t.eq);
    ca.kc = t.kc;
    float* state = reinterpret_cast<float*>(t.ws + p.off_state);
    float* state_z = reinterpret_cast<float*>(t.ws + p.off_state_z);
    ca.state = state;
    ca.state_z = state_z;
    const dim3 grid(p.nspan, (unsigned)p.BH);
    if (g_launch_hook) g_launch_hook("gma_span_state", s, 1);
    if (t.kc == 32)
      hipLaunchKernelGGL((gma_gt_totals_kernel<C, 32>), grid, dim3(kThreads), 0, s, ca, state, state_z);
    else
      hipLaunchKernelGGL((gma_gt_totals_kernel<C, 64>), grid, dim3(kThreads), 0, s, ca, state, state_z);
    if (g_launch_hook) g_launch_hook("gma_span_state", s, 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (causal) {
      if (g_launch_hook) g_launch_hook("gma_causal", s, 1);
      hipLaunchKernelGGL((gma_causal2_kernel<C, false, 0, C, true>), grid, dim3(kThreads), 0, s, ca);
      if (g_launch_hook) g_launch_hook("gma_causal", s, 0);
    } else {
      // the spans' totals summed in span order into the read-out's operand
      // table, then the read-out over runs of four chunks
      if (!t.vtab) return hipErrorInvalidValue;
      if (g_launch_hook) g_launch_hook("gma_reduce", s, 1);
      e = launch_reduce_table(state, state_z, p.nspan, p.BH, C::Kp, C::DV,
                              reinterpret_cast<float*>(t.ws + p.off_carry),
                              reinterpret_cast<float*>(t.ws + p.off_carry_z),
                              static_cast<bf16*>(t.vtab), s);
      if (g_launch_hook) g_launch_hook("gma_reduce", s, 0);
      if (e != hipSuccess) return e;
      ca.vtab = static_cast<const bf16*>(t.vtab);
      ca.span_tiles = p.tiles < 4 ? (int)p.tiles : 4;
      const dim3 rgrid((unsigned)((p.tiles + ca.span_tiles - 1) / ca.span_tiles), (unsigned)p.BH);
      if (g_launch_hook) g_launch_hook("gma_read", s, 1);
      hipLaunchKernelGGL((gma_causal2_kernel<C, false, 0, C, true, true>), rgrid, dim3(kThreads), 0, s, ca);
      if (g_launch_hook) g_launch_hook("gma_read", s, 0);
    }
    return hipGetLastError();
  }
}

template <class C>
static hipError_t run_causal(const Plan& p, const Tensors& t, hipStream_t s) {
  // K_pad = 256 where the scan tables exceed LDS: the scan runs once per half
  // of the components (CH)
  constexpr bool KH = causal_khalf(C::kBF, C::DRP, C::DV, C::Kp);
  using CH = Cfg<C::kBF, (C::CPW > 1 ? C::CPW / 2 : 1), 4, C::DR, C::DV>;
  static_assert(!KH || (WriteTeam<C>::kOK && Causal2<CH>::kOK && CH::Kp * 2 == C::Kp),
                "K-half scan");
  // the token-owner scan takes the keys' responsibilities (and assignments)
  // from the span-totals pass, which must then be a token-owner write
  constexpr bool TOK = KH || Causal2<C>::kOK;
  static_assert(!TOK || WriteTeam<C>::kOK || Write2<C>::kOK, "span pass storing Gamma^K^T");
  if constexpr (!KH && causal_lds_bytes(C::kBF, C::DR, C::DV, C::Kp) > kMaxLds) {
    return hipErrorNotSupported;     // rejected earlier by validation
  } else {
  // 1. span totals through the latent-write kernel (one split per span)
  BidirArgs wa{};
  const bool split = t.k_lo != nullptr;
  if (split && (KH || !(Causal2<C>::kOK && (WriteTeam<C>::kOK || Write2<C>::kOK))))
    return hipErrorNotSupported;
  wa.x = t.k;
  wa.x_lo = t.k_lo;
  wa.v = t.v;
  wa.params = t.ws + p.off_params;
  wa.head_bytes = p.head_bytes;
  wa.partial = reinterpret_cast<float*>(t.ws + p.off_state);
  wa.partial_z = reinterpret_cast<float*>(t.ws + p.off_state_z);
  wa.N = p.N;
  wa.H = (int)p.H;
  wa.K = p.K;
  wa.S = p.nspan;
  wa.tiles_per_split = p.span_tiles;
  wa.assign = nullptr;
  const dim3 grid(p.nspan, (unsigned)p.BH);
  if (g_launch_hook) g_launch_hook("gma_span_state", s, 1);
  if constexpr (TOK) {
    // a token-owner write (one split per span of 2 span_tiles 32-key groups)
    // that also stores the keys' Gamma^K^T tiles and assignments
    wa.gpw = 2 * p.span_tiles;
    wa.gt = reinterpret_cast<bf16*>(t.ws + p.off_gt);
    wa.assign = t.assign_k;
    if constexpr (WriteTeam<C>::kOK) {
      if (split) {
        if (t.assign_k) hipLaunchKernelGGL((gma_write_team_kernel<C, true, true, true>), grid, dim3(512), 0, s, wa);
        else hipLaunchKernelGGL((gma_write_team_kernel<C, true, false, true>), grid, dim3(512), 0, s, wa);
      } else {
        if (t.assign_k) hipLaunchKernelGGL((gma_write_team_kernel<C, false, true, true>), grid, dim3(512), 0, s, wa);
        else hipLaunchKernelGGL((gma_write_team_kernel<C, false, false, true>), grid, dim3(512), 0, s, wa);
      }
    } else if constexpr (Write2<C>::kOK) {
      if (split) hipLaunchKernelGGL((gma_write2_kernel<C, true, true>), grid, dim3(256), 0, s, wa);
      else hipLaunchKernelGGL((gma_write2_kernel<C, false, true>), grid, dim3(256), 0, s, wa);
    }
  } else if (WriteTeam<C>::kOK && (split || p.span_tiles >= 4)) {
    // the token-owner write pays a per-workgroup set-up (its coefficient
    // table): use it for spans of at least four 32-token steps per wave, or
    // eight where it runs one wave per SIMD; one split per span.  Team write:
    // a span is 2 span_tiles 32-key groups.
    wa.gpw = 2 * p.span_tiles;
    if constexpr (WriteTeam<C>::kOK) {
      if (split) hipLaunchKernelGGL((gma_write_team_kernel<C, true, false>), grid, dim3(512), 0, s, wa);
      else hipLaunchKernelGGL((gma_write_team_kernel<C, false, false>), grid, dim3(512), 0, s, wa);
    }
  } else if (Write2<C>::kOK && (split || p.span_tiles >= (Write2<C>::WPE == 2 ? 4 : 16))) {
    wa.gpw = 2 * p.span_tiles;
    if constexpr (Write2<C>::kOK) {
      if (split) hipLaunchKernelGGL((gma_write2_kernel<C, true>), grid, dim3(256), 0, s, wa);
      else hipLaunchKernelGGL((gma_write2_kernel<C, false>), grid, dim3(256), 0, s, wa);
    }
  } else if constexpr (C::kBF) {
    hipLaunchKernelGGL(gma_write_bf16_kernel<C>, grid, dim3(kThreads), 0, s, wa);
  } else {
    hipLaunchKernelGGL(gma_write_kernel<C>, grid, dim3(kThreads), 0, s, wa);
  }
  if (g_launch_hook) g_launch_hook("gma_span_state", s, 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  // 2. exclusive scan over spans (the token-owner scan sums the earlier spans'
  // totals itself)
  if constexpr (!TOK) {
  const int nred = C::Kp * C::DV + C::Kp;
  if (g_launch_hook) g_launch_hook("gma_span_scan", s, 1);
  hipLaunchKernelGGL(gma_span_scan_kernel, dim3((nred + 255) / 256, (unsigned)p.BH), dim3(256), 0,
                     s, wa.partial, wa.partial_z, p.nspan, C::Kp, C::DV,
                     reinterpret_cast<float*>(t.ws + p.off_carry),
                     reinterpret_cast<float*>(t.ws + p.off_carry_z));
  if (g_launch_hook) g_launch_hook("gma_span_scan", s, 0);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  }

  // 3. chunked scan
  CausalArgs ca{};
  ca.q = t.q;
  ca.k = t.k;
  ca.v = t.v;
  ca.out = t.out;
  ca.params = t.ws + p.off_params;
  ca.head_bytes = p.head_bytes;
  ca.carry = reinterpret_cast<const float*>(t.ws + p.off_carry);
  ca.carry_z = reinterpret_cast<const float*>(t.ws + p.off_carry_z);
  ca.assign_q = t.assign_q;
  ca.assign_k = t.assign_k;
  ca.N = p.N;
  ca.H = (int)p.H;
  ca.nspan = p.nspan;
  ca.span_tiles = p.span_tiles;
  ca.eps = t.eps;
  ca.out_bf = p.out_bf ? 1 : 0;
  ca.q_lo = t.q_lo;
  ca.k_lo = t.k_lo;
  if (g_launch_hook) g_launch_hook("gma_causal", s, 1);
  ca.gt = TOK ? reinterpret_cast<const bf16*>(t.ws + p.off_gt) : nullptr;
  ca.state = reinterpret_cast<const float*>(t.ws + p.off_state);
  ca.state_z = reinterpret_cast<const float*>(t.ws + p.off_state_z);
  if constexpr (KH) {
    // the first half leaves its partials, the second combines them
    ca.qpart = reinterpret_cast<float*>(t.ws + p.off_qpart);
    ca.qpart2 = reinterpret_cast<float4*>(t.ws + p.off_qpart2);
    ca.koff = 0;
    hipLaunchKernelGGL((gma_causal2_kernel<CH, false, 1, C>), grid, dim3(kThreads), 0, s, ca);
    ca.koff = CH::Kp;
    hipLaunchKernelGGL((gma_causal2_kernel<CH, false, 2, C>), grid, dim3(kThreads), 0, s, ca);
  } else if constexpr (Causal2<C>::kOK) {
    if (split) hipLaunchKernelGGL((gma_causal2_kernel<C, true>), grid, dim3(kThreads), 0, s, ca);
    else hipLaunchKernelGGL((gma_causal2_kernel<C, false>), grid, dim3(kThreads), 0, s, ca);
  } else {
    hipLaunchKernelGGL(gma_causal_kernel<C>, grid, dim3(kThreads), 0, s, ca);
  }
  if (g_launch_hook) g_launch_hook("gma_causal", s, 0);
  return hipGetLastError();
  }
}

#define GMA_CDV_CASES(BF, CPW, DR)                                          \
  switch (p.DV) {                                                           \
    case 16: return run_causal<Cfg<BF, CPW, 4, DR, 16>>(p, t, s);           \
    case 32: return run_causal<Cfg<BF, CPW, 4, DR, 32>>(p, t, s);           \
    case 64: return run_causal<Cfg<BF, CPW, 4, DR, 64>>(p, t, s);           \
    case 128: return run_causal<Cfg<BF, CPW, 4, DR, 128>>(p, t, s);         \
  }                                                                         \
  break;
#define GMA_CDR_CASES(BF, CPW)                                              \
  switch (p.DR) {                                                           \
    case 16: GMA_CDV_CASES(BF, CPW, 16)                                     \
    case 32: GMA_CDV_CASES(BF, CPW, 32)                                     \
    case 64: GMA_CDV_CASES(BF, CPW, 64)                                     \
    case 128: GMA_CDV_CASES(BF, CPW, 128)                                   \
  }                                                                         \
  break;

template <class C>
static hipError_t causal_split_query(const Plan&, const Tensors&, hipStream_t) {
  return Causal2<C>::kOK && (WriteTeam<C>::kOK || Write2<C>::kOK) ? hipSuccess
                                                                   : hipErrorNotSupported;
}
#define GMA_CSDV_CASES(CPW, DR)                                             \
  switch (p.DV) {                                                           \
    case 16: return causal_split_query<Cfg<true, CPW, 4, DR, 16>>(p, t, s); \
    case 32: return causal_split_query<Cfg<true, CPW, 4, DR, 32>>(p, t, s); \
    case 64: return causal_split_query<Cfg<true, CPW, 4, DR, 64>>(p, t, s); \
    case 128: return causal_split_query<Cfg<true, CPW, 4, DR, 128>>(p, t, s); \
  }                                                                         \
  break;
static hipError_t causal_split_query_all(const Plan& p, const Tensors& t, hipStream_t s) {
  if (p.NG != 4) return hipErrorNotSupported;
  switch (p.DR) {
    case 16: if (p.CPW == 1) { GMA_CSDV_CASES(1, 16) } else if (p.CPW == 2) { GMA_CSDV_CASES(2, 16) } else { GMA_CSDV_CASES(4, 16) } break;
    case 32: if (p.CPW == 1) { GMA_CSDV_CASES(1, 32) } else if (p.CPW == 2) { GMA_CSDV_CASES(2, 32) } else { GMA_CSDV_CASES(4, 32) } break;
    case 64: if (p.CPW == 1) { GMA_CSDV_CASES(1, 64) } else if (p.CPW == 2) { GMA_CSDV_CASES(2, 64) } else { GMA_CSDV_CASES(4, 64) } break;
    case 128: if (p.CPW == 1) { GMA_CSDV_CASES(1, 128) } else if (p.CPW == 2) { GMA_CSDV_CASES(2, 128) } else { GMA_CSDV_CASES(4, 128) } break;
  }
  return hipErrorNotSupported;
}

bool causal_split_ok(const Plan& p) {
  return p.bf && causal_split_query_all(p, Tensors{}, nullptr) == hipSuccess;
}

bool layer_fused_ok(const Plan& p) {
  return p.bf && !p.prod && !p.khalf && p.NG == 4 && p.Kp == 64 && p.DR == 64 &&
         p.DV >= 32 && causal2_lds_bytes(true, p.DRP, p.DV, p.Kp) > 0;
}

#define GMA_FUSED_DV(DR)                                                            \
  switch (p.DV) {                                                                   \
    case 32: return run_causal_fused<Cfg<true, 1, 4, DR, 32>>(p, t, causal, s);     \
    case 64: return run_causal_fused<Cfg<true, 1, 4, DR, 64>>(p, t, causal, s);     \
    case 128: return run_causal_fused<Cfg<true, 1, 4, DR, 128>>(p, t, causal, s);   \
  }                                                                                 \
  break;
hipError_t launch_layer_fused(const Plan& p, const Tensors& t, bool causal, hipStream_t s) {
  if (!layer_fused_ok(p)) return hipErrorInvalidValue;
  switch (0) {
    default: GMA_FUSED_DV(64)
  }
  return hipErrorInvalidValue;
}

hipError_t launch_causal(const Plan& p, const Tensors& t, hipStream_t s) {
  if (p.NG != 4) return hipErrorInvalidValue;
  if (p.bf) {
    if (p.CPW == 1) { switch (0) { default: GMA_CDR_CASES(true, 1) } }
    else if (p.CPW == 2) { switch (0) { default: GMA_CDR_CASES(true, 2) } }
    else { switch (0) { default: GMA_CDR_CASES(true, 4) } }
  } else {
    if (p.CPW == 1) { switch (0) { default: GMA_CDR_CASES(false, 1) } }
    else if (p.CPW == 2) { switch (0) { default: GMA_CDR_CASES(false, 2) } }
    else { switch (0) { default: GMA_CDR_CASES(false, 4) } }
  }
  return hipErrorInvalidValue;
}

}  // namespace gma
