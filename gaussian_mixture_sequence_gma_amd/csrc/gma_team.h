// Team latent write: the token-owner write of gma_owner.h with the components
// of every 32-key group split over a team of waves, so that each wave holds
// only a 64-component slice of V~ and the kernel runs two waves per SIMD at
// K_pad = 128 (four-wave teams at K_pad = 256).
//
// What is computed is the latent aggregation of "Gaussian Mixture Attention:
// Linear-Time Sequence Mixing via Probabilistic Latent Routing", Eqs. 5-6:
// V~ = Gamma^K^T V_X and Z = Gamma^K^T 1, with gamma the posterior of Eq. 3
// (a softmax over all K components of the Gaussian scores, Eq. 16).
//
// Wave r of a team owns components [64 r, 64 r + 64).  Per group it scores its
// components for the team's 32 keys (split-bf16 MFMA, coefficients from the
// LDS operand table), takes the per-key maximum m_r and sum l_r = sum_k
// exp2(s_k - m_r) over its own components, and posts (m_r, l_r) to LDS.  Once
// every wave of the team has posted, each combines the records of the whole
// team: M = max_w m_w, L = sum_w l_w exp2(m_w - M), and its responsibilities
// are gamma = exp2(s - m_r) exp2(m_r - M) / L, the softmax over all K
// components.  Then V~_slice += Gamma_slice^T V on MFMA from a V tile the team
// shares (staged by direct global -> LDS copies, split over the team's waves).
// The only synchronisation is between the waves of a team, through LDS flags;
// teams run independently (no workgroup barrier in the main loop).
//
// The V tiles live in an LDS array of their own: the compiler then knows that
// no other LDS access aliases the copies in flight and does not wait for them
// before the coefficient reads or the team's records.  The next round's copies
// are issued after this round's reads of the current tile.
#pragma once

#include "gma_owner.h"

namespace gma {

template <class C>
struct WriteTeam {
  static constexpr int KP = C::Kp;
  static constexpr int TS = KP / 64 > 0 ? KP / 64 : 1;    // waves per team
  static constexpr int CTW = 4;                           // 16-component tiles per wave
  static constexpr int NKS = C::DRP / 32;
  static constexpr int DVT = C::DV / 16;
  static constexpr int ROWCH = C::DV / 8;                 // 16-byte chunks per V row
  static constexpr int VT = 32 * C::DV;                   // bf16 elements of one V tile
  static constexpr int NDMA = VT * 2 / 1024;              // 1 KB wave copies per V tile
  static constexpr int NDW = NDMA / TS > 0 ? NDMA / TS : 1;   // copies per wave
  static constexpr int NW = 8;                            // waves per workgroup
  static constexpr int NT = NW / TS;                      // teams per workgroup
  static constexpr int COEF = (KP / 16) * NKS * 4;        // 1 KB operand chunks
  // V tiles: [team][NVB buffers] of VT bf16, their own array; two buffers
  // where they fit, else one (the team then also waits for its waves' reads
  // of a tile before the next tile's copies)
  static constexpr int MAIN0 = COEF * 1024 + KP * 4 + NT * 2 * TS * 32 * 16 + NW * 64 * 4 + 2 * NW * 4;
  static constexpr int NVB = MAIN0 + NT * 2 * VT * 2 <= 160 * 1024 ? 2 : 1;
  static constexpr int VSH = NT * NVB * VT;
  // the other LDS: coefficient table, c, exchange records [team][round
  // parity][wave] of 128 floats (m of the 32 keys, then l, then the argmax,
  // then unused), factor tables [wave][64], flags [wave] for the records and
  // [wave] for the V tile reads
  static constexpr int OFF_C = COEF * 1024;
  static constexpr int OFF_X = OFF_C + KP * 4;
  static constexpr int OFF_FT = OFF_X + NT * 2 * TS * 32 * 16;
  static constexpr int OFF_F = OFF_FT + NW * 64 * 4;
  static constexpr int MAIN = OFF_F + 2 * NW * 4;
  // epilogue: one wave's V~ slice and Z per slot; the main array holds
  // SLOTS_M slots, the V array SLOTS_V
  static constexpr int SLICE = (CTW * DVT * 4 + CTW) * 64;  // floats
  static constexpr int SLOTS_M = MAIN / (SLICE * 4);
  static constexpr int SLOTS_V = 0;
  static constexpr bool kOK = C::kBF && (KP == 128 || KP == 256) && C::DRP <= 64 &&
                              C::DV >= 32 && NDMA % TS == 0 && SLOTS_M >= 1 &&
                              MAIN + VSH * 2 <= 160 * 1024;
};

// LDS flag of a team member: post a round number after the records (release:
// every LDS write of this wave before it is visible first), wait for one.
// Both fences order LDS only, so global loads in flight stay in flight.
__device__ __forceinline__ void team_post(int* flag, int v) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __hip_atomic_store(flag, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void team_wait(const int* flag, int v) {
  while (__builtin_amdgcn_readfirstlane(
             __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) < v)
    __builtin_amdgcn_s_sleep(1);
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// AS: key assignments are written (a.assign non-null); GT: the keys'
// Gamma^K^T tiles are stored to a.gt (the causal span-totals pass)
template <class C, bool XS, bool AS, bool GT = false>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
gma_write_team_kernel(BidirArgs a) {
  using R = WriteTeam<C>;
  constexpr int TS = R::TS, NT = R::NT, CTW = R::CTW;
  __shared__ __attribute__((aligned(16))) char lds[R::MAIN];
  __shared__ __attribute__((aligned(16))) bf16 vsh[R::VSH];
  bf16x8* coef = reinterpret_cast<bf16x8*>(lds);
  float* cperm = reinterpret_cast<float*>(lds + R::OFF_C);
  int* flags = reinterpret_cast<int*>(lds + R::OFF_F);

  // the wave index is uniform within a wave: keep it (and everything derived
  // from it) in scalar registers
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int team = wave / TS, r = wave % TS;
  const int c = lane & 15, g = lane >> 4;
  const int64_t bh = blockIdx.y;
  const int h = (int)(bh % a.H);
  constexpr bool want_assign = AS;

  {
    const char* tb = a.params + (size_t)h * a.head_bytes + a.head_bytes / 2;
    const bf16x8* src = reinterpret_cast<const bf16x8*>(tb);
    for (int idx = threadIdx.x; idx < R::COEF * 64; idx += R::NW * 64) coef[idx] = src[idx];
    const float* cp = reinterpret_cast<const float*>(tb + (size_t)8 * C::Kp * C::DRP);
    for (int j = threadIdx.x; j < R::KP; j += R::NW * 64) cperm[j] = cp[j];
    if (threadIdx.x < 2 * R::NW) flags[threadIdx.x] = 0;
  }
  __syncthreads();

  bf16* const vbuf = vsh + team * R::NVB * R::VT;
  float4* xch = reinterpret_cast<float4*>(lds + R::OFF_X) + team * 2 * TS * 32;
  int* tflags = flags + team * TS;
  int* vflags = flags + R::NW + team * TS;            // one V buffer: reads done
  float* ftab = reinterpret_cast<float*>(lds + R::OFF_FT) + wave * 64;   // [32] factor, [32] argmax

  // with Gamma^K^T tiles requested, every 64-key chunk is covered whole (the
  // keys past N get responsibilities 0)
  const int64_t G32 = GT ? 2 * ((a.N + 63) / 64) : (a.N + 31) / 32;
  const int64_t gpw = a.gpw > 0 ? a.gpw : (G32 + gridDim.x - 1) / gridDim.x;
  const int64_t gb = (int64_t)blockIdx.x * gpw;
  const int64_t ge = gb + gpw < G32 ? gb + gpw : G32;
  // per-sequence slabs as buffer resources (their sizes are below 2^31 bytes):
  // keys past the end and routing columns past d_r read as zeros
  const bf16* xs = reinterpret_cast<const bf16*>(a.x) + (size_t)bh * a.N * C::DR;
  const bf16* vs = reinterpret_cast<const bf16*>(a.v) + (size_t)bh * a.N * C::DV;
  const bf16* xls = XS ? reinterpret_cast<const bf16*>(a.x_lo) + (size_t)bh * a.N * C::DR : xs;
  const uint32_t xbytes = (uint32_t)(a.N * C::DR * 2), vbytes = (uint32_t)(a.N * C::DV * 2);
  const buf_rsrc xrs = make_rsrc(xs, xbytes), xlrs = make_rsrc(xls, xbytes);
  const buf_rsrc vrs = make_rsrc(vs, vbytes);

  // routing vectors of a group: key row r' of key tile tt is key 8 (r' / 4) +
  // 4 tt + r' % 4 (tile_token order); keys past the end (their
  // responsibilities are set to zero below) load zeros
  bf16x8 xr[2][R::NKS], xl[2][R::NKS];
  auto load_x = [&](int64_t grp) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const uint32_t tok = (uint32_t)(grp * 32 + tile_token(tt, c));
#pragma unroll
      for (int s = 0; s < R::NKS; ++s) {
        const int col = 32 * s + 8 * g;
        const uint32_t off = col < C::DR ? (tok * C::DR + col) * 2 : 0xFFFFFFF0u;
        xr[tt][s] = buf_ld16_nt<bf16x8>(xrs, off);
        if constexpr (XS) xl[tt][s] = buf_ld16_nt<bf16x8>(xlrs, off);
      }
    }
  };
  constexpr int NXL = (XS ? 2 : 1) * 2 * R::NKS;          // loads per load_x
  // this wave's share of a group's V tile (copies j = r, r + TS, ...): lane l of
  // copy j fills row j * 512 / d_v + l / ROWCH, physical chunk l % ROWCH; rows
  // past the end are zeros
  auto load_v = [&](int64_t grp, int b) {
    constexpr int RPK = 512 / C::DV;
#pragma unroll
    for (int jj = 0; jj < R::NDW; ++jj) {
      const int j = r + TS * jj;
      const int row = j * RPK + lane / R::ROWCH, pc = lane % R::ROWCH;
      const int lc = R::ROWCH >= 2 ? (pc ^ ((2 * row) & (R::ROWCH - 2))) : pc;
      const uint32_t tok = (uint32_t)(grp * 32 + row);
      buf_to_lds16_nt(vrs, (tok * C::DV + lc * 8) * 2, vbuf + b * R::VT + j * 512);
    }
  };

  f32x4 acc[CTW][R::DVT];
#pragma unroll
  for (int ct = 0; ct < CTW; ++ct)
#pragma unroll
    for (int dt = 0; dt < R::DVT; ++dt) acc[ct][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Z accumulates the same bf16 responsibilities as V~ (pairs summed by a bf16
  // dot product with (1, 1))
  float zacc[CTW];
#pragma unroll
  for (int ct = 0; ct < CTW; ++ct) zacc[ct] = 0.f;
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  unsigned ones_bits;
  asm("v_mov_b32 %0, 0x3f803f80" : "=v"(ones_bits));
  const bf16x2 ones2 = __builtin_bit_cast(bf16x2, ones_bits);

  // Issue order per round: x(next) after the scores, V(next) after the V~
  // update; so at the top of a round x(this) is followed only by V(this)'s
  // copies, and before the post V(this) is followed only by x(next).
  int64_t grp = gb + team;
  int round = 0;
  if (grp < ge) {
    load_x(grp);
    load_v(grp, 0);
  }
  for (; grp < ge; grp += NT, ++round) {
    const int buf = round & 1;                        // record parity
    const int vbi = R::NVB == 2 ? buf : 0;            // V buffer
    asm volatile("" ::: "memory");      // keep the table reads inside the loop
    const bool more = grp + NT < ge;
    wait_vmcnt<R::NDW>();

    // ---- scores of this wave's components, D[key][component] -----------------
    f32x4 S[2][CTW];
#pragma unroll
    for (int ct = 0; ct < CTW; ++ct) {
      const float cv = cperm[(r * CTW + ct) * 16 + c];
      S[0][ct] = f32x4{cv, cv, cv, cv};
      S[1][ct] = S[0][ct];
    }
    // the score MFMAs at a raised wave priority: when the other wave on this SIMD
    // is in its softmax (VALU) phase, the two phases overlap instead of the
    // arbiter alternating between two waves in the same phase
    __builtin_amdgcn_s_setprio(2);
#pragma unroll
    for (int s = 0; s < R::NKS; ++s) {
      bf16x8 f[2][NFX<XS>];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) make_features<XS>(xr[tt][s], xl[tt][s], f[tt]);
#pragma unroll
      for (int ct = 0; ct < CTW; ++ct) {
        bf16x8 w[4];
        const int ctg = r * CTW + ct;
#pragma unroll
        for (int ar = 0; ar < 4; ++ar) w[ar] = coef[((ctg * R::NKS + s) * 4 + ar) * 64 + lane];
#pragma unroll
        for (int q = 0; q < NQX<XS>; ++q)
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
            S[tt][ct] = mma(f[tt][kFI[q]], w[kWI[q]], S[tt][ct]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    if (more) load_x(grp + NT);

    // ---- per key: local maximum and sum over this wave's components, posted as
    // the records m, l, argmax of keys 8 g + 4 tt + i by lane c = 0 of each
    // lane group ------------------------------------------------------------------
    // (each key tile's four records are posted as soon as they are formed, so
    // that only four keys' values are live at a time)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      float mm[4], ll[4];
      int bb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float m = S[tt][0][i];
#pragma unroll
        for (int ct = 1; ct < CTW; ++ct) m = fmaxf(m, S[tt][ct][i]);
        m = row16_max(m);
        m = fmaxf(m, -3.0e38f);          // a slice of padded components only: e = 0
        int bi = 0;
        if (want_assign) {
          // lowest component index of this slice at the maximum
          bi = 1 << 30;
#pragma unroll
          for (int ct = 0; ct < CTW; ++ct) {
            const int k = pair_row(r * CTW + ct, c);
            bi = (S[tt][ct][i] == m && k < bi) ? k : bi;
          }
          bi = min(bi, dpp_i<0xB1>(bi));
          bi = min(bi, dpp_i<0x4E>(bi));
          bi = min(bi, dpp_i<0x141>(bi));
          bi = min(bi, dpp_i<0x140>(bi));
        }
        float l = 0.f;
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct) {
          const float e = exp2_fast(S[tt][ct][i] - m);
          S[tt][ct][i] = e;
          l = ct == 0 ? e : l + e;
        }
        l = row16_sum(l);
        mm[i] = m;
        ll[i] = l;
        bb[i] = bi;
      }
      if (c == 0) {
        float4* rec = xch + (buf * TS + r) * 32 + 2 * g + tt;
        rec[0] = float4{mm[0], mm[1], mm[2], mm[3]};
        rec[8] = float4{ll[0], ll[1], ll[2], ll[3]};
        if (want_assign)
          rec[16] = float4{__int_as_float(bb[0]), __int_as_float(bb[1]), __int_as_float(bb[2]),
                           __int_as_float(bb[3])};
      }
    }
    // this wave's copies of V(grp) have landed once at most the x loads of the
    // next group are outstanding
    if (more) {
      wait_vmcnt<NXL>();
    } else {
      wait_global_loads();
    }
    team_post(tflags + r, round + 1);
#pragma unroll
    for (int w = 0; w < TS; ++w)
      if (w != r) team_wait(tflags + w, round + 1);

    // ---- combine the team's records, one key per lane (lane c < 8 of group g:
    // key 8 g + c): gamma = e * exp2(m_r - M) / L, written to this wave's factor
    // table and read back by the 16 lanes of each group ---------------------------
    if (c < 8) {
      const int key = 8 * g + c;
      const float* rb = reinterpret_cast<const float*>(xch + buf * TS * 32) + key;
      float mw[TS], lw[TS];
      int iw[TS];
#pragma unroll
      for (int w = 0; w < TS; ++w) {
        mw[w] = rb[w * 128];
        lw[w] = rb[w * 128 + 32];
        iw[w] = want_assign ? __float_as_int(rb[w * 128 + 64]) : 0;
      }
      float M = mw[0];
#pragma unroll
      for (int w = 1; w < TS; ++w) M = fmaxf(M, mw[w]);
      float L = 0.f, own = 0.f;
      int best = iw[TS - 1];
#pragma unroll
      for (int w = TS - 1; w >= 0; --w) {
        const float t = exp2_fast(mw[w] - M);
        L += lw[w] * t;
        if (w == r) own = t;
        if (mw[w] == M) best = iw[w];     // the lowest wave at the maximum wins
      }
      const int64_t tok = grp * 32 + key;
      ftab[key] = tok < a.N ? own * fast_rcp(L) : 0.f;
      if (want_assign) ftab[32 + key] = __int_as_float(best);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
    float fac[2][4];
    {
      const f32x4 f0 = *reinterpret_cast<const f32x4*>(ftab + 8 * g);
      const f32x4 f1 = *reinterpret_cast<const f32x4*>(ftab + 8 * g + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        fac[0][i] = f0[i];
        fac[1][i] = f1[i];
      }
    }
    bf16x8 A[CTW];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct) A[ct][4 * tt + i] = to_bf16(S[tt][ct][i] * fac[tt][i]);
#pragma unroll
    for (int ct = 0; ct < CTW; ++ct) {
      zacc[ct] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(A[ct], A[ct], 0, 1),
                                                 ones2, zacc[ct], false);
      zacc[ct] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(A[ct], A[ct], 2, 3),
                                                 ones2, zacc[ct], false);
      zacc[ct] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(A[ct], A[ct], 4, 5),
                                                 ones2, zacc[ct], false);
      zacc[ct] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(A[ct], A[ct], 6, 7),
                                                 ones2, zacc[ct], false);
    }
    if (want_assign && r == 0 && lane < 32) {
      const int64_t tok = grp * 32 + lane;
      if (tok < a.N) a.assign[(size_t)bh * a.N + tok] = __float_as_int(ftab[32 + lane]);
    }
    // Gamma^K^T for the causal scan: lane (c, g) holds component
    // pair_row(r CTW + ct, c) of keys 8g .. 8g + 7, one 16-byte store each
    if constexpr (GT) {
      bf16* gdst = a.gt + ((size_t)bh * ((a.N + 63) / 64) + (size_t)(grp >> 1)) * C::Kp * 64 +
                   (grp & 1) * 32 + 8 * g;
#pragma unroll
      for (int ct = 0; ct < CTW; ++ct)
        st16(gdst + (size_t)pair_row(r * CTW + ct, c) * 64, A[ct]);
    }

    // ---- V~_slice += Gamma_slice^T V ---------------------------------------------
    const bf16* vt = vbuf + vbi * R::VT;
#pragma unroll
    for (int dt = 0; dt < R::DVT; ++dt) {
      const bf16x8 vb = tr_chunk_swz<R::ROWCH>(vt, 0, dt * 16);
#pragma unroll
      for (int ct = 0; ct < CTW; ++ct) acc[ct][dt] = mma(A[ct], vb, acc[ct][dt]);
    }
    // every wave of the team has posted this round, so all have finished the
    // previous round's V~ update: its buffer takes the next group's tile (issued
    // after this wave's reads of the current tile).  With one buffer the team
    // first waits for all its waves' reads of this tile.
    if constexpr (R::NVB == 2) {
      if (more) load_v(grp + NT, buf ^ 1);
    } else {
      team_post(vflags + r, round + 1);
#pragma unroll
      for (int w = 0; w < TS; ++w)
        if (w != r) team_wait(vflags + w, round + 1);
      if (more) load_v(grp + NT, 0);
    }
  }

  // ---- the teams' slices, added into team 0 in a fixed order (team 1, 2, ...),
  // through slots in both LDS arrays --------------------------------------------
  constexpr int NV = CTW * R::DVT * 4;
  auto slot_ptr = [&](int k) -> float* { return reinterpret_cast<float*>(lds) + k * R::SLICE; };
  auto put = [&](float* q) {
#pragma unroll
    for (int ct = 0; ct < CTW; ++ct) {
#pragma unroll
      for (int dt = 0; dt < R::DVT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) q[((ct * R::DVT + dt) * 4 + i) * 64 + lane] = acc[ct][dt][i];
      q[(NV + ct) * 64 + lane] = zacc[ct];
    }
  };
  auto add = [&](const float* q) {
#pragma unroll
    for (int ct = 0; ct < CTW; ++ct) {
#pragma unroll
      for (int dt = 0; dt < R::DVT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[ct][dt][i] += q[((ct * R::DVT + dt) * 4 + i) * 64 + lane];
      zacc[ct] += q[(NV + ct) * 64 + lane];
    }
  };
  constexpr int NSLOT = R::SLOTS_M + R::SLOTS_V;
  // slices (t, r) for t >= 1 in order; each step moves up to NSLOT of them
  for (int first = TS; first < NT * TS; first += NSLOT) {
    __syncthreads();
    const int k = wave - first;
    if (k >= 0 && k < NSLOT) put(slot_ptr(k));
    __syncthreads();
    if (team == 0) {
      // wave (0, r) adds the slices (t, r) moved in this step, in order of t
      for (int k2 = 0; k2 < NSLOT && first + k2 < NT * TS; ++k2)
        if ((first + k2) % TS == r) add(slot_ptr(k2));
    }
  }
  if (team == 0) {
    const size_t pslot = (size_t)bh * gridDim.x + blockIdx.x;
    float* pv = a.partial + pslot * C::Kp * C::DV;
    float* pz = a.partial_z + pslot * C::Kp;
#pragma unroll
    for (int ct = 0; ct < CTW; ++ct) {
      const int ctg = r * CTW + ct;
#pragma unroll
      for (int dt = 0; dt < R::DVT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) pv[pair_row(ctg, 4 * g + i) * C::DV + dt * 16 + c] = acc[ct][dt][i];
      // lanes of one column c hold different keys: sum the four groups
      const float zt = groups_sum(zacc[ct]);
      if (g == 0) pz[pair_row(ctg, c)] = zt;
    }
  }
}

}  // namespace gma
