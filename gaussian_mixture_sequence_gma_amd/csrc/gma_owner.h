// Token-owner building blocks shared by the bidirectional and causal paths:
// the paired row order of 32-row blocks, a transpose read with per-lane
// column blocks, and the token-owner latent write.  See gma_bidir.hip for the
// method summary.
#pragma once

#include "gma_tiles.h"

namespace gma {

// Row r of the t-th 16-row MFMA tile of a 32-row pair block: 32 (t / 2) +
// 8 (r / 4) + 4 (t % 2) + r % 4.  With it, lane group g (rows 4g .. 4g+3 of a
// D tile) of tiles 2p and 2p + 1 together holds the eight consecutive indices
// 32p + 8g .. 32p + 8g + 7.
__host__ __device__ constexpr int pair_row(int t, int r) {
  return 32 * (t >> 1) + 8 * (r >> 2) + 4 * (t & 1) + (r & 3);
}
// Inverse: index i -> (tile, row).
__host__ __device__ constexpr int pair_tile(int i) { return 2 * (i >> 5) + ((i & 7) >> 2); }
__host__ __device__ constexpr int pair_rowof(int i) { return 4 * ((i & 31) >> 3) + (i & 3); }

// Score operands of one 8-wide routing chunk.  bf16 routing vectors x (exact
// squares): features (x^2 hi, x^2 lo, x) and five products x^2_hi A_hi,
// x^2_lo A_hi, x^2_hi A_lo, x B_hi, x B_lo.  Split routing vectors x = xh + xl
// (two bf16 parts, 16 significant bits): x^2 is formed in fp32 and split, the
// features gain xl and a sixth product xl B_hi (xl B_lo is below 2^-16 of x B).
template <bool XS> constexpr int NFX = XS ? 4 : 3;
template <bool XS> constexpr int NQX = XS ? 6 : 5;
constexpr int kWI[6] = {0, 0, 1, 2, 3, 2};   // A_hi, A_hi, A_lo, B_hi, B_lo, B_hi
constexpr int kFI[6] = {0, 1, 0, 2, 2, 3};   // x^2_hi, x^2_lo, x^2_hi, x, x, x_lo
template <bool XS>
__device__ __forceinline__ void make_features(const bf16x8& xh, const bf16x8& xl,
                                              bf16x8 (&f)[NFX<XS>]) {
  if constexpr (!XS) {
    // Per pair of elements (one 32-bit word): widen both to fp32 (a shift and a
    // mask), square, round the pair to bf16 in one conversion (x^2 hi), and
    // take the remainders x^2 - hi with one bf16 dot product each (hi . (-1, 0)
    // + x^2): exact, since x^2 has at most 16 significant bits and the
    // remainder at most 8, so its top half is the exact bf16 (x^2 lo).
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const u32x4 p = __builtin_bit_cast(u32x4, xh);
    // the bf16 pairs (-1, 0) and (0, -1), materialised in registers by a move
    // the compiler cannot see through: as an inline constant of the dot
    // product's packed-bf16 operand, -1.0 would be open to reinterpretation
    unsigned k0, k1;
    asm("v_mov_b32 %0, 0xbf80" : "=v"(k0));
    asm("v_mov_b32 %0, 0xbf800000" : "=v"(k1));
    const bf16x2 m0 = __builtin_bit_cast(bf16x2, k0);   // (-1, 0)
    const bf16x2 m1 = __builtin_bit_cast(bf16x2, k1);   // (0, -1)
    u32x4 hi, lo;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a0 = __uint_as_float(p[j] << 16), a1 = __uint_as_float(p[j] & 0xffff0000u);
      const float q0 = a0 * a0, q1 = a1 * a1;
      const bf16x2 h = {(bf16)q0, (bf16)q1};      // one v_cvt_pk_bf16_f32 (RNE)
      const float l0 = __builtin_amdgcn_fdot2_f32_bf16(h, m0, q0, false);
      const float l1 = __builtin_amdgcn_fdot2_f32_bf16(h, m1, q1, false);
      hi[j] = __builtin_bit_cast(unsigned, h);
      lo[j] = __builtin_amdgcn_perm(__float_as_uint(l1), __float_as_uint(l0), 0x07060302u);
    }
    f[0] = __builtin_bit_cast(bf16x8, hi);
    f[1] = __builtin_bit_cast(bf16x8, lo);
    f[2] = xh;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = from_bf16(xh[e]) + from_bf16(xl[e]);
      bf16 hh, ll;
      split_bf16(x * x, hh, ll);
      f[0][e] = hh;
      f[1][e] = ll;
    }
    f[2] = xh;
    f[3] = xl;
  }
}

// Like tr_chunk_swz, but source lane s reads the 4-column block blk (a multiple
// of 4) chosen by the caller for s % 4: destination lane 4a + e then receives
// column blk(a) + e of the eight rows tok0 + 8g .. tok0 + 8g + 7.
template <int ROWCH>
__device__ __forceinline__ bf16x8 tr_chunk_swz_blk(const bf16* M, int tok0, int blk) {
  const int lane = threadIdx.x & 63, s = lane & 15, g = lane >> 4;
  const int row = tok0 + 8 * g + (s >> 2);
  const short4_t lo = lds_read_tr16(M + swz_elem<ROWCH>(row, blk));
  const short4_t hi = lds_read_tr16(M + swz_elem<ROWCH>(row + 4, blk));
  typedef short short8_t __attribute__((ext_vector_type(8)));
  const short8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// ============================================================================
// Latent write, bf16 inputs, token-owner form.  Every wave owns 32 keys at a
// time and all K_pad components, and accumulates its own V~ (K_pad x d_v, in
// the accumulation registers) and Z over all its keys, so the main loop has no
// barrier and no exchange between waves: the per-key softmax stays inside the
// wave.  The workgroup shares the score-coefficient table of the read-out
// (same LDS layout); each wave stages its own V tiles (32 keys, swizzled rows)
// by direct global -> LDS copies, double-buffered.
// Scores use D[key][component] with key rows in tile_token order, so lane
// group g of the two key tiles holds keys 8g .. 8g + 7: the normalised
// responsibilities are the A operand of V~ += Gamma^T V straight from
// registers.  The four waves' partial V~ and Z are added in LDS at the end, in
// a fixed order.
// ============================================================================
template <class C>
struct Write2 {
  static constexpr int KP = C::Kp;
  static constexpr int CT = KP / 16;
  static constexpr int NKS = C::DRP / 32;
  static constexpr int DVT = C::DV / 16;
  static constexpr int ROWCH = C::DV / 8;                 // 16-byte chunks per V row
  static constexpr int VT = 32 * C::DV;                   // bf16 elements of one V tile
  static constexpr int NDMA = VT * 2 / 1024;               // 1 KB wave copies per V tile
  static constexpr int COEF = CT * NKS * 4;
  static constexpr int LOOP_LDS = COEF * 1024 + KP * 4 + 4 * 2 * VT * 2;
  static constexpr int RED_LDS = 2 * (KP * C::DV + 4 * KP) * 4;   // two partial slots
  static constexpr int LDS = LOOP_LDS > RED_LDS ? LOOP_LDS : RED_LDS;
  static constexpr bool kOK = C::kBF && KP % 32 == 0 && C::DRP <= 64 && C::DV >= 32 &&
                              LDS <= 160 * 1024 && CT * DVT * 4 <= 256;
  // waves per SIMD: two where V~ takes at most 64 accumulation registers
  static constexpr int WPE = CT * DVT * 4 <= 64 ? 2 : 1;
};

// GT: the keys' Gamma^K^T tiles are stored to a.gt (the causal span-totals pass)
template <class C, bool XS, bool GT = false>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(Write2<C>::WPE, Write2<C>::WPE)))
gma_write2_kernel(BidirArgs a) {
  using R = Write2<C>;
  constexpr int NW = 4;
  __shared__ __attribute__((aligned(16))) char lds[R::LDS];
  bf16x8* coef = reinterpret_cast<bf16x8*>(lds);
  float* cperm = reinterpret_cast<float*>(lds + R::COEF * 1024);
  bf16* vbuf = reinterpret_cast<bf16*>(lds + R::COEF * 1024 + R::KP * 4);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int64_t bh = blockIdx.y;
  const int h = (int)(bh % a.H);
  const bool want_assign = a.assign != nullptr;

  {
    const char* tb = a.params + (size_t)h * a.head_bytes + a.head_bytes / 2;
    const bf16x8* src = reinterpret_cast<const bf16x8*>(tb);
    for (int idx = threadIdx.x; idx < R::COEF * 64; idx += NW * 64) coef[idx] = src[idx];
    const float* cp = reinterpret_cast<const float*>(tb + (size_t)8 * C::Kp * C::DRP);
    for (int j = threadIdx.x; j < R::KP; j += NW * 64) cperm[j] = cp[j];
  }
  __syncthreads();

  // with Gamma^K^T tiles requested, every 64-key chunk is covered whole (the
  // keys past N get responsibilities 0)
  const int64_t G32 = GT ? 2 * ((a.N + 63) / 64) : (a.N + 31) / 32;
  const int64_t gpw = a.gpw > 0 ? a.gpw : (G32 + gridDim.x - 1) / gridDim.x;
  const int64_t gb = (int64_t)blockIdx.x * gpw;
  const int64_t ge = gb + gpw < G32 ? gb + gpw : G32;
  const bf16* xs = reinterpret_cast<const bf16*>(a.x) + (size_t)bh * a.N * C::DR;
  const bf16* vs = reinterpret_cast<const bf16*>(a.v) + (size_t)bh * a.N * C::DV;
  bf16* myv = vbuf + wave * 2 * R::VT;

  // key row r of key tile tt is key 8 (r / 4) + 4 tt + r % 4 of the group.  The
  // loads are unconditional (clamped address, value zeroed afterwards) so that
  // every group issues the same number of memory operations: the wait for the
  // V copies below counts them.
  const bf16* xls = XS ? reinterpret_cast<const bf16*>(a.x_lo) + (size_t)bh * a.N * C::DR : xs;
  bf16x8 xr[2][R::NKS], xl[2][R::NKS];
  auto load_x = [&](int64_t grp) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int64_t tok = grp * 32 + tile_token(tt, c);
#pragma unroll
      for (int s = 0; s < R::NKS; ++s) {
        const int col = 32 * s + 8 * g;
        const bool ok = tok < a.N && col < C::DR;
        const size_t off = (size_t)(ok ? tok : 0) * C::DR + (ok ? col : 0);
        const bf16x8 v = ld16_nt<bf16x8>(xs + off);
        xr[tt][s] = ok ? v : bf16x8{};
        if constexpr (XS) {
          const bf16x8 vl = ld16_nt<bf16x8>(xls + off);
          xl[tt][s] = ok ? vl : bf16x8{};
        }
      }
    }
  };
  // V tile of a group -> buffer b: lane l of copy j fills row j * 1024 / (2 d_v) +
  // l / ROWCH, physical chunk l % ROWCH (swizzled as swz_elem<ROWCH>)
  auto load_v = [&](int64_t grp, int b) {
    constexpr int RPK = 512 / C::DV;      // rows per 1 KB copy
#pragma unroll
    for (int j = 0; j < R::NDMA; ++j) {
      const int row = j * RPK + lane / R::ROWCH, pc = lane % R::ROWCH;
      const int lc = R::ROWCH >= 2 ? (pc ^ ((2 * row) & (R::ROWCH - 2))) : pc;
      int64_t tok = grp * 32 + row;
      if (tok >= a.N) tok = a.N - 1;                       // rows past the end get Gamma = 0
      global_to_lds16_nt(vs + (size_t)tok * C::DV + lc * 8, myv + b * R::VT + j * 512);
    }
  };

  f32x4 acc[R::CT][R::DVT];
#pragma unroll
  for (int ct = 0; ct < R::CT; ++ct)
#pragma unroll
    for (int dt = 0; dt < R::DVT; ++dt) acc[ct][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float zacc[R::CT];
#pragma unroll
  for (int ct = 0; ct < R::CT; ++ct) zacc[ct] = 0.f;

  int64_t grp = gb + wave;
  int buf = 0;
  if (grp < ge) {
    load_x(grp);
    load_v(grp, 0);
  }
  for (; grp < ge; grp += NW, buf ^= 1) {
    asm volatile("" ::: "memory");      // keep the table reads inside the loop
    bf16x8 f[2][R::NKS][NFX<XS>];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int s = 0; s < R::NKS; ++s) make_features<XS>(xr[tt][s], xl[tt][s], f[tt][s]);
    const bool more = grp + NW < ge;
    if (more) load_v(grp + NW, buf ^ 1);

    f32x4 S[2][R::CT];
#pragma unroll
    for (int ct = 0; ct < R::CT; ++ct) {
      const float cv = cperm[ct * 16 + c];
      S[0][ct] = f32x4{cv, cv, cv, cv};
      S[1][ct] = S[0][ct];
    }
    // half-steps h = (component tile, routing chunk): the four operands of
    // half-step h + 1 are read from LDS while the MFMAs of h run
    constexpr int NH = R::CT * R::NKS;
    auto load_w = [&](int hs, bf16x8 (&w)[4]) {
      const int ct = hs / R::NKS, s = hs % R::NKS;
#pragma unroll
      for (int ar = 0; ar < 4; ++ar) w[ar] = coef[((ct * R::NKS + s) * 4 + ar) * 64 + lane];
    };
    bf16x8 wbuf[2][4];
    load_w(0, wbuf[0]);
#pragma unroll
    for (int hs = 0; hs < NH; ++hs) {
      if (hs + 1 < NH) load_w(hs + 1, wbuf[(hs + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      const int ct = hs / R::NKS, s = hs % R::NKS;
#pragma unroll
      for (int q = 0; q < NQX<XS>; ++q)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
          S[tt][ct] = mma(f[tt][s][kFI[q]], wbuf[hs & 1][kWI[q]], S[tt][ct]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (more) load_x(grp + NW);

    // per key (row 4g + i of key tile tt): softmax over the CT columns of this
    // lane and the 16 lanes of its row
    bf16x8 A[R::CT];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float m = S[tt][0][i];
#pragma unroll
        for (int ct = 1; ct < R::CT; ++ct) m = fmaxf(m, S[tt][ct][i]);
        m = row16_max(m);
        const int64_t tok = grp * 32 + 8 * g + 4 * tt + i;
        if (want_assign) {
          // the lowest component index whose score equals the maximum m (one
          // of the scores: the maxima select, they do not round)
          int bi = 0x7fffffff;
#pragma unroll
          for (int ct = 0; ct < R::CT; ++ct)
            bi = min(bi, S[tt][ct][i] == m ? pair_row(ct, c) : 0x7fffffff);
          bi = min(bi, dpp_i<0xB1>(bi));
          bi = min(bi, dpp_i<0x4E>(bi));
          bi = min(bi, dpp_i<0x141>(bi));
          bi = min(bi, dpp_i<0x140>(bi));
          if (c == 0 && tok < a.N) a.assign[(size_t)bh * a.N + tok] = bi;
        }
        float l = 0.f;
#pragma unroll
        for (int ct = 0; ct < R::CT; ++ct) {
          const float e = exp2_fast(S[tt][ct][i] - m);
          S[tt][ct][i] = e;
          l += e;
        }
        l = row16_sum(l);
        const float inv = tok < a.N ? fast_rcp(l) : 0.f;
#pragma unroll
        for (int ct = 0; ct < R::CT; ++ct) {
          const float gm = S[tt][ct][i] * inv;
          zacc[ct] += gm;
          A[ct][4 * tt + i] = to_bf16(gm);
        }
      }
    // Gamma^K^T for the causal scan: lane (c, g) holds component pair_row(ct, c)
    // of keys 8g .. 8g + 7, one 16-byte store each
    if constexpr (GT) {
      bf16* gdst = a.gt + ((size_t)bh * ((a.N + 63) / 64) + (size_t)(grp >> 1)) * C::Kp * 64 +
                   (grp & 1) * 32 + 8 * g;
#pragma unroll
      for (int ct = 0; ct < R::CT; ++ct) st16(gdst + (size_t)pair_row(ct, c) * 64, A[ct]);
    }

    // V(grp) has arrived once at most the copies and loads of the next group
    // (issued after it) are outstanding
    if (more) {
      wait_vmcnt<R::NDMA + (XS ? 4 : 2) * R::NKS>();
    } else {
      wait_global_loads();
    }
    const bf16* vt = myv + buf * R::VT;
#pragma unroll
    for (int dt = 0; dt < R::DVT; ++dt) {
      const bf16x8 vb = tr_chunk_swz<R::ROWCH>(vt, 0, dt * 16);
#pragma unroll
      for (int ct = 0; ct < R::CT; ++ct) acc[ct][dt] = mma(A[ct], vb, acc[ct][dt]);
    }
  }

  // ---- the four waves' partials, added in LDS in a fixed order --------------------
  __syncthreads();
  float* red = reinterpret_cast<float*>(lds);
  constexpr int NV = R::CT * R::DVT * 4;
  auto put = [&](int slot) {
    float* r = red + slot * (NV + R::CT) * 64;
#pragma unroll
    for (int ct = 0; ct < R::CT; ++ct) {
#pragma unroll
      for (int dt = 0; dt < R::DVT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) r[((ct * R::DVT + dt) * 4 + i) * 64 + lane] = acc[ct][dt][i];
      r[(NV + ct) * 64 + lane] = zacc[ct];
    }
  };
  auto add = [&](int slot) {
    const float* r = red + slot * (NV + R::CT) * 64;
#pragma unroll
    for (int ct = 0; ct < R::CT; ++ct) {
#pragma unroll
      for (int dt = 0; dt < R::DVT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[ct][dt][i] += r[((ct * R::DVT + dt) * 4 + i) * 64 + lane];
      zacc[ct] += r[(NV + ct) * 64 + lane];
    }
  };
  if (wave >= 2) put(wave - 2);
  __syncthreads();
  if (wave < 2) add(wave);
  __syncthreads();
  if (wave == 1) put(0);
  __syncthreads();
  if (wave == 0) {
    add(0);
    const size_t pslot = (size_t)bh * gridDim.x + blockIdx.x;
    float* pv = a.partial + pslot * C::Kp * C::DV;
    float* pz = a.partial_z + pslot * C::Kp;
#pragma unroll
    for (int ct = 0; ct < R::CT; ++ct) {
#pragma unroll
      for (int dt = 0; dt < R::DVT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) pv[pair_row(ct, 4 * g + i) * C::DV + dt * 16 + c] = acc[ct][dt][i];
      // lanes of one column c hold different keys: sum the four groups
      const float zt = groups_sum(zacc[ct]);
      if (g == 0) pz[pair_row(ct, c)] = zt;
    }
  }
}

}  // namespace gma
