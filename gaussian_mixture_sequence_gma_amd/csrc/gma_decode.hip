// Causal decode step: one new token per sequence against a carried prefix
// state ("Gaussian Mixture Attention: Linear-Time Sequence Mixing via
// Probabilistic Latent Routing", Section "Causal GMA", the prefix memories and
// Eq. 8b).  With S = sum_{j<i} gamma^K_j v_j^T and z = sum_{j<i} gamma^K_j
// carried from the previous tokens, token i does
//   S' = S + gamma^K(k_i) v_i^T,  z' = z + gamma^K(k_i),
//   o_i = gamma^Q(q_i)^T S' / (gamma^Q(q_i)^T z' + eps),
// and S', z' replace S, z in place.  The responsibilities are Eq. 3 with the
// diagonal log-density written out directly (Eq. 2), in fp32.
//
// One workgroup (four waves) per sequence.  The step is bound by the state
// traffic (K x d_v fp32 read and written per sequence), so every thread
// issues the loads of its state rows first and the posterior is computed while
// they are in flight:
//   1. state rows -> registers (row r, four columns per thread, coalesced);
//   2. scores: d_r/16 lanes per component, 16 routing dims per lane, the
//      component parameters read once per component for q and k together;
//   3. posteriors: wave 0 softmax + argmax over the query scores, wave 1 over
//      the key scores (two components per lane), wave 1 also updates z;
//   4. S' = S + gamma^K v^T written back, each thread's share of
//      gamma^Q^T S' summed over its rows, then across rows through LDS.
#include <hip/hip_runtime.h>

#include "gma.h"
#include "gma_device.h"
#include "gma_internal.h"

namespace gma {

namespace {

struct DecodeArgs {
  const void* q;       // [BH, d_r]
  const void* k;       // [BH, d_r]
  const void* v;       // [BH, d_v]
  const float* mu;     // [H, K, d_r]
  const float* ls2;    // [H, K, d_r]
  const float* lpi;    // [H, K]
  float* sv;           // [BH, K, d_v] in/out
  float* sz;           // [BH, K] in/out
  void* out;           // [BH, d_v]
  int32_t* assign_q;   // [BH] or null
  int32_t* assign_k;   // [BH] or null
  int H, K;
  float eps;
};

// 16 consecutive elements starting at p (32-byte aligned for bf16, 64 for fp32) as fp32.
__device__ __forceinline__ void load16(const bf16* p, float (&x)[16]) {
  const bf16x8 a = ld16<bf16x8>(p), b = ld16<bf16x8>(p + 8);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    x[e] = from_bf16(a[e]);
    x[8 + e] = from_bf16(b[e]);
  }
}
__device__ __forceinline__ void load16(const float* p, float (&x)[16]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x4 a = ld16<f32x4>(p + 4 * i);
#pragma unroll
    for (int e = 0; e < 4; ++e) x[4 * i + e] = a[e];
  }
}
__device__ __forceinline__ f32x4 load4(const bf16* p) {
  const bf16* q = static_cast<const bf16*>(__builtin_assume_aligned(p, 8));
  return f32x4{from_bf16(q[0]), from_bf16(q[1]), from_bf16(q[2]), from_bf16(q[3])};
}
__device__ __forceinline__ f32x4 load4(const float* p) { return ld16<f32x4>(p); }
__device__ __forceinline__ void store1(bf16* p, float x) { *p = to_bf16(x); }
__device__ __forceinline__ void store1(float* p, float x) { *p = x; }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += xor_lane(v, o);
  return v;
}

template <class T, int DR, int DV, int KM>
__global__ void __launch_bounds__(256) gma_decode_kernel(DecodeArgs a) {
  constexpr int L = DR / 16;                 // lanes per component in the score pass
  constexpr int CW = 64 / L;                 // components per wave per score pass
  constexpr int C4 = DV / 4;                 // four-column groups of a state row
  constexpr int SR = 256 / C4;               // state rows per pass of the workgroup
  constexpr int NP = (KM + SR - 1) / SR;     // passes at the largest K (KM: 128 or 256)
  constexpr int CL = KM / 64;                // components per lane in the posterior
  static_assert(DR % 16 == 0 && DR <= 128 && DV % 16 == 0 && DV <= 128, "shape");
  static_assert(KM == 128 || KM == 256, "K bound");

  __shared__ float s_sc[2][KM];              // scores: queries, keys
  __shared__ float s_g[2][KM];               // responsibilities: queries, keys
  __shared__ float s_z[KM];                  // updated normaliser z'
  __shared__ __attribute__((aligned(16))) float s_red[SR * DV];
  __shared__ float s_den;

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t bh = blockIdx.x;
  const int h = (int)(bh % a.H);
  const int K = a.K;

  // 1. the token's routing vectors (16 dims per lane) and the component
  //    parameters of the first score passes are requested first, so that the
  //    scores wait only for them and not for the state behind them
  const int sl = (lane % L) * 16;
  float xq[16], xk[16];
  load16(static_cast<const T*>(a.q) + (size_t)bh * DR + sl, xq);
  load16(static_cast<const T*>(a.k) + (size_t)bh * DR + sl, xk);
  const float* mu = a.mu + (size_t)h * K * DR;
  const float* ls = a.ls2 + (size_t)h * K * DR;
  constexpr int PC = 4 * CW;                 // components per score pass
  constexpr int NPRE = PC >= 128 ? 1 : 2;    // passes whose parameters are preloaded
  f32x4 pm[NPRE][4], pv[NPRE][4];
  auto load_pass = [&](int c0, f32x4 (&m)[4], f32x4 (&l)[4]) {
    // rows past K re-read row K - 1; their scores are not stored
    const int c = min(c0 + wave * CW + lane / L, K - 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m[i] = ld16<f32x4>(mu + (size_t)c * DR + sl + 4 * i);
      l[i] = ld16<f32x4>(ls + (size_t)c * DR + sl + 4 * i);
    }
  };
#pragma unroll
  for (int j = 0; j < NPRE; ++j) load_pass(j * PC, pm[j], pv[j]);

  // 2. this thread's state rows r0 + p * SR, columns col .. col + 3.  Rows
  //    past K re-read row K - 1 (no branch around the loads) and are neither
  //    stored nor counted.
  const int col = (t % C4) * 4, r0 = t / C4;
  float* sv = a.sv + (size_t)bh * K * DV;
  f32x4 st[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p)
    st[p] = __builtin_nontemporal_load(
        reinterpret_cast<const f32x4*>(sv + (size_t)min(r0 + p * SR, K - 1) * DV + col));
  float zc[CL];
#pragma unroll
  for (int j = 0; j < CL; ++j) zc[j] = 0.f;
  if (wave == 1) {
#pragma unroll
    for (int j = 0; j < CL; ++j)
      if (lane + 64 * j < K) zc[j] = a.sz[(size_t)bh * K + lane + 64 * j];
  }
  const f32x4 vv = load4(static_cast<const T*>(a.v) + (size_t)bh * DV + col);

  // 3. scores s_c(x) = log pi_c - (1/2) sum_d [(x_d - mu_cd)^2 / sigma^2_cd + log sigma^2_cd]
  //    (the 2 pi term is common to all components and cancels in the posterior)
  auto score_pass = [&](int c0, const f32x4 (&m)[4], const f32x4 (&l)[4]) {
    const int c = c0 + wave * CW + lane / L;
    float pq = 0.f, pk = 0.f, pl = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float prec = expf(-l[i][e]);
        const float dq = xq[4 * i + e] - m[i][e], dk = xk[4 * i + e] - m[i][e];
        pq += dq * dq * prec;
        pk += dk * dk * prec;
        pl += l[i][e];
      }
    }
#pragma unroll
    for (int o = 1; o < L; o <<= 1) {
      pq += xor_lane(pq, o);
      pk += xor_lane(pk, o);
      pl += xor_lane(pl, o);
    }
    if (c < K && lane % L == 0) {
      const float lp = a.lpi[(size_t)h * K + c];
      s_sc[0][c] = lp - 0.5f * (pq + pl);
      s_sc[1][c] = lp - 0.5f * (pk + pl);
    }
  };
#pragma unroll
  for (int j = 0; j < NPRE; ++j)
    if (j * PC < K) score_pass(j * PC, pm[j], pv[j]);
#pragma unroll 1
  for (int c0 = NPRE * PC; c0 < K; c0 += PC) {
    f32x4 m[4], l[4];
    load_pass(c0, m, l);
    score_pass(c0, m, l);
  }
  __syncthreads();

  // 3. posteriors (Eq. 3): wave 0 queries, wave 1 keys; lane holds components
  //    lane + 64 j, j < KM / 64.  Hard assignment: argmax, lowest index on ties.
  if (wave < 2) {
    const float* sc = s_sc[wave];
    float v[CL];
#pragma unroll
    for (int j = 0; j < CL; ++j) v[j] = lane + 64 * j < K ? sc[lane + 64 * j] : -INFINITY;
    float m = v[0];
    int im = lane;
#pragma unroll
    for (int j = 1; j < CL; ++j) argmax_merge(m, im, v[j], lane + 64 * j);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) argmax_merge(m, im, xor_lane(m, o), xor_lane_i(im, o));
    float e[CL], esum = 0.f;
#pragma unroll
    for (int j = 0; j < CL; ++j) {
      e[j] = lane + 64 * j < K ? expf(v[j] - m) : 0.f;
      esum += e[j];
    }
    const float inv = 1.f / wave_sum(esum);
#pragma unroll
    for (int j = 0; j < CL; ++j) {
      const float gj = e[j] * inv;
      s_g[wave][lane + 64 * j] = gj;
      if (wave == 1) {
        const float zn = zc[j] + gj;
        s_z[lane + 64 * j] = zn;
        if (lane + 64 * j < K) a.sz[(size_t)bh * K + lane + 64 * j] = zn;
      }
    }
    int32_t* as = wave ? a.assign_k : a.assign_q;
    if (as && lane == 0) as[bh] = im;
  }
  __syncthreads();

  // 4. S' = S + gamma^K v^T (stored back) and this thread's part of gamma^Q^T S'
  f32x4 num = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    if (p * SR < K) {
      const int r = r0 + p * SR;             // < KM: s_g holds zeros past K
      const float gk = s_g[1][r], gq = s_g[0][r];
      const f32x4 s = st[p] + gk * vv;
      if (r < K) {
        __builtin_nontemporal_store(s, reinterpret_cast<f32x4*>(sv + (size_t)r * DV + col));
        num += gq * s;
      }
    }
  }
  if (wave == 0) {
    float d = 0.f;
#pragma unroll
    for (int j = 0; j < CL; ++j)
      d += lane + 64 * j < K ? s_g[0][lane + 64 * j] * s_z[lane + 64 * j] : 0.f;
    const float den = wave_sum(d);
    if (lane == 0) s_den = den + a.eps;
  }
  *reinterpret_cast<f32x4*>(&s_red[r0 * DV + col]) = num;
  __syncthreads();
  if (t < DV) {
    float acc = 0.f;
#pragma unroll 8
    for (int r = 0; r < SR; ++r) acc += s_red[r * DV + t];
    store1(static_cast<T*>(a.out) + (size_t)bh * DV + t, acc / s_den);
  }
}

template <class T, int DR, int KM>
hipError_t launch_dv(const DecodeArgs& a, int DV, int64_t BH, hipStream_t s) {
  const dim3 grid((unsigned)BH), block(256);
  switch (DV) {
    case 16: hipLaunchKernelGGL((gma_decode_kernel<T, DR, 16, KM>), grid, block, 0, s, a); break;
    case 32: hipLaunchKernelGGL((gma_decode_kernel<T, DR, 32, KM>), grid, block, 0, s, a); break;
    case 64: hipLaunchKernelGGL((gma_decode_kernel<T, DR, 64, KM>), grid, block, 0, s, a); break;
    case 128: hipLaunchKernelGGL((gma_decode_kernel<T, DR, 128, KM>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <class T, int KM>
hipError_t launch_dr(const DecodeArgs& a, int DR, int DV, int64_t BH, hipStream_t s) {
  switch (DR) {
    case 16: return launch_dv<T, 16, KM>(a, DV, BH, s);
    case 32: return launch_dv<T, 32, KM>(a, DV, BH, s);
    case 64: return launch_dv<T, 64, KM>(a, DV, BH, s);
    case 128: return launch_dv<T, 128, KM>(a, DV, BH, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const Plan& p, const Tensors& t, float* state_v, float* state_z,
                         hipStream_t s) {
  DecodeArgs a;
  a.q = t.q;
  a.k = t.k;
  a.v = t.v;
  a.mu = t.mu;
  a.ls2 = t.ls2;
  a.lpi = t.lpi;
  a.sv = state_v;
  a.sz = state_z;
  a.out = t.out;
  a.assign_q = t.assign_q;
  a.assign_k = t.assign_k;
  a.H = (int)p.H;
  a.K = p.K;
  a.eps = t.eps;
  if (g_launch_hook) g_launch_hook("gma_decode", s, 1);
  // the component count bounds the LDS arrays and the passes: 128 or 256
  const bool wide = p.K > 128;
  const hipError_t e = p.out_bf ? (wide ? launch_dr<bf16, 256>(a, p.DR, p.DV, p.BH, s)
                                        : launch_dr<bf16, 128>(a, p.DR, p.DV, p.BH, s))
                                : (wide ? launch_dr<float, 256>(a, p.DR, p.DV, p.BH, s)
                                        : launch_dr<float, 128>(a, p.DR, p.DV, p.BH, s));
  if (g_launch_hook) g_launch_hook("gma_decode", s, 0);
  return e;
}

}  // namespace gma
