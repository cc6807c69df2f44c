// Device-side building blocks for the gfx950 GMA kernels.
//
// Notation follows "Gaussian Mixture Attention: Linear-Time Sequence Mixing via
// Probabilistic Latent Routing": K components, routing dimension d_r, value
// dimension d_v, responsibilities gamma (Eq. 3), latent memory V~ and
// normaliser Z (Eqs. 5-6), read-out O (Eq. 7).
//
// MFMA shapes used (CDNA4 / gfx950):
//   v_mfma_f32_16x16x32_bf16  A 16x32, B 32x16, D 16x16 fp32
//   v_mfma_f32_16x16x4_f32    A 16x4,  B 4x16,  D 16x16 fp32
// Operand registers: lane l holds row/column (l % 16) of A/B and contraction
// indices g*E .. g*E+E-1 of one "chunk" (g = l / 16, E = 8 bf16 or 4 fp32,
// i.e. 16 bytes per lane).  A bf16 chunk is one MFMA; an fp32 chunk is four
// k=4 MFMAs that pair element e of A with element e of B.  Either way a chunk
// contracts CS = 4*E indices and needs one 16-byte load per operand.
// D layout: lane l holds column (l % 16), rows 4*(l/16) + i, i = 0..3.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace gma {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 64;        // tokens per workgroup tile (four 16-token MFMA tiles)
constexpr int kWaves = 4;        // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr double kLog2eD = 1.44269504088896340736;

// Token permutation inside a 64-token tile.  MFMA tile gt (0..3), row r = 4g+i
// maps to token 32*(gt/2) + 8g + 4*(gt%2) + i.  With it, the four rows a lane
// holds in D layout are consecutive tokens, and the union over a pair of
// tiles (2p, 2p+1) gives lane group g the eight consecutive tokens
// 32p + 8g .. 32p + 8g + 7 -- exactly one bf16 operand chunk when the token
// index is the contraction index.
__host__ __device__ constexpr int tile_token(int gt, int r) {
  return 32 * (gt >> 1) + 8 * (r >> 2) + 4 * (gt & 1) + (r & 3);
}

template <bool BF> struct Prec;
template <> struct Prec<true> {        // bf16 storage, split-bf16 MFMA arithmetic
  using in_t = bf16;
  using op_t = bf16;
  using chunk_t = bf16x8;
  static constexpr int E = 8;
  static constexpr int CS = 32;
  static constexpr int NARR = 4;       // A_hi, A_lo, B_hi, B_lo
};
template <> struct Prec<false> {       // fp32 storage, fp32 MFMA arithmetic
  using in_t = float;
  using op_t = float;
  using chunk_t = f32x4;
  static constexpr int E = 4;
  static constexpr int CS = 16;
  static constexpr int NARR = 2;       // A, B
};

__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(f32x4 a, f32x4 b, f32x4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
  return c;
}

template <class T>
__device__ __forceinline__ T ld16(const void* p) {
  return *reinterpret_cast<const T*>(__builtin_assume_aligned(p, 16));
}
template <class T>
__device__ __forceinline__ void st16(void* p, T v) {
  *reinterpret_cast<T*>(__builtin_assume_aligned(p, 16)) = v;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
// Hardware reciprocal (v_rcp_f32, about 1 ulp); the normalisers it inverts are
// positive sums well inside the normal range.
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// ---- cross-lane reductions ------------------------------------------------
// (The patterns used -- quad permutes and row mirrors -- read valid lanes
// only, so bound_ctrl is immaterial; with it set the compiler can fold the
// move into the consuming ALU instruction.)
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true);
}
// Butterfly over the 16 lanes of a DPP row; every lane receives the result
// (each step pairs lanes symmetrically, so all lanes compute identical values).
#define GMA_ROW16(OP, v)            \
  v = OP(v, dpp<0xB1>(v));          \
  v = OP(v, dpp<0x4E>(v));          \
  v = OP(v, dpp<0x141>(v));         \
  v = OP(v, dpp<0x140>(v));

__device__ __forceinline__ float add_f(float a, float b) { return a + b; }
__device__ __forceinline__ float max_f(float a, float b) { return fmaxf(a, b); }

__device__ __forceinline__ float row16_max(float v) { GMA_ROW16(max_f, v) return v; }
__device__ __forceinline__ float row16_sum(float v) { GMA_ROW16(add_f, v) return v; }

// Exchange with lane ^ mask (any mask < 64) through the LDS crossbar.
__device__ __forceinline__ float xor_lane(float v, int mask) {
  int src = (int)(threadIdx.x & 63) ^ mask;
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(v)));
}
__device__ __forceinline__ int xor_lane_i(int v, int mask) {
  int src = (int)(threadIdx.x & 63) ^ mask;
  return __builtin_amdgcn_ds_bpermute(src << 2, v);
}
// The reparameterisations used for training ("Learning", Eqs. 14-15): the log
// variance from its unconstrained parameter, log(log(1 + exp(w)) + eps_sigma)
// with the softplus as max(w, 0) + log1p(exp(-|w|)), and the log-normaliser
// of a head's K prior logits (one wave: lane-strided max and sum, then a
// butterfly over the 64 lanes; every lane returns it).  Shared by the
// reparameterisation kernel and the prologue, so both give the same bits.
__device__ __forceinline__ float reparam_log_var(float w, float eps_sigma) {
  const float sp = fmaxf(w, 0.f) + log1pf(expf(-fabsf(w)));
  return logf(sp + eps_sigma);
}
__device__ __forceinline__ float xor_lane(float v, int mask);
__device__ __forceinline__ float wave_log_norm(const float* __restrict__ a, int K) {
  const int lane = threadIdx.x & 63;
  float m = -INFINITY;
  for (int k = lane; k < K; k += 64) m = fmaxf(m, a[k]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, xor_lane(m, o));
  float s = 0.f;
  for (int k = lane; k < K; k += 64) s += expf(a[k] - m);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += xor_lane(s, o);
  return m + logf(s);
}

// Exchanges between the four lane groups g (16-lane rows) without the LDS
// crossbar: v_permlane16_swap with both operands = v returns, in every lane,
// the pair {v of the even row, v of the odd row} of its row pair (lanes l and
// l ^ 16); v_permlane32_swap does the same for the two halves (l and l ^ 32).
// Either order of the pair gives bitwise the same max / sum in both lanes.
__device__ __forceinline__ void pair_xor16(float v, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void pair_xor32(float v, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void pair_xor16_i(int v, int& a, int& b) {
  const auto r = __builtin_amdgcn_permlane16_swap((unsigned)v, (unsigned)v, false, false);
  a = (int)r[0];
  b = (int)r[1];
}
__device__ __forceinline__ void pair_xor32_i(int v, int& a, int& b) {
  const auto r = __builtin_amdgcn_permlane32_swap((unsigned)v, (unsigned)v, false, false);
  a = (int)r[0];
  b = (int)r[1];
}
// Reductions over the four lane groups g (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float groups_max(float v) {
  float a, b;
  pair_xor16(v, a, b);
  pair_xor32(fmaxf(a, b), a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float groups_sum(float v) {
  float a, b;
  pair_xor16(v, a, b);
  pair_xor32(a + b, a, b);
  return a + b;
}
__device__ __forceinline__ int groups_min_i(int v) {
  int a, b;
  pair_xor16_i(v, a, b);
  pair_xor32_i(min(a, b), a, b);
  return min(a, b);
}

// (value, index) argmax merge, ties to the lower index.
__device__ __forceinline__ void argmax_merge(float& v, int& i, float v2, int i2) {
  bool take = (v2 > v) || (v2 == v && i2 < i);
  v = take ? v2 : v;
  i = take ? i2 : i;
}
__device__ __forceinline__ void row16_argmax(float& v, int& i) {
  argmax_merge(v, i, dpp<0xB1>(v), dpp_i<0xB1>(i));
  argmax_merge(v, i, dpp<0x4E>(v), dpp_i<0x4E>(i));
  argmax_merge(v, i, dpp<0x141>(v), dpp_i<0x141>(i));
  argmax_merge(v, i, dpp<0x140>(v), dpp_i<0x140>(i));
}
__device__ __forceinline__ void groups_argmax(float& v, int& i) {
  float a, b;
  int ia, ib;
  pair_xor16(v, a, b);
  pair_xor16_i(i, ia, ib);
  argmax_merge(a, ia, b, ib);
  pair_xor32(a, v, b);
  pair_xor32_i(ia, i, ib);
  argmax_merge(v, i, b, ib);
}

// ---- conversions -----------------------------------------------------------
__device__ __forceinline__ bf16 to_bf16(float x) { return (bf16)x; }   // RNE
__device__ __forceinline__ float from_bf16(bf16 x) { return (float)x; }

// Split an fp32 value into bf16 hi + lo with hi + lo == x to 16 significant bits
// (exact when x has at most 16 significant bits, e.g. the square of a bf16).
__device__ __forceinline__ void split_bf16(float x, bf16& hi, bf16& lo) {
  hi = (bf16)x;
  lo = (bf16)(x - (float)hi);
}

template <class T> __device__ __forceinline__ T load_elem(const T* p) { return *p; }

// Wait until at most N vector memory operations of this wave are outstanding
// (they complete in issue order, so everything issued before the last N has).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt takes 0..63");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier that orders LDS only: outstanding global loads (prefetch of
// the next tile) stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ds_read_b64_tr_b16: within each 16-lane group, source lane s = a + 4m
// supplies an 8-byte block; destination lane 4a + e receives element e of the
// blocks of source lanes a, a+4, a+8, a+12 (in that order).
typedef short short4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ short4_t lds_read_tr16(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) short4_t*)(p));
}

// MFMA operand chunk from a row-major LDS matrix M[token][col] (bf16, row
// stride ld elements, multiple of 4): lane (l % 16, g) receives the eight
// tokens tok0 + 8g .. tok0 + 8g + 7 of column col0 + (l % 16), i.e. the
// contraction runs over tokens.  Two transpose reads.
__device__ __forceinline__ bf16x8 tr_chunk(const bf16* M, int ld, int tok0, int col0) {
  const int lane = threadIdx.x & 63, s = lane & 15, g = lane >> 4;
  const bf16* p = M + (tok0 + 8 * g + (s >> 2)) * ld + col0 + 4 * (s & 3);
  const short4_t lo = lds_read_tr16(p);
  const short4_t hi = lds_read_tr16(p + 4 * ld);
  typedef short short8_t __attribute__((ext_vector_type(8)));
  const short8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// Row offset of token row r in a row-major [token][column] bf16 tile read by
// tr_chunk_g: a bank skew of 16 B for bit 3 and 8 B for bit 4 of r keeps both
// the 8-byte stores of 16 rows tile_token(gt, 0..15) and the transpose reads
// of 4 consecutive rows conflict-free (row stride ld must be 16 mod 32 elements).
__device__ __forceinline__ int gtr_row(int r, int ld) {
  return r * ld + 8 * ((r >> 3) & 1) + 4 * ((r >> 4) & 1);
}
__device__ __forceinline__ bf16x8 tr_chunk_g(const bf16* M, int ld, int tok0, int col0) {
  const int lane = threadIdx.x & 63, s = lane & 15, g = lane >> 4;
  const int row = tok0 + 8 * g + (s >> 2), col = col0 + 4 * (s & 3);
  const short4_t lo = lds_read_tr16(M + gtr_row(row, ld) + col);
  const short4_t hi = lds_read_tr16(M + gtr_row(row + 4, ld) + col);
  typedef short short8_t __attribute__((ext_vector_type(8)));
  const short8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// Swizzled row-major tile: ROWCH 16-byte chunks per row, logical chunk j of
// row r stored at physical chunk j ^ swz(r), swz(r) = 2r mod ROWCH (even, so
// the two 8-byte halves a transpose read touches stay together and the four
// rows of one read land on distinct banks).  Unpadded, so a wave can fill it
// with 1 KB direct global-to-LDS loads.
template <int ROWCH>
__device__ __forceinline__ int swz_elem(int row, int col) {
  constexpr int mask = ROWCH >= 2 ? ROWCH - 2 : 0;
  return row * ROWCH * 8 + ((((col >> 3) ^ ((2 * row) & mask))) << 3) + (col & 7);
}
template <int ROWCH>
__device__ __forceinline__ bf16x8 tr_chunk_swz(const bf16* M, int tok0, int col0) {
  const int lane = threadIdx.x & 63, s = lane & 15, g = lane >> 4;
  const int row = tok0 + 8 * g + (s >> 2), col = col0 + 4 * (s & 3);
  const short4_t lo = lds_read_tr16(M + swz_elem<ROWCH>(row, col));
  const short4_t hi = lds_read_tr16(M + swz_elem<ROWCH>(row + 4, col));
  typedef short short8_t __attribute__((ext_vector_type(8)));
  const short8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// Direct global -> LDS copy of 16 bytes per lane: lane l's bytes land at
// lds_base + 16*l (lds_base must be the same for the whole wave).
__device__ __forceinline__ void global_to_lds16(const void* gsrc, void* lds_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (__attribute__((address_space(3))) void*)(lds_base), 16, 0, 0);
}
// The same for data read once per call (streamed keys and values): the
// non-temporal cache policy (aux bit 1).
__device__ __forceinline__ void global_to_lds16_nt(const void* gsrc, void* lds_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (__attribute__((address_space(3))) void*)(lds_base), 16, 0, 2);
}
// 16-byte loads and stores of streamed data with the non-temporal policy.
template <class T>
__device__ __forceinline__ T ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const T*>(__builtin_assume_aligned(p, 16)));
}
template <class T>
__device__ __forceinline__ void st16_nt(void* p, T v) {
  __builtin_nontemporal_store(v, reinterpret_cast<T*>(__builtin_assume_aligned(p, 16)));
}
__device__ __forceinline__ void wait_global_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Raw buffer resource over [base, base + bytes) (bytes < 2^31): a load whose
// byte offset reaches past the end returns zeros (and a copy to LDS writes
// zeros), so tails need no clamping.  Offsets are 32-bit per lane, the base and
// size live in scalar registers.
typedef __amdgpu_buffer_rsrc_t buf_rsrc;
__device__ __forceinline__ buf_rsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
// 16-byte load of streamed data (non-temporal policy).
template <class T>
__device__ __forceinline__ T buf_ld16_nt(buf_rsrc rs, uint32_t off) {
  return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 2));
}
// 16 bytes per lane straight into LDS: lane l's bytes land at lds_base + 16 l.
__device__ __forceinline__ void buf_to_lds16_nt(buf_rsrc rs, uint32_t off, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rs, (__attribute__((address_space(3))) void*)(lds_base), 16, off, 0, 0, 2);
}

}  // namespace gma
