// C ABI of the GMA library: validation, planning, workspace layout, launch
// sequencing, status strings and the kernel-timing facility.  See include/gma.h.
#include <math.h>
#include <string.h>

#include <mutex>

#include <string>
#include <vector>

#include "gma.h"
#include "gma_internal.h"
#include "gma_tiles.h"

namespace gma {

thread_local launch_hook_t g_launch_hook = nullptr;

namespace {

thread_local std::string t_err;

int fail(int status, const std::string& msg) {
  t_err = msg;
  return status;
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

bool supported_dim(int v) { return v == 16 || v == 32 || v == 64 || v == 128; }

int check_dims(const gma_dims* d, float eps, int causal) {
  if (!d) return fail(GMA_ERR_INVALID_ARG, "dims is NULL");
  if (d->B < 1 || d->H < 1 || d->N < 1) return fail(GMA_ERR_INVALID_ARG, "B, H and N must be >= 1");
  if (d->d_r < 1 || d->d_v < 1 || d->K < 1)
    return fail(GMA_ERR_INVALID_ARG, "d_r, d_v and K must be >= 1");
  if (d->dtype != GMA_F32 && d->dtype != GMA_BF16) return fail(GMA_ERR_INVALID_ARG, "unknown dtype");
  if (d->chunk < 0) return fail(GMA_ERR_INVALID_ARG, "chunk must be >= 0");
  if (causal != 0 && causal != 1) return fail(GMA_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (!(eps >= 0.f) || !isfinite(eps)) return fail(GMA_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (!supported_dim(d->d_r)) return fail(GMA_ERR_UNSUPPORTED, "d_r must be 16, 32, 64 or 128");
  if (!supported_dim(d->d_v)) return fail(GMA_ERR_UNSUPPORTED, "d_v must be 16, 32, 64 or 128");
  if (d->K > 256) return fail(GMA_ERR_UNSUPPORTED, "K above 256 is not supported");
  if (d->chunk != 0 && d->chunk != 64) return fail(GMA_ERR_UNSUPPORTED, "chunk must be 0 or 64");
  const int64_t lim = (int64_t)1 << 40;
  if (d->B > lim / d->H) return fail(GMA_ERR_UNSUPPORTED, "B*H too large");
  const int64_t BH = d->B * d->H;
  if (BH > 65535) return fail(GMA_ERR_UNSUPPORTED, "B*H above 65535 is not supported");
  if (d->N > lim / (BH * 128)) return fail(GMA_ERR_UNSUPPORTED, "B*H*N*d too large");
  return GMA_OK;
}

int make_plan(const gma_dims* d, int causal, bool fp32_compute, Plan& p);

// The bidirectional plan at N rounded up to the 64-token chunk, on which the
// causal product path runs; its chunk products are batched over B*H*N/64.
int prod_plan(const gma_dims* d, bool fp32_compute, Plan& pp) {
  gma_dims dp = *d;
  dp.N = (d->N + 63) / 64 * 64;
  int st = make_plan(&dp, 0, fp32_compute, pp);
  if (st != GMA_OK) return st;
  if (pp.BH * (dp.N / 64) > 65535)
    return fail(GMA_ERR_UNSUPPORTED,
                "causal product path: B*H*ceil(N/64) must be at most 65535 for this K, d_r, d_v");
  return GMA_OK;
}

int make_plan(const gma_dims* d, int causal, bool fp32_compute, Plan& p) {
  int st = check_dims(d, 0.f, causal);
  if (st != GMA_OK) return st;
  p = Plan{};
  p.bf = !fp32_compute && d->dtype == GMA_BF16;
  p.out_bf = d->dtype == GMA_BF16;
  p.B = d->B;
  p.H = d->H;
  p.N = d->N;
  p.BH = d->B * d->H;
  p.DR = d->d_r;
  p.DV = d->d_v;
  p.K = d->K;
  int ct = (d->K + 15) / 16, ct2 = 1;
  while (ct2 < ct) ct2 *= 2;
  p.CT = ct2;
  switch (p.CT) {
    case 1: p.CPW = 1; p.NG = 1; break;
    case 2: p.CPW = 2; p.NG = 1; break;
    case 4: p.CPW = 2; p.NG = 2; break;
    case 8: p.CPW = 2; p.NG = 4; break;
    default: p.CPW = 4; p.NG = 4; break;        // 16 tiles: K up to 256
  }
  if (causal) {
    // the scan kernel needs four component groups: K padded to at least 64
    if (p.CT < 4) p.CT = 4;
    p.CPW = p.CT / 4;
    p.NG = 4;
  }
  p.Kp = 16 * p.CT;
  const int cs = p.bf ? 32 : 16;
  p.DRP = p.DR < cs ? cs : p.DR;
  p.TG = 4 / p.NG;
  p.khalf = causal ? causal_khalf(p.bf, p.DRP, p.DV, p.Kp) : bidir_khalf(p.bf, p.DRP, p.DV, p.Kp);
  if (causal && !p.khalf && causal_lds_bytes(p.bf, p.DR, p.DV, p.Kp) > kMaxLds) {
    // the scan kernel's tiles do not fit in LDS: the causal forward runs as a
    // chain of products over stored responsibilities, on the bidirectional
    // plan at the length rounded up to the 64-token chunk
    Plan pp;
    int st2 = prod_plan(d, fp32_compute, pp);
    if (st2 != GMA_OK) return st2;
    p.prod = true;
    p.total = prod_forward_workspace_bytes(pp, true, d->N);
    return GMA_OK;
  }
  p.tiles = (p.N + 63) / 64;
  // About two workgroups per compute unit (256 CUs) for each streaming kernel.
  int64_t want = (512 + p.BH - 1) / p.BH;
  if (want < 1) want = 1;
  if (want > p.tiles) want = p.tiles;
  p.tiles_per_split = (int)((p.tiles + want - 1) / want);
  p.S = (int)((p.tiles + p.tiles_per_split - 1) / p.tiles_per_split);
  // causal spans: a span is the unit one workgroup scans sequentially.  The
  // bf16 scan kernel holds two 4-wave workgroups per compute unit when its LDS
  // allows (else one): as many spans as fit the chip at once, so every
  // workgroup scans in the same round; otherwise about four per compute unit.
  {
    int64_t want_c = (1024 + p.BH - 1) / p.BH;
    const int lds2 = causal2_lds_bytes(p.bf, p.DRP, p.DV, p.khalf ? p.Kp / 2 : p.Kp);
    if (lds2 > 0) {
      const int64_t resident = 256 * (2 * lds2 <= kMaxLds ? 2 : 1);
      want_c = resident / p.BH;
    }
    if (want_c < 1) want_c = 1;
    if (want_c > p.tiles) want_c = p.tiles;
    p.span_tiles = (int)((p.tiles + want_c - 1) / want_c);
    p.nspan = (int)((p.tiles + p.span_tiles - 1) / p.span_tiles);
  }
  // per head: the coefficient arrays and c, then (bf16) the same values in
  // MFMA-operand order for the token-owner read-out
  p.head_bytes = 2 * round256((size_t)8 * p.Kp * p.DRP + (size_t)4 * p.Kp);
  size_t off = 0;
  p.off_params = off;
  off += round256(p.head_bytes * (size_t)p.H);
  if (!causal) {
    const size_t PS = (size_t)p.S * p.TG;
    p.off_partial = off;
    off += round256((size_t)p.BH * PS * p.Kp * p.DV * 4);
    p.off_partial_z = off;
    off += round256((size_t)p.BH * PS * p.Kp * 4);
    p.off_vt = off;
    off += round256((size_t)p.BH * p.Kp * p.DV * 4);
    p.off_z = off;
    off += round256((size_t)p.BH * p.Kp * 4);
    // V~^T and (Z_hi, Z_lo, 1) as bf16 MFMA operands: (d_v/16 + 1) blocks x K_pad/32
    // steps x 1 KB per sequence
    p.off_vtab = off;
    off += round256((size_t)p.BH * (p.DV / 16 + 1) * ((p.Kp + 31) / 32) * 1024);
    if (p.khalf) {
      // the first half's numerators and (denominator, maximum, best score,
      // its component) per query
      p.off_qpart = off;
      off += round256((size_t)p.BH * p.N * p.DV * 4);
      p.off_qpart2 = off;
      off += round256((size_t)p.BH * p.N * 16);
    }
  } else {
    const size_t ns = (size_t)p.nspan;
    p.off_state = off;
    off += round256((size_t)p.BH * ns * p.Kp * p.DV * 4);
    p.off_state_z = off;
    off += round256((size_t)p.BH * ns * p.Kp * 4);
    p.off_carry = off;
    off += round256((size_t)p.BH * ns * p.Kp * p.DV * 4);
    p.off_carry_z = off;
    off += round256((size_t)p.BH * ns * p.Kp * 4);
    if (p.bf && (causal2_lds_bytes(true, p.DRP, p.DV, p.Kp) > 0 || p.khalf)) {
      // the keys' responsibilities from the span-totals pass for the
      // token-owner scan: Gamma^K^T per 64-key chunk, [Kp][64] bf16
      p.off_gt = off;
      off += round256((size_t)p.BH * p.tiles * p.Kp * 64 * 2);
    }
    if (p.khalf) {
      // per query the first half's numerator [d_v] and (denominator, maximum,
      // best score, its component)
      p.off_qpart = off;
      off += round256((size_t)p.BH * p.N * p.DV * 4);
      p.off_qpart2 = off;
      off += round256((size_t)p.BH * p.N * 16);
    }
  }
  p.total = off;
  return GMA_OK;
}

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15) == 0; }

// ---- timing ----------------------------------------------------------------
// Per calling thread: each thread that enables timing records and collects
// only the launches it makes itself.
struct Pending {
  const char* tag = nullptr;
  hipEvent_t start = nullptr, stop = nullptr;
  hipError_t err = hipSuccess;      // the first failure creating or recording this pair
};
struct Total {
  std::string name;
  int64_t launches;
  double ms;
};
struct TimingState {
  std::vector<Pending> pending;
  Pending open{};
};
thread_local TimingState t_timing;

void timing_hook(const char* tag, hipStream_t s, int begin) {
  TimingState& ts = t_timing;
  if (begin) {
    ts.open = Pending{};
    ts.open.tag = tag;
    hipError_t e = hipEventCreate(&ts.open.start);
    if (e == hipSuccess) e = hipEventCreate(&ts.open.stop);
    if (e == hipSuccess) e = hipEventRecord(ts.open.start, s);
    ts.open.err = e;
  } else {
    if (ts.open.err == hipSuccess) ts.open.err = hipEventRecord(ts.open.stop, s);
    ts.pending.push_back(ts.open);
  }
}

int finish_launch(hipError_t e, const char* what) {
  if (e != hipSuccess)
    return fail(GMA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  if (getenv("GMA_SYNC_DEBUG")) {
    e = hipDeviceSynchronize();
    if (e != hipSuccess)
      return fail(GMA_ERR_HIP, std::string(what) + " (synchronised): " + hipGetErrorString(e));
  }
  return GMA_OK;
}

}  // namespace
}  // namespace gma

using namespace gma;

extern "C" {

int gma_validate(const gma_dims* d, float eps, int causal, const void* const* ptrs, int nptrs,
                 size_t workspace_bytes, size_t workspace_needed) {
  t_err.clear();
  int st = check_dims(d, eps, causal);
  if (st != GMA_OK) return st;
  Plan p;
  st = make_plan(d, causal, false, p);
  if (st != GMA_OK) return st;
  if (nptrs < 0 || (nptrs > 0 && !ptrs))
    return fail(GMA_ERR_INVALID_ARG, "pointer list is NULL or nptrs is negative");
  for (int i = 0; i < nptrs; ++i) {
    if (!ptrs[i]) return fail(GMA_ERR_INVALID_ARG, "pointer " + std::to_string(i) + " is NULL");
    if (!aligned16(ptrs[i]))
      return fail(GMA_ERR_INVALID_ARG, "pointer " + std::to_string(i) + " is not 16-byte aligned");
  }
  if (workspace_bytes < workspace_needed) return fail(GMA_ERR_WORKSPACE, "workspace too small");
  return GMA_OK;
}

int gma_forward_workspace_bytes(const gma_dims* d, int causal, size_t* bytes) {
  t_err.clear();
  if (!bytes) return fail(GMA_ERR_INVALID_ARG, "bytes is NULL");
  Plan p;
  int st = make_plan(d, causal, false, p);
  if (st != GMA_OK) return st;
  *bytes = p.total;
  return GMA_OK;
}

static int forward_impl(const Plan& p, const Tensors& t, int causal, hipStream_t s,
                        const gma_dims* d, bool fp32_compute) {
  if (p.prod) {
    Plan pp;
    int st = prod_plan(d, fp32_compute, pp);
    if (st != GMA_OK) return st;
    return finish_launch(launch_prod_forward(pp, t, true, p.N, p.out_bf, s),
                         "causal product-path launch");
  }
  hipError_t e = launch_prologue(p, t, s);
  if (e != hipSuccess) return finish_launch(e, "prologue launch");
  e = causal ? launch_causal(p, t, s) : launch_bidir(p, t, s);
  return finish_launch(e, causal ? "causal launch" : "bidirectional launch");
}

int gma_forward(const void* Q_X, const void* K_X, const void* V_X, const float* mu,
                const float* log_sigma2, const float* log_pi, float eps, int causal, void* out,
                const gma_dims* d, int32_t* assign_q, int32_t* assign_k, void* workspace,
                size_t workspace_bytes, void* stream) {
  t_err.clear();
  int st = check_dims(d, eps, causal);
  if (st != GMA_OK) return st;
  if (!Q_X || !K_X || !V_X || !mu || !log_sigma2 || !log_pi || !out || !workspace)
    return fail(GMA_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(Q_X) || !aligned16(K_X) || !aligned16(V_X) || !aligned16(out) ||
      !aligned16(workspace) || !aligned16(mu) || !aligned16(log_sigma2) ||
      ((uintptr_t)log_pi & 3) || ((uintptr_t)assign_q & 3) || ((uintptr_t)assign_k & 3))
    return fail(GMA_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  Plan p;
  st = make_plan(d, causal, false, p);
  if (st != GMA_OK) return st;
  if (workspace_bytes < p.total) return fail(GMA_ERR_WORKSPACE, "workspace too small");
  Tensors t;
  t.q = Q_X;
  t.k = K_X;
  t.v = V_X;
  t.mu = mu;
  t.ls2 = log_sigma2;
  t.lpi = log_pi;
  t.out = out;
  t.assign_q = assign_q;
  t.assign_k = assign_k;
  t.eps = eps;
  t.ws = static_cast<char*>(workspace);
  return forward_impl(p, t, causal, static_cast<hipStream_t>(stream), d, false);
}

int gma_forward_reparam(const void* Q_X, const void* K_X, const void* V_X, const float* mu,
                        const float* omega, const float* alpha, float eps_sigma, float eps,
                        int causal, void* out, const gma_dims* d, int32_t* assign_q,
                        int32_t* assign_k, void* workspace, size_t workspace_bytes,
                        void* stream) {
  t_err.clear();
  int st = check_dims(d, eps, causal);
  if (st != GMA_OK) return st;
  if (!(eps_sigma > 0.f) || !isfinite(eps_sigma))
    return fail(GMA_ERR_INVALID_ARG, "eps_sigma must be finite and > 0");
  if (!Q_X || !K_X || !V_X || !mu || !omega || !alpha || !out || !workspace)
    return fail(GMA_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(Q_X) || !aligned16(K_X) || !aligned16(V_X) || !aligned16(out) ||
      !aligned16(workspace) || !aligned16(mu) || ((uintptr_t)omega & 3) ||
      ((uintptr_t)alpha & 3) || ((uintptr_t)assign_q & 3) || ((uintptr_t)assign_k & 3))
    return fail(GMA_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned (omega, alpha: 4)");
  Plan p;
  st = make_plan(d, causal, false, p);
  if (st != GMA_OK) return st;
  if (workspace_bytes < p.total) return fail(GMA_ERR_WORKSPACE, "workspace too small");
  Tensors t;
  t.q = Q_X;
  t.k = K_X;
  t.v = V_X;
  t.mu = mu;
  t.omega = omega;
  t.alpha = alpha;
  t.eps_sigma = eps_sigma;
  t.out = out;
  t.assign_q = assign_q;
  t.assign_k = assign_k;
  t.eps = eps;
  t.ws = static_cast<char*>(workspace);
  return forward_impl(p, t, causal, static_cast<hipStream_t>(stream), d, false);
}

// ---- the workspace of gma_forward_noalloc ------------------------------------
// A file-scope device array: each GPU the library runs on holds its own copy.
// In host code `scratch` is only a host-side stand-in for the symbol; its
// device address (per device) comes from hipGetSymbolAddress and is the only
// form ever passed to a kernel.
static __device__ __attribute__((aligned(256))) char scratch[GMA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`, looked up once per device (with
// that device current) and kept.
int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(GMA_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(GMA_ERR_UNSUPPORTED, "device index above 63");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(GMA_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return GMA_OK;
}
}  // namespace

int gma_forward_noalloc(const void* Q_X, const void* K_X, const void* V_X, const float* mu,
                        const float* log_sigma2, const float* log_pi, float eps, int causal,
                        void* out, const gma_dims* d, int32_t* assign_q, int32_t* assign_k,
                        void* stream) {
  t_err.clear();
  int st = check_dims(d, eps, causal);
  if (st != GMA_OK) return st;
  if (!Q_X || !K_X || !V_X || !mu || !log_sigma2 || !log_pi || !out)
    return fail(GMA_ERR_INVALID_ARG, "a required pointer is NULL");
  Plan p;
  st = make_plan(d, causal, false, p);
  if (st != GMA_OK) return st;
  if (p.total > GMA_NOALLOC_SCRATCH_BYTES)
    return fail(GMA_ERR_UNSUPPORTED, "this shape needs " + std::to_string(p.total) +
                                         " bytes of workspace, above the " +
                                         std::to_string((size_t)GMA_NOALLOC_SCRATCH_BYTES) +
                                         " of the static scratch array");
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != GMA_OK) return st;
  return gma_forward(Q_X, K_X, V_X, mu, log_sigma2, log_pi, eps, causal, out, d, assign_q,
                     assign_k, ws, GMA_NOALLOC_SCRATCH_BYTES, stream);
}

// The layer's plan and where its projections sit.  Fused (bf16, d_r = 64, at
// most 64 components, the scan kernel's shapes; either variant): the
// projection epilogue forms the routing responsibilities and Q_X, K_X are
// never stored; V_X is kept in bf16.  Otherwise, where the bf16 kernels take
// split routing vectors for this shape, the projection epilogue writes Q_X and
// K_X as bf16 pairs (16 significant bits) and V_X in bf16, and the bf16 GMA
// kernels run on them; else the projections stay fp32 and feed the fp32 GMA
// path.
struct LayerPlan {
  Plan p;
  int split = 0;
  int fused = 0;
  int kc = 0;                        // fused: components formed (32 or 64)
  size_t gma_bytes = 0;
  size_t off[5] = {0, 0, 0, 0, 0};   // from the start of the workspace
  size_t off_eq = 0;                 // fused: the queries' exponentials
  size_t off_vtab = 0;               // fused, bidirectional: the state's operand table
  size_t total = 0;
};

static int layer_plan(const gma_dims* d, int32_t d_model, int causal, LayerPlan& L) {
  if (d->dtype != GMA_BF16) return fail(GMA_ERR_UNSUPPORTED, "the projection layer takes bf16 X and W");
  if (d_model < 64 || d_model > 8192 || d_model % 64)
    return fail(GMA_ERR_UNSUPPORTED, "d_model must be a multiple of 64 in 64..8192");
  // the fused form runs on the causal plan (K_pad 64, spans) in both variants
  int st = make_plan(d, 1, false, L.p);
  L.fused = st == GMA_OK && layer_fused_ok(L.p);
  L.kc = L.p.K <= 32 ? 32 : 64;
  if (!L.fused) st = make_plan(d, causal, false, L.p);
  L.split = !L.fused && st == GMA_OK && !L.p.prod &&
            (causal ? causal_split_ok(L.p) : bidir_split_ok(L.p));
  if (!L.split && !L.fused) {
    st = make_plan(d, causal, true, L.p);
    if (st != GMA_OK) return st;
  }
  t_err.clear();
  const Plan& p = L.p;
  L.gma_bytes = round256(p.total);
  size_t off = L.gma_bytes;
  const size_t nr = (size_t)p.BH * p.N * p.DR, nv = (size_t)p.BH * p.N * p.DV;
  if (L.fused) {
    L.off[4] = off;
    off += round256(2 * nv);
    L.off_eq = off;
    off += round256((size_t)p.BH * p.N * L.kc * 2);
    L.off_vtab = off;
    off += round256((size_t)p.BH * (p.DV / 16 + 1) * (p.Kp / 32) * 1024);
  } else if (L.split) {
    for (int m = 0; m < 4; ++m) {
      L.off[m] = off;
      off += round256(2 * nr);
    }
    L.off[4] = off;
    off += round256(2 * nv);
  } else {
    L.off[0] = off;
    L.off[1] = off + 4 * nr;
    L.off[2] = off + 8 * nr;
    off += round256(4 * (2 * nr + nv));
  }
  L.total = off;
  return GMA_OK;
}

int gma_layer_workspace_bytes(const gma_dims* d, int32_t d_model, int causal, size_t* bytes) {
  t_err.clear();
  if (!bytes) return fail(GMA_ERR_INVALID_ARG, "bytes is NULL");
  int st = check_dims(d, 0.f, causal);
  if (st != GMA_OK) return st;
  LayerPlan L;
  st = layer_plan(d, d_model, causal, L);
  if (st != GMA_OK) return st;
  *bytes = L.total;
  return GMA_OK;
}

int gma_layer_projection_layout(const gma_dims* d, int32_t d_model, int causal, int32_t* format,
                                size_t offsets[5]) {
  t_err.clear();
  if (!format || !offsets) return fail(GMA_ERR_INVALID_ARG, "format or offsets is NULL");
  int st = check_dims(d, 0.f, causal);
  if (st != GMA_OK) return st;
  LayerPlan L;
  st = layer_plan(d, d_model, causal, L);
  if (st != GMA_OK) return st;
  *format = L.fused ? GMA_PROJ_FUSED_BF16 : (L.split ? GMA_PROJ_SPLIT_BF16 : GMA_PROJ_F32);
  for (int m = 0; m < 5; ++m) offsets[m] = L.off[m];
  return GMA_OK;
}

int gma_layer_forward(const void* X, const void* W_Q, const void* W_K, const void* W_V,
                      int32_t d_model, const float* mu, const float* log_sigma2,
                      const float* log_pi, float eps, int causal, void* out, const gma_dims* d,
                      int32_t* assign_q, int32_t* assign_k, void* workspace,
                      size_t workspace_bytes, void* stream) {
  t_err.clear();
  int st = check_dims(d, eps, causal);
  if (st != GMA_OK) return st;
  if (!X || !W_Q || !W_K || !W_V || !mu || !log_sigma2 || !log_pi || !out || !workspace)
    return fail(GMA_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(X) || !aligned16(W_Q) || !aligned16(W_K) || !aligned16(W_V) || !aligned16(out) ||
      !aligned16(workspace) || !aligned16(mu) || !aligned16(log_sigma2) ||
      ((uintptr_t)log_pi & 3) || ((uintptr_t)assign_q & 3) || ((uintptr_t)assign_k & 3))
    return fail(GMA_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  LayerPlan L;
  st = layer_plan(d, d_model, causal, L);
  if (st != GMA_OK) return st;
  const Plan& p = L.p;
  if (workspace_bytes < L.total) return fail(GMA_ERR_WORKSPACE, "workspace too small");
  char* ws = static_cast<char*>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const void* const W[3] = {W_Q, W_K, W_V};
  void* P[3];
  void* lo[2] = {nullptr, nullptr};
  if (L.fused) {
    // prologue (the epilogue's coefficient tables), projections with the
    // responsibilities formed in their epilogue, span totals, scan
    Tensors t;
    t.mu = mu;
    t.ls2 = log_sigma2;
    t.lpi = log_pi;
    t.out = out;
    t.eps = eps;
    t.ws = ws;
    hipError_t e = launch_prologue(p, t, s);
    st = finish_launch(e, "prologue launch");
    if (st != GMA_OK) return st;
    P[0] = P[1] = nullptr;
    P[2] = ws + L.off[4];
    ProjFused fz;
    fz.params = ws + p.off_params;
    fz.head_bytes = p.head_bytes;
    fz.Kp = p.Kp;
    fz.DRP = p.DRP;
    fz.kc = L.kc;
    fz.eq = ws + L.off_eq;
    fz.gt = ws + p.off_gt;
    fz.assign_q = assign_q;
    fz.assign_k = assign_k;
    e = launch_proj(X, W, P, lo, 1, p.B, p.N, (int)p.H, d_model, p.DR, p.DV, s, &fz);
    st = finish_launch(e, "projection launch");
    if (st != GMA_OK) return st;
    t.v = P[2];
    t.eq = ws + L.off_eq;
    t.kc = L.kc;
    t.vtab = ws + L.off_vtab;
    return finish_launch(launch_layer_fused(p, t, causal != 0, s),
                         causal ? "causal launch" : "bidirectional launch");
  }
  if (L.split) {
    P[0] = ws + L.off[0];
    lo[0] = ws + L.off[1];
    P[1] = ws + L.off[2];
    lo[1] = ws + L.off[3];
    P[2] = ws + L.off[4];
  } else {
    for (int m = 0; m < 3; ++m) P[m] = ws + L.off[m];
  }
  hipError_t e = launch_proj(X, W, P, lo, L.split, p.B, p.N, (int)p.H, d_model, p.DR, p.DV, s);
  st = finish_launch(e, "projection launch");
  if (st != GMA_OK) return st;
  Tensors t;
  t.q = P[0];
  t.k = P[1];
  t.v = P[2];
  t.q_lo = lo[0];
  t.k_lo = lo[1];
  t.mu = mu;
  t.ls2 = log_sigma2;
  t.lpi = log_pi;
  t.out = out;
  t.assign_q = assign_q;
  t.assign_k = assign_k;
  t.eps = eps;
  t.ws = ws;
  return forward_impl(p, t, causal, s, d, !L.split);
}

int gma_responsibilities(const void* X_r, const float* mu, const float* log_sigma2,
                         const float* log_pi, const gma_dims* d, float* gamma, int32_t* assign,
                         void* workspace, size_t workspace_bytes, void* stream) {
  t_err.clear();
  int st = check_dims(d, 0.f, 0);
  if (st != GMA_OK) return st;
  if (!X_r || !mu || !log_sigma2 || !log_pi || !workspace)
    return fail(GMA_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(X_r) || !aligned16(workspace) || !aligned16(mu) || !aligned16(log_sigma2) ||
      ((uintptr_t)log_pi & 3) || ((uintptr_t)gamma & 3) || ((uintptr_t)assign & 3))
    return fail(GMA_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  Plan p;
  st = make_plan(d, 0, false, p);
  if (st != GMA_OK) return st;
  if (workspace_bytes < p.total) return fail(GMA_ERR_WORKSPACE, "workspace too small");
  Tensors t;
  t.q = X_r;
  t.mu = mu;
  t.ls2 = log_sigma2;
  t.lpi = log_pi;
  t.gamma = gamma;
  t.assign_q = assign;
  t.ws = static_cast<char*>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_prologue(p, t, s);
  if (e == hipSuccess) e = launch_resp(p, t, s);
  return finish_launch(e, "responsibility launch");
}

// Usage statistics: the bidirectional plan's parameter tables, then the
// per-workgroup partials of the statistics kernel.
static size_t usage_diag_offset(const Plan& p) { return round256(p.total); }
static size_t usage_total(const Plan& p) {
  return usage_diag_offset(p) + round256((size_t)p.BH * p.S * (3 * p.Kp + 4) * 4);
}

int gma_usage_workspace_bytes(const gma_dims* d, size_t* bytes) {
  t_err.clear();
  if (!bytes) return fail(GMA_ERR_INVALID_ARG, "bytes is NULL");
  Plan p;
  int st = make_plan(d, 0, false, p);
  if (st != GMA_OK) return st;
  *bytes = usage_total(p);
  return GMA_OK;
}

int gma_usage_stats(const void* X_r, const float* mu, const float* log_sigma2,
                    const float* log_pi, const gma_dims* d, float util_threshold,
                    int32_t* counts, float* mean_gamma, float* utilization, float* head_stats,
                    void* workspace, size_t workspace_bytes, void* stream) {
  t_err.clear();
  int st = check_dims(d, 0.f, 0);
  if (st != GMA_OK) return st;
  if (!X_r || !mu || !log_sigma2 || !log_pi || !workspace)
    return fail(GMA_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(X_r) || !aligned16(workspace) || !aligned16(mu) || !aligned16(log_sigma2) ||
      ((uintptr_t)log_pi & 3) || ((uintptr_t)counts & 3) || ((uintptr_t)mean_gamma & 3) ||
      ((uintptr_t)utilization & 3) || ((uintptr_t)head_stats & 3))
    return fail(GMA_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  if (!isfinite(util_threshold)) return fail(GMA_ERR_INVALID_ARG, "util_threshold must be finite");
  Plan p;
  st = make_plan(d, 0, false, p);
  if (st != GMA_OK) return st;
  if (d->B * d->N >= ((int64_t)1 << 31))
    return fail(GMA_ERR_UNSUPPORTED, "B*N must be below 2^31 for the int32 counts");
  if (workspace_bytes < usage_total(p)) return fail(GMA_ERR_WORKSPACE, "workspace too small");
  Tensors t;
  t.q = X_r;
  t.mu = mu;
  t.ls2 = log_sigma2;
  t.lpi = log_pi;
  t.ws = static_cast<char*>(workspace);
  t.diag = reinterpret_cast<float*>(t.ws + usage_diag_offset(p));
  t.thr = util_threshold;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_prologue(p, t, s);
  if (e == hipSuccess) e = launch_usage(p, t, counts, mean_gamma, utilization, head_stats, s);
  return finish_launch(e, "usage statistics launch");
}

// The backward's plan: the bidirectional plan at N, or (causal) at N rounded
// up to the 64-token chunk.
static int backward_plan(const gma_dims* d, int causal, Plan& p) {
  gma_dims dp = *d;
  if (causal) dp.N = (d->N + 63) / 64 * 64;
  int st = make_plan(&dp, 0, false, p);
  if (st != GMA_OK) return st;
  if (dp.N > (int64_t)65535 * 64)
    return fail(GMA_ERR_UNSUPPORTED, "the backward takes N up to 65535 * 64");
  if (causal && p.BH * (dp.N / 64) > 65535)
    return fail(GMA_ERR_UNSUPPORTED, "the causal backward takes B*H*ceil(N/64) up to 65535");
  return GMA_OK;
}

int gma_backward_workspace_bytes(const gma_dims* d, int causal, size_t* bytes) {
  t_err.clear();
  if (!bytes) return fail(GMA_ERR_INVALID_ARG, "bytes is NULL");
  int st = check_dims(d, 0.f, causal);
  if (st != GMA_OK) return st;
  Plan p;
  st = backward_plan(d, causal, p);
  if (st != GMA_OK) return st;
  *bytes = backward_workspace_bytes(p, causal != 0, d->N);
  return GMA_OK;
}

int gma_backward(const void* Q_X, const void* K_X, const void* V_X, const float* mu,
                 const float* log_sigma2, const float* log_pi, float eps, int causal,
                 const void* dO, const gma_dims* d, void* dQ, void* dK, void* dV, float* dmu,
                 float* dlog_sigma2, float* dlog_pi, void* workspace, size_t workspace_bytes,
                 void* stream) {
  t_err.clear();
  int st = check_dims(d, eps, causal);
  if (st != GMA_OK) return st;
  if (!Q_X || !K_X || !V_X || !mu || !log_sigma2 || !log_pi || !dO || !dQ || !dK || !dV ||
      !dmu || !dlog_sigma2 || !dlog_pi || !workspace)
    return fail(GMA_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(Q_X) || !aligned16(K_X) || !aligned16(V_X) || !aligned16(dO) ||
      !aligned16(dQ) || !aligned16(dK) || !aligned16(dV) || !aligned16(workspace) ||
      !aligned16(mu) || !aligned16(log_sigma2) || ((uintptr_t)log_pi & 3) ||
      ((uintptr_t)dmu & 3) || ((uintptr_t)dlog_sigma2 & 3) || ((uintptr_t)dlog_pi & 3))
    return fail(GMA_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  Plan p;
  st = backward_plan(d, causal, p);
  if (st != GMA_OK) return st;
  if (workspace_bytes < backward_workspace_bytes(p, causal != 0, d->N))
    return fail(GMA_ERR_WORKSPACE, "workspace too small");
  Tensors t;
  t.q = Q_X;
  t.k = K_X;
  t.v = V_X;
  t.mu = mu;
  t.ls2 = log_sigma2;
  t.lpi = log_pi;
  t.eps = eps;
  t.ws = static_cast<char*>(workspace);
  BwdTensors g;
  g.dO = dO;
  g.dQ = dQ;
  g.dK = dK;
  g.dV = dV;
  g.dmu = dmu;
  g.dls2 = dlog_sigma2;
  g.dlpi = dlog_pi;
  return finish_launch(launch_backward(p, t, g, causal != 0, d->N,
                                       static_cast<hipStream_t>(stream)),
                       "backward launch");
}

int gma_prefix_state(const void* K_X, const void* V_X, const float* mu, const float* log_sigma2,
                     const float* log_pi, float* state_v, float* state_z, const gma_dims* d,
                     int32_t* assign_k, void* workspace, size_t workspace_bytes, void* stream) {
  t_err.clear();
  int st = check_dims(d, 0.f, 0);
  if (st != GMA_OK) return st;
  if (!K_X || !V_X || !mu || !log_sigma2 || !log_pi || !state_v || !state_z || !workspace)
    return fail(GMA_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(K_X) || !aligned16(V_X) || !aligned16(workspace) || !aligned16(mu) ||
      !aligned16(log_sigma2) || !aligned16(state_v) || ((uintptr_t)log_pi & 3) ||
      ((uintptr_t)state_z & 3) || ((uintptr_t)assign_k & 3))
    return fail(GMA_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  Plan p;
  st = make_plan(d, 0, false, p);
  if (st != GMA_OK) return st;
  if (workspace_bytes < p.total) return fail(GMA_ERR_WORKSPACE, "workspace too small");
  Tensors t;
  t.k = K_X;
  t.v = V_X;
  t.mu = mu;
  t.ls2 = log_sigma2;
  t.lpi = log_pi;
  t.assign_k = assign_k;
  t.state_v = state_v;
  t.state_z = state_z;
  t.ws = static_cast<char*>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_prologue(p, t, s);
  if (e == hipSuccess) e = launch_bidir(p, t, s);
  return finish_launch(e, "prefix state launch");
}

int gma_decode_step(const void* q, const void* k, const void* v, const float* mu,
                    const float* log_sigma2, const float* log_pi, float eps, float* state_v,
                    float* state_z, void* out, const gma_dims* d, int32_t* assign_q,
                    int32_t* assign_k, void* stream) {
  t_err.clear();
  if (!d) return fail(GMA_ERR_INVALID_ARG, "dims is NULL");
  gma_dims dd = *d;
  dd.chunk = 0;           // a decode step has no chunk
  d = &dd;
  int st = check_dims(d, eps, 1);
  if (st != GMA_OK) return st;
  if (d->N != 1) return fail(GMA_ERR_INVALID_ARG, "a decode step takes N = 1 token per sequence");
  if (!q || !k || !v || !mu || !log_sigma2 || !log_pi || !state_v || !state_z || !out)
    return fail(GMA_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(mu) ||
      !aligned16(log_sigma2) || !aligned16(state_v) || ((uintptr_t)log_pi & 3) ||
      ((uintptr_t)state_z & 3) || ((uintptr_t)assign_q & 3) || ((uintptr_t)assign_k & 3))
    return fail(GMA_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  Plan p;
  p.out_bf = d->dtype == GMA_BF16;
  p.B = d->B;
  p.H = d->H;
  p.N = 1;
  p.BH = d->B * d->H;
  p.DR = d->d_r;
  p.DV = d->d_v;
  p.K = d->K;
  Tensors t;
  t.q = q;
  t.k = k;
  t.v = v;
  t.mu = mu;
  t.ls2 = log_sigma2;
  t.lpi = log_pi;
  t.out = out;
  t.assign_q = assign_q;
  t.assign_k = assign_k;
  t.eps = eps;
  return finish_launch(launch_decode(p, t, state_v, state_z, static_cast<hipStream_t>(stream)),
                       "decode launch");
}

int gma_reparameterize(const float* omega, const float* alpha, float eps_sigma, int64_t H,
                       int32_t K, int32_t d_r, float* log_sigma2, float* log_pi, void* stream) {
  t_err.clear();
  if (!omega || !alpha || !log_sigma2 || !log_pi)
    return fail(GMA_ERR_INVALID_ARG, "a required pointer is NULL");
  if (((uintptr_t)omega & 3) || ((uintptr_t)alpha & 3) || ((uintptr_t)log_sigma2 & 3) ||
      ((uintptr_t)log_pi & 3))
    return fail(GMA_ERR_INVALID_ARG, "tensor pointers must be 4-byte aligned");
  if (H < 1 || K < 1 || d_r < 1) return fail(GMA_ERR_INVALID_ARG, "H, K and d_r must be >= 1");
  if (!(eps_sigma > 0.f) || !isfinite(eps_sigma))
    return fail(GMA_ERR_INVALID_ARG, "eps_sigma must be finite and > 0");
  if (H > 65535 || (int64_t)K * d_r > ((int64_t)1 << 24) || H * K * (int64_t)d_r > ((int64_t)1 << 30))
    return fail(GMA_ERR_UNSUPPORTED, "parameter arrays too large");
  return finish_launch(launch_reparam(omega, alpha, eps_sigma, H, K, d_r, log_sigma2, log_pi,
                                      static_cast<hipStream_t>(stream)),
                       "reparameterisation launch");
}

const char* gma_status_string(int status) {
  switch (status) {
    case GMA_OK: return "GMA_OK";
    case GMA_ERR_INVALID_ARG: return "GMA_ERR_INVALID_ARG: invalid argument";
    case GMA_ERR_UNSUPPORTED: return "GMA_ERR_UNSUPPORTED: shape outside the supported set";
    case GMA_ERR_WORKSPACE: return "GMA_ERR_WORKSPACE: workspace too small";
    case GMA_ERR_HIP: return "GMA_ERR_HIP: HIP runtime or launch failure";
    default: return "unknown gma status";
  }
}

const char* gma_last_error(void) { return t_err.c_str(); }

int gma_timing_enable(int enable) {
  g_launch_hook = enable ? timing_hook : nullptr;
  return GMA_OK;
}

int gma_timing_collect(gma_kernel_time* out, int max, int* count) {
  t_err.clear();
  std::vector<Pending> pend;
  pend.swap(t_timing.pending);
  std::vector<Total> totals;
  hipError_t first_err = hipSuccess;
  for (auto& pe : pend) {
    float ms = 0.f;
    hipError_t e = pe.err;
    if (e == hipSuccess) e = hipEventSynchronize(pe.stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, pe.start, pe.stop);
    // every event is released, also after a failure
    if (pe.start) (void)hipEventDestroy(pe.start);
    if (pe.stop) (void)hipEventDestroy(pe.stop);
    if (e != hipSuccess) {
      if (first_err == hipSuccess) first_err = e;
      continue;
    }
    bool found = false;
    for (auto& tt : totals)
      if (tt.name == pe.tag) {
        tt.launches += 1;
        tt.ms += ms;
        found = true;
      }
    if (!found) totals.push_back(Total{pe.tag, 1, (double)ms});
  }
  if (count) *count = (int)totals.size();
  for (int i = 0; out && i < max && i < (int)totals.size(); ++i) {
    memset(out[i].name, 0, sizeof(out[i].name));
    strncpy(out[i].name, totals[i].name.c_str(), sizeof(out[i].name) - 1);
    out[i].launches = totals[i].launches;
    out[i].total_ms = totals[i].ms;
  }
  if (first_err != hipSuccess)
    return fail(GMA_ERR_HIP, std::string("timing: ") + hipGetErrorString(first_err));
  return GMA_OK;
}

}  // extern "C"
