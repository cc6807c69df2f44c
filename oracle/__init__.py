"""fp64 CPU oracle for the GMA forward pass (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never does, and the
oracle imports nothing from it.

The numerical work is in ``gma_oracle.c`` (plain C, double precision, straight
loops).  This module builds it with gcc, marshals numpy arrays, and adds the
projection step of the full layer (Eq. 4 of "Gaussian Mixture Attention:
Linear-Time Sequence Mixing via Probabilistic Latent Routing", Section
"Projections"), for which ``numpy.matmul`` in float64 serves as the library
matrix product.

``backward`` (gradients of the bidirectional forward) is plain numpy over the
C responsibilities; its pins are in tests/test_oracle_backward.py (central
finite differences of the C forward, invariants, closed cases).
``usage_stats`` (component-usage diagnostics) is plain numpy over the C
responsibilities; its pins are in tests/test_oracle_usage.py.
``reparameterize`` (Eqs. 14-15) is plain numpy; its pins are in
tests/test_oracle_reparam.py (scipy's softplus and log_softmax, closed
values, the simplex and shift invariance).

Pins (see tests/test_oracle.py): responsibilities against scikit-learn's
diagonal-covariance GaussianMixture posterior; outputs against a brute-force
materialised affinity built from scikit-learn's responsibilities; closed
forms (K=1 mean and running mean, two-component logistic posterior,
well-separated clusters, identical components); invariants (row sums, causal
future-perturbation, last causal row equals the bidirectional row).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gma_oracle.c")
_LIB_PATH = os.path.join(_HERE, "_gma_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (IEEE double, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall",
                               "-o", tmp, _SRC, "-lm", "-lpthread"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _bind(path: str):
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i64, i32 = ctypes.c_int64, ctypes.c_int
    lib.gmao_forward.argtypes = [P, P, P, P, P, P, i64, i64, i64, i32, i32, i32,
                                 ctypes.c_double, i32, P, i64, P, P, P, P, P, i32]
    lib.gmao_forward.restype = ctypes.c_int
    lib.gmao_resp.argtypes = [P, i64, i64, i64, i32, P, P, P, i32, P, P, P]
    lib.gmao_resp.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        _lib = _bind(_LIB_PATH)
    return _lib


class using_library:
    """Context manager: route calls to another build of the oracle source
    (used by the mutation tests, which compile deliberately broken copies)."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _lib
        self._saved = _load()
        _lib = _bind(self.path)
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self._saved
        return False


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def forward(Q, K, V, mu, log_sigma2, log_pi, eps: float, causal: bool,
            rows: Optional[np.ndarray] = None, want_assign: bool = False,
            want_latent: bool = False, nthreads: Optional[int] = None) -> dict:
    """GMA forward (Eqs. 3, 5-7; causal: the prefix form of Eq. 8b).

    Q, K: [B,H,N,d_r]; V: [B,H,N,d_v]; mu, log_sigma2: [H,K,d_r]; log_pi: [H,K]
    (any additive per-head constant).  ``rows``: optional sorted row indices
    to produce.  Returns dict(out=[B,H,R,d_v] float64, assign_q, assign_k,
    vtilde=[B,H,K,d_v], z=[B,H,K]).
    """
    lib = _load()
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    mu, ls2, lpi = _f64(mu), _f64(log_sigma2), _f64(log_pi)
    B, H, N, d_r = Q.shape
    d_v = V.shape[-1]
    Kc = mu.shape[1]
    assert K.shape == Q.shape and V.shape[:3] == (B, H, N)
    assert mu.shape == (H, Kc, d_r) and ls2.shape == mu.shape and lpi.shape == (H, Kc)
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
    R = N if rows is None else rows.shape[0]
    out = np.empty((B, H, R, d_v), np.float64)
    aq = np.empty((B, H, R), np.int32) if want_assign else None
    ak = np.empty((B, H, N), np.int32) if want_assign else None
    vt = np.empty((B, H, Kc, d_v), np.float64) if (want_latent and not causal) else None
    zt = np.empty((B, H, Kc), np.float64) if (want_latent and not causal) else None
    rc = lib.gmao_forward(_ptr(Q), _ptr(K), _ptr(V), _ptr(mu), _ptr(ls2), _ptr(lpi),
                          B, H, N, d_r, d_v, Kc, float(eps), int(bool(causal)),
                          _ptr(rows), 0 if rows is None else R,
                          _ptr(out), _ptr(aq), _ptr(ak), _ptr(vt), _ptr(zt),
                          nthreads or default_threads())
    if rc != 0:
        raise ValueError("gmao_forward rejected its arguments (code %d)" % rc)
    return {"out": out, "assign_q": aq, "assign_k": ak, "vtilde": vt, "z": zt}


def responsibilities(X, mu, log_sigma2, log_pi) -> dict:
    """Eq. 3 for X [U,N,d_r] (or [B,H,N,d_r]); unit u uses head u % H.

    Returns gamma [...,N,K], assign [...,N], score [...,N,K] (natural log of
    prior times density, i.e. the quantity Eq. 16 takes a softmax of).
    """
    lib = _load()
    X = _f64(X)
    lead = X.shape[:-2]
    N, d_r = X.shape[-2:]
    U = int(np.prod(lead)) if lead else 1
    mu, ls2, lpi = _f64(mu), _f64(log_sigma2), _f64(log_pi)
    H, Kc = lpi.shape
    gamma = np.empty(lead + (N, Kc), np.float64)
    score = np.empty(lead + (N, Kc), np.float64)
    assign = np.empty(lead + (N,), np.int32)
    rc = lib.gmao_resp(_ptr(X), U, H, N, d_r, _ptr(mu), _ptr(ls2), _ptr(lpi), Kc,
                       _ptr(gamma), _ptr(assign), _ptr(score))
    if rc != 0:
        raise ValueError("gmao_resp rejected its arguments (code %d)" % rc)
    return {"gamma": gamma, "assign": assign, "score": score}


def decode_step(S, z, q, k, v, mu, log_sigma2, log_pi, eps: float) -> dict:
    """One token of the causal form from a carried prefix state ("Causal GMA":
    the prefix memories V~^(i), Z^(i) and Eq. 8b, prefix j <= i inclusive).

    The state of a prefix is V~ = sum_j gamma^K_j (outer) v_j and Z = sum_j
    gamma^K_j over its tokens.  Appending token i adds its own key term, then
    its query reads the updated state:
      S' = S + gamma^K(k_i) (outer) v_i,  z' = z + gamma^K(k_i),
      o_i = gamma^Q(q_i) . S' / (gamma^Q(q_i) . z' + eps).
    S [B,H,K,d_v], z [B,H,K], q, k [B,H,d_r], v [B,H,d_v]; the responsibilities
    are the C oracle's (Eq. 3).  Returns dict(S, z, out [B,H,d_v], assign_q,
    assign_k), all float64 (assignments int32).
    """
    S, z, v = _f64(S), _f64(z), _f64(v)
    rq = responsibilities(_f64(q)[:, :, None, :], mu, log_sigma2, log_pi)
    rk = responsibilities(_f64(k)[:, :, None, :], mu, log_sigma2, log_pi)
    gq, gk = rq["gamma"][:, :, 0], rk["gamma"][:, :, 0]          # [B,H,K]
    S2 = S + gk[:, :, :, None] * v[:, :, None, :]
    z2 = z + gk
    num = np.einsum("bhk,bhkd->bhd", gq, S2)
    den = np.einsum("bhk,bhk->bh", gq, z2) + eps
    return {"S": S2, "z": z2, "out": num / den[:, :, None],
            "assign_q": rq["assign"][:, :, 0], "assign_k": rk["assign"][:, :, 0]}


def backward(Q, K, V, mu, log_sigma2, log_pi, eps: float, dO, causal: bool = False) -> dict:
    """Gradients of a scalar loss through the bidirectional forward, given
    dL/dO ("Gradient structure": the score gradient of Eq. 18 and its
    footnote, chained to the score's arguments by the chain rule of Eq. 17).

    Forward, per unit: gamma = softmax_k(s) (Eq. 3), V~ = Gk^T V, Z = Gk^T 1
    (Eqs. 5-6), n_i = Gq_i V~, d_i = Gq_i . Z + eps, o_i = n_i / d_i (Eq. 7).
    Backward, in that order:
      a_i = dO_i / d_i,  b_i = -(dO_i . o_i) / d_i
      dGq_ik = a_i . V~_k + b_i Z_k
      dV~_k = sum_i Gq_ik a_i,  dZ_k = sum_i Gq_ik b_i
      dV_j = sum_k Gk_jk dV~_k,  dGk_jk = v_j . dV~_k + dZ_k
      ds_ik = gamma_ik (dG_ik - sum_l gamma_il dG_il)                 (Eq. 18)
    and with s_ik = log pi_k - (1/2) sum_d [(x_id - mu_kd)^2 w_kd + log sigma^2_kd],
    w = exp(-log sigma^2):
      dx_id = -sum_k ds_ik (x_id - mu_kd) w_kd
      dmu_kd = sum_i ds_ik (x_id - mu_kd) w_kd
      dlog sigma^2_kd = sum_i ds_ik ((x_id - mu_kd)^2 w_kd - 1) / 2
      dlog pi_k = sum_i ds_ik
    where the parameter sums run over queries and keys of every batch.
    Causal ("Causal GMA", Eq. 8b): V~ and Z become the inclusive prefix sums
    S_i, z_i over j <= i, so dGq_ik = a_i . S_i,k + b_i z_i,k, and a key j
    receives the suffix sums over the queries i >= j:
    dV_j = sum_k Gk_jk sum_{i>=j} Gq_ik a_i,
    dGk_jk = v_j . sum_{i>=j} Gq_ik a_i + sum_{i>=j} Gq_ik b_i.
    Shapes as forward; dO [B,H,N,d_v].  Returns float64 dQ, dK, dV, dmu,
    dlog_sigma2, dlog_pi.
    """
    Q, K, V, dO = _f64(Q), _f64(K), _f64(V), _f64(dO)
    mu, ls2, lpi = _f64(mu), _f64(log_sigma2), _f64(log_pi)
    Gq = responsibilities(Q, mu, ls2, lpi)["gamma"]                 # [B,H,N,K]
    Gk = responsibilities(K, mu, ls2, lpi)["gamma"]
    if not causal:
        Vt = np.einsum("bhnk,bhnd->bhkd", Gk, V)
        Z = Gk.sum(axis=2)                                         # [B,H,K]
        den = np.einsum("bhnk,bhk->bhn", Gq, Z) + eps
        O = np.einsum("bhnk,bhkd->bhnd", Gq, Vt) / den[..., None]
        a = dO / den[..., None]
        bb = -(dO * O).sum(-1) / den
        dGq = np.einsum("bhnd,bhkd->bhnk", a, Vt) + bb[..., None] * Z[:, :, None, :]
        dVt = np.einsum("bhnk,bhnd->bhkd", Gq, a)
        dZ = np.einsum("bhnk,bhn->bhk", Gq, bb)
        dV = np.einsum("bhnk,bhkd->bhnd", Gk, dVt)
        dGk = np.einsum("bhnd,bhkd->bhnk", V, dVt) + dZ[:, :, None, :]
    else:
        # prefix states per position (inclusive), [B,H,N,K,d_v] and [B,H,N,K]
        S = np.cumsum(Gk[..., :, None] * V[..., None, :], axis=2)
        z = np.cumsum(Gk, axis=2)
        den = np.einsum("bhnk,bhnk->bhn", Gq, z) + eps
        O = np.einsum("bhnk,bhnkd->bhnd", Gq, S) / den[..., None]
        a = dO / den[..., None]
        bb = -(dO * O).sum(-1) / den
        dGq = np.einsum("bhnd,bhnkd->bhnk", a, S) + bb[..., None] * z
        # suffix sums over the queries i >= j
        T = Gq[..., :, None] * a[..., None, :]                     # [B,H,N,K,d_v]
        G = np.flip(np.cumsum(np.flip(T, axis=2), axis=2), axis=2)
        Hs = np.flip(np.cumsum(np.flip(Gq * bb[..., None], axis=2), axis=2), axis=2)
        dV = np.einsum("bhnk,bhnkd->bhnd", Gk, G)
        dGk = np.einsum("bhnd,bhnkd->bhnk", V, G) + Hs
    w = np.exp(-ls2)                                               # [H,K,d_r]
    out = {"dV": dV}
    dmu = np.zeros_like(mu)
    dls2 = np.zeros_like(ls2)
    dlpi = np.zeros_like(lpi)
    for name, X, G, dG in (("dQ", Q, Gq, dGq), ("dK", K, Gk, dGk)):
        ds = G * (dG - (G * dG).sum(-1, keepdims=True))            # Eq. 18
        diff = X[:, :, :, None, :] - mu[None, :, None, :, :]       # [B,H,N,K,d_r]
        out[name] = -np.einsum("bhnk,bhnkd,hkd->bhnd", ds, diff, w)
        dmu += np.einsum("bhnk,bhnkd,hkd->hkd", ds, diff, w)
        dls2 += 0.5 * (np.einsum("bhnk,bhnkd,hkd->hkd", ds, diff ** 2, w)
                       - ds.sum(axis=(0, 2))[:, :, None])
        dlpi += ds.sum(axis=(0, 2))
    out.update(dmu=dmu, dlog_sigma2=dls2, dlog_pi=dlpi)
    return out


def usage_stats(X, mu, log_sigma2, log_pi, util_threshold: float) -> dict:
    """Component-usage diagnostics of the responsibilities of X [B,H,N,d_r]
    (the marginal use of the components and the hard assignments
    z_i = argmax_k gamma_ik, monitored for under-use and collapse), per head
    over the T = B*N tokens of that head:

      counts[h,k]      #{i : z_i = k}
      mean_gamma[h,k]  (1/T) sum_i gamma_ik
      utilization[h,k] (1/T) #{i : gamma_ik > util_threshold}
      token_entropy[h] (1/T) sum_i -sum_k gamma_ik ln gamma_ik   (0 ln 0 = 0)
      usage_entropy[h] -sum_k p_k ln p_k / ln K, p_k = counts[h,k] / T (0 if K = 1)
      used[h]          #{k : counts[h,k] > 0}

    The responsibilities and assignments are the C oracle's (Eq. 3).
    """
    r = responsibilities(X, mu, log_sigma2, log_pi)
    g, z = r["gamma"], r["assign"]
    B, H, N, K = g.shape
    T = B * N
    counts = np.zeros((H, K), np.int64)
    for h in range(H):
        for b in range(B):
            for k in range(K):
                counts[h, k] += int(np.count_nonzero(z[b, h] == k))
    mean_gamma = g.sum(axis=(0, 2)) / T
    utilization = (g > util_threshold).sum(axis=(0, 2)) / T
    glng = np.where(g > 0, g * np.log(np.where(g > 0, g, 1.0)), 0.0)
    token_entropy = -glng.sum(axis=(0, 2, 3)) / T
    p = counts / T
    plnp = np.where(p > 0, p * np.log(np.where(p > 0, p, 1.0)), 0.0)
    usage_entropy = -plnp.sum(-1) / np.log(K) if K > 1 else np.zeros(H)
    used = (counts > 0).sum(-1)
    return {"counts": counts, "mean_gamma": mean_gamma, "utilization": utilization,
            "token_entropy": token_entropy, "usage_entropy": usage_entropy, "used": used,
            "gamma": g, "assign": z}


def reparameterize(omega, alpha, eps_sigma: float) -> dict:
    """Constrained mixture parameters from the unconstrained ones (the
    reparameterisations used for training: Eq. 14, sigma^2 = log(1 + exp(omega)) +
    eps_sigma per component and routing dimension; Eq. 15, pi = softmax over
    the components of the logits alpha).

    omega [H,K,d_r], alpha [H,K].  Returns dict(log_sigma2 [H,K,d_r],
    log_pi [H,K]) in float64, the arrays the forward takes.  log(1 + exp(w))
    is evaluated as max(w, 0) + log1p(exp(-|w|)) (the same number, without
    overflow for large w); log pi_k = alpha_k - log sum_l exp(alpha_l), with
    the largest logit subtracted inside the exponentials.
    """
    w = _f64(omega)
    a = _f64(alpha)
    sp = np.maximum(w, 0.0) + np.log1p(np.exp(-np.abs(w)))
    log_sigma2 = np.log(sp + float(eps_sigma))
    m = a.max(axis=-1, keepdims=True)
    lse = m + np.log(np.exp(a - m).sum(axis=-1, keepdims=True))
    return {"log_sigma2": log_sigma2, "log_pi": a - lse}


def project(X, W, H: int) -> np.ndarray:
    """Eq. 4: X [B,N,d_model] times W [d_model, H*d] in float64, split into heads.

    Head h takes columns [h*d, (h+1)*d).  Returns [B,H,N,d].
    """
    X = _f64(X)
    W = _f64(W)
    B, N, _ = X.shape
    d = W.shape[1] // H
    P = np.matmul(X, W)                       # [B,N,H*d]
    return np.ascontiguousarray(P.reshape(B, N, H, d).transpose(0, 2, 1, 3))


def layer_forward(X, W_Q, W_K, W_V, H: int, mu, log_sigma2, log_pi, eps: float,
                  causal: bool, rows: Optional[np.ndarray] = None,
                  want_assign: bool = False, nthreads: Optional[int] = None) -> dict:
    """Projection (Eq. 4, no bias, no output projection) followed by the GMA forward."""
    Q = project(X, W_Q, H)
    K = project(X, W_K, H)
    V = project(X, W_V, H)
    return forward(Q, K, V, mu, log_sigma2, log_pi, eps, causal, rows=rows,
                   want_assign=want_assign, nthreads=nthreads)
