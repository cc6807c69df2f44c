"""Seeded synthetic inputs for the GMA forward workloads.

This module only draws random numbers and rounds them to the storage type.
It holds none of the method's arithmetic: no densities, no posteriors, no
softmax over components.  Both the HIP path (through the binding) and the CPU
oracle consume exactly the arrays produced here.

Workloads (names describe the shape; all use numpy ``default_rng(seed)``):

* ``tiny_bidir_f32``      B1 H1 N256   d_r16 d_v32  K8    fp32, bidirectional
* ``lra_bidir_f32``       B8 H8 N4096  d_r64 d_v64  K64   fp32, bidirectional
  (the long-context-classification shape of the paper's LRA experiments)
* ``lm_causal_bf16``      B4 H12 N8192 d_r64 d_v64  K64   bf16, causal, chunk 64
  (the autoregressive language-modelling shape of the WikiText-103 runs)
* ``lm_causal_k256_bf16`` the same shape with K256, the component count of the
  WikiText-103 language model
* ``long_bidir_bf16``     B1 H32 N32768 d_r64 d_v128 K128 bf16, bidirectional,
  skewed parameters: mu ~ N(0, 1.5), log sigma^2 ~ U(-1.5, 0.5),
  prior logits ~ N(0, 2)
* ``long_bidir_k256_bf16`` the long-context shape at K256
* ``layer_causal_bf16``   X[2,16384,1024] bf16, W_Q/W_K/W_V [1024, 16*64] with
  entries ~ N(0, 1/1024) rounded to bf16, H16 d_r64 d_v64 K32, causal
* ``decode_bf16``         one causal decode step for a serving batch: B64 H32,
  one new token per sequence (N1), d_r64 d_v128 K128 bf16, the long-context
  parameter distributions, and a carried state standing for a 4096-token
  prefix (see ``make_state``)

``N(0, a)`` denotes variance ``a``.  Routing vectors and values are standard
normal, the stand-in for learned projections (no dataset or trained weights
are used).  Component parameters per head: mu [H,K,d_r], log sigma^2 [H,K,d_r],
prior logits alpha [H,K].  The priors are pi = softmax(alpha) (the paper's
Eq. 15); what is handed to the library and the oracle as ``log_pi`` is alpha
itself, i.e. log pi up to an additive per-head constant.

Draw order: Q_X, K_X, V_X, mu, log_sigma2, alpha (layer workload: X, W_Q, W_K,
W_V, then mu, log_sigma2, alpha).  Draws are float32 standard normals scaled
by the stated standard deviation; bf16 workloads then round to bf16 with
round-to-nearest-even and keep the rounded values (exactly representable in
float32) as the ground truth for every consumer.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d_r: int
    d_v: int
    K: int
    dtype: str            # "f32" or "bf16": storage type of Q_X/K_X/V_X (and X, W)
    causal: bool
    mu_var: float = 1.0
    ls2_lo: float = -1.0
    ls2_hi: float = 1.0
    logit_var: float = 1.0
    eps: float = 1e-6
    chunk: int = 64
    d_model: int = 0      # > 0: projection-layer workload (X and W are drawn)
    w_var: float = 0.0
    state_len: int = 0    # > 0: decode-step workload (a carried state is drawn)

    @property
    def tokens_heads(self) -> int:
        return self.B * self.H * self.N

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny_bidir_f32", 1, 1, 256, 16, 32, 8, "f32", False),
        Workload("lra_bidir_f32", 8, 8, 4096, 64, 64, 64, "f32", False),
        Workload("lm_causal_bf16", 4, 12, 8192, 64, 64, 64, "bf16", True),
        Workload("lm_causal_k256_bf16", 4, 12, 8192, 64, 64, 256, "bf16", True),
        Workload("long_bidir_bf16", 1, 32, 32768, 64, 128, 128, "bf16", False,
                 mu_var=1.5, ls2_lo=-1.5, ls2_hi=0.5, logit_var=2.0),
        Workload("long_bidir_k256_bf16", 1, 32, 32768, 64, 128, 256, "bf16", False,
                 mu_var=1.5, ls2_lo=-1.5, ls2_hi=0.5, logit_var=2.0),
        Workload("layer_causal_bf16", 2, 16, 16384, 64, 64, 32, "bf16", True,
                 d_model=1024, w_var=1.0 / 1024.0),
        Workload("decode_bf16", 64, 32, 1, 64, 128, 128, "bf16", True,
                 mu_var=1.5, ls2_lo=-1.5, ls2_hi=0.5, logit_var=2.0, state_len=4096),
    ]
}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even).

    Returns the uint16 bit patterns.  Inputs here are finite by construction.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1))
    return ((bits + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Tensor:
    """A generated tensor: exact float32 values plus, for bf16 storage, the bits."""
    f32: np.ndarray
    bf16_bits: Optional[np.ndarray] = None

    @property
    def shape(self):
        return self.f32.shape


def _normal(rng: np.random.Generator, shape, var: float) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if var != 1.0:
        x *= np.float32(np.sqrt(var))
    return x


def _store(x: np.ndarray, dtype: str) -> Tensor:
    if dtype == "bf16":
        bits = round_to_bf16(x)
        return Tensor(bf16_bits_to_f32(bits), bits)
    return Tensor(np.ascontiguousarray(x, dtype=np.float32))


def make_params(rng: np.random.Generator, w: Workload):
    """Component parameters, float32: mu [H,K,d_r], log sigma^2 [H,K,d_r], alpha [H,K]."""
    mu = _normal(rng, (w.H, w.K, w.d_r), w.mu_var)
    ls2 = rng.uniform(w.ls2_lo, w.ls2_hi, size=(w.H, w.K, w.d_r)).astype(np.float32)
    alpha = _normal(rng, (w.H, w.K), w.logit_var)
    return mu, ls2, alpha


def make_state(rng: np.random.Generator, B: int, H: int, K: int, d_v: int, length: int):
    """A carried causal state standing for a prefix of ``length`` tokens, float32:
    the per-component counts z [B,H,K] split ``length`` by a flat Dirichlet
    draw, and S [B,H,K,d_v] has entries ~ N(0, z) (a sum of z standard normal
    values).  Draw order: the Dirichlet weights, then the normals."""
    wts = rng.dirichlet(np.ones(K), size=(B, H))
    z = (length * wts).astype(np.float32)
    S = rng.standard_normal(size=(B, H, K, d_v), dtype=np.float32)
    S *= np.sqrt(z)[..., None]
    return np.ascontiguousarray(S), np.ascontiguousarray(z)


def generate(w: Workload, seed: int = 0) -> Dict[str, object]:
    """Draw one batch of inputs for workload ``w``.

    Returns a dict with Tensor entries ``Q``, ``K``, ``V`` ([B,H,N,d]) or, for
    a projection-layer workload, ``X`` ([B,N,d_model]), ``W_Q``, ``W_K``
    ([d_model, H*d_r]), ``W_V`` ([d_model, H*d_v]); and float32 arrays ``mu``,
    ``log_sigma2``, ``log_pi``; for a decode-step workload also the carried
    state ``S`` [B,H,K,d_v] and ``z`` [B,H,K] (float32, drawn last).
    """
    rng = np.random.default_rng(seed)
    out: Dict[str, object] = {"workload": w, "seed": seed}
    if w.d_model > 0:
        out["X"] = _store(_normal(rng, (w.B, w.N, w.d_model), 1.0), w.dtype)
        out["W_Q"] = _store(_normal(rng, (w.d_model, w.H * w.d_r), w.w_var), w.dtype)
        out["W_K"] = _store(_normal(rng, (w.d_model, w.H * w.d_r), w.w_var), w.dtype)
        out["W_V"] = _store(_normal(rng, (w.d_model, w.H * w.d_v), w.w_var), w.dtype)
    else:
        out["Q"] = _store(_normal(rng, (w.B, w.H, w.N, w.d_r), 1.0), w.dtype)
        out["K"] = _store(_normal(rng, (w.B, w.H, w.N, w.d_r), 1.0), w.dtype)
        out["V"] = _store(_normal(rng, (w.B, w.H, w.N, w.d_v), 1.0), w.dtype)
    mu, ls2, alpha = make_params(rng, w)
    out["mu"], out["log_sigma2"], out["log_pi"] = mu, ls2, alpha
    if w.state_len > 0:
        out["S"], out["z"] = make_state(rng, w.B, w.H, w.K, w.d_v, w.state_len)
    return out


def sample_rows(N: int, count: int, seed: int = 1) -> np.ndarray:
    """Sorted distinct row indices for sampled checks; always includes 0 and N-1."""
    rng = np.random.default_rng(seed)
    count = min(count, N)
    rows = set(rng.choice(N, size=count, replace=False).tolist())
    rows.update({0, N - 1})
    return np.array(sorted(rows), dtype=np.int64)
