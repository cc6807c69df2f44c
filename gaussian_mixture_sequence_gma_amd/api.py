"""Convenience layer over the C ABI: derives gma_dims from tensor shapes and
allocates outputs and workspace with torch (device memory plumbing only).

Every entry checks its tensors before anything reaches the library: shapes
consistent with the derived dims, dtypes (routing vectors and values bf16 or
fp32 and alike; mixture parameters fp32), contiguity, and that every tensor
sits on the same CUDA device.  A mismatch raises ValueError; the C ABI only
sees raw pointers and would otherwise read or write out of bounds.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import binding as B


def _req(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _shape(t: torch.Tensor, shape, name: str):
    _req(isinstance(t, torch.Tensor), "%s must be a torch.Tensor" % name)
    _req(tuple(t.shape) == tuple(int(x) for x in shape),
         "%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))


def _check(tensors: dict, params: dict = None, io_dtype=None, H: int = None, Kc: int = None,
           d_r: int = None, extra: dict = None):
    """Validate one call's tensors.  tensors: name -> (tensor or None, shape);
    tensors of io_dtype (routing vectors, values, outputs) must share it, which
    must be bfloat16 or float32.  params: mu, log_sigma2, log_pi (fp32, [H,K,d_r],
    [H,K,d_r], [H,K]), or omega and alpha in place of the last two.  extra: name -> (tensor or None, shape, dtype).  Shapes,
    dtypes and contiguity are checked first, then that all tensors share one
    CUDA device."""
    allt = []
    if io_dtype is not None:
        _req(io_dtype in (torch.bfloat16, torch.float32),
             "unsupported dtype %s (bfloat16 or float32)" % io_dtype)
    for name, (t, shape) in tensors.items():
        if t is None:
            continue
        _shape(t, shape, name)
        _req(t.dtype == io_dtype, "%s has dtype %s, expected %s" % (name, t.dtype, io_dtype))
        allt.append((name, t))
    if params is not None:
        shapes = {"mu": (H, Kc, d_r), "log_sigma2": (H, Kc, d_r), "log_pi": (H, Kc),
                  "omega": (H, Kc, d_r), "alpha": (H, Kc)}
        for name, t in params.items():
            _shape(t, shapes[name], name)
            _req(t.dtype == torch.float32, "%s must be float32, got %s" % (name, t.dtype))
            allt.append((name, t))
    for name, (t, shape, dt) in (extra or {}).items():
        if t is None:
            continue
        if shape is not None:
            _shape(t, shape, name)
        _req(t.dtype == dt, "%s has dtype %s, expected %s" % (name, t.dtype, dt))
        allt.append((name, t))
    for name, t in allt:
        _req(t.is_contiguous(), "%s must be contiguous" % name)
    dev = None
    for name, t in allt:
        _req(t.is_cuda, "%s must be a CUDA tensor (device %s)" % (name, t.device))
        if dev is None:
            dev = t.device
        _req(t.device == dev, "%s is on %s, expected %s" % (name, t.device, dev))


def _ws(workspace):
    return {"workspace": (workspace, None, torch.uint8)} if workspace is not None else {}


def torch_dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return B.GMA_BF16
    if t.dtype == torch.float32:
        return B.GMA_F32
    raise TypeError("unsupported dtype %s (bfloat16 or float32)" % t.dtype)


def host_tensor_to_device(t, device) -> torch.Tensor:
    """Upload a generated inputs.Tensor (bf16 bits or float32 values)."""
    if getattr(t, "bf16_bits", None) is not None:
        bits = torch.from_numpy(np.ascontiguousarray(t.bf16_bits).view(np.int16))
        return bits.to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(t.f32)).to(device)


def alloc_workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def forward(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, mu: torch.Tensor,
            log_sigma2: torch.Tensor, log_pi: torch.Tensor, eps: float = 1e-6,
            causal: bool = False, assign: bool = False, chunk: int = 0,
            workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
            stream=None):
    """O (and optionally z^Q, z^K) for Q, K [B,H,N,d_r], V [B,H,N,d_v]."""
    _req(Q.dim() == 4 and V.dim() == 4 and mu.dim() == 3, "Q, V must be 4-D and mu 3-D")
    Bb, H, N, d_r = Q.shape
    d_v = V.shape[-1]
    Kc = mu.shape[1]
    _check({"Q": (Q, (Bb, H, N, d_r)), "K": (K, (Bb, H, N, d_r)), "V": (V, (Bb, H, N, d_v)),
            "out": (out, (Bb, H, N, d_v))},
           {"mu": mu, "log_sigma2": log_sigma2, "log_pi": log_pi}, Q.dtype, H, Kc, d_r,
           _ws(workspace))
    dims = B.make_dims(Bb, H, N, d_r, d_v, Kc, torch_dtype_code(Q), chunk)
    need = B.gma_forward_workspace_bytes(dims, int(causal))
    if workspace is None or workspace.numel() < need:
        workspace = alloc_workspace(need, Q.device)
    if out is None:
        out = torch.empty((Bb, H, N, d_v), dtype=V.dtype, device=V.device)
    aq = ak = None
    if assign:
        aq = torch.empty((Bb, H, N), dtype=torch.int32, device=Q.device)
        ak = torch.empty((Bb, H, N), dtype=torch.int32, device=Q.device)
    B.gma_forward(Q, K, V, mu, log_sigma2, log_pi, eps, int(causal), out, dims, aq, ak,
                  workspace, workspace.numel(), stream)
    return (out, aq, ak) if assign else out


def forward_reparam(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, mu: torch.Tensor,
                    omega: torch.Tensor, alpha: torch.Tensor, eps_sigma: float = 1e-4,
                    eps: float = 1e-6, causal: bool = False, assign: bool = False,
                    chunk: int = 0, workspace: Optional[torch.Tensor] = None,
                    out: Optional[torch.Tensor] = None, stream=None):
    """forward() from the unconstrained parameters: omega [H,K,d_r] in place of
    log sigma^2 and the prior logits alpha [H,K] in place of log pi (gma_forward_reparam)."""
    _req(Q.dim() == 4 and V.dim() == 4 and mu.dim() == 3, "Q, V must be 4-D and mu 3-D")
    Bb, H, N, d_r = Q.shape
    d_v = V.shape[-1]
    Kc = mu.shape[1]
    _check({"Q": (Q, (Bb, H, N, d_r)), "K": (K, (Bb, H, N, d_r)), "V": (V, (Bb, H, N, d_v)),
            "out": (out, (Bb, H, N, d_v))},
           {"mu": mu, "omega": omega, "alpha": alpha}, Q.dtype, H, Kc, d_r,
           _ws(workspace))
    dims = B.make_dims(Bb, H, N, d_r, d_v, Kc, torch_dtype_code(Q), chunk)
    need = B.gma_forward_workspace_bytes(dims, int(causal))
    if workspace is None or workspace.numel() < need:
        workspace = alloc_workspace(need, Q.device)
    if out is None:
        out = torch.empty((Bb, H, N, d_v), dtype=V.dtype, device=V.device)
    aq = ak = None
    if assign:
        aq = torch.empty((Bb, H, N), dtype=torch.int32, device=Q.device)
        ak = torch.empty((Bb, H, N), dtype=torch.int32, device=Q.device)
    B.gma_forward_reparam(Q, K, V, mu, omega, alpha, eps_sigma, eps, int(causal), out, dims, aq,
                          ak, workspace, workspace.numel(), stream)
    return (out, aq, ak) if assign else out


def layer_forward(X: torch.Tensor, W_Q: torch.Tensor, W_K: torch.Tensor, W_V: torch.Tensor,
                  H: int, mu: torch.Tensor, log_sigma2: torch.Tensor, log_pi: torch.Tensor,
                  eps: float = 1e-6, causal: bool = True, assign: bool = False,
                  workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                  stream=None):
    _req(X.dim() == 3 and W_Q.dim() == 2 and W_V.dim() == 2 and mu.dim() == 3,
         "X must be 3-D, W_Q / W_V 2-D and mu 3-D")
    Bb, N, d_model = X.shape
    _req(H >= 1 and W_Q.shape[1] % H == 0 and W_V.shape[1] % H == 0,
         "projection widths must be multiples of H")
    d_r = W_Q.shape[1] // H
    d_v = W_V.shape[1] // H
    Kc = mu.shape[1]
    _check({"X": (X, (Bb, N, d_model)), "W_Q": (W_Q, (d_model, H * d_r)),
            "W_K": (W_K, (d_model, H * d_r)), "W_V": (W_V, (d_model, H * d_v)),
            "out": (out, (Bb, H, N, d_v))},
           {"mu": mu, "log_sigma2": log_sigma2, "log_pi": log_pi}, X.dtype, H, Kc, d_r,
           _ws(workspace))
    dims = B.make_dims(Bb, H, N, d_r, d_v, Kc, torch_dtype_code(X))
    need = B.gma_layer_workspace_bytes(dims, d_model, int(causal))
    if workspace is None or workspace.numel() < need:
        workspace = alloc_workspace(need, X.device)
    if out is None:
        out = torch.empty((Bb, H, N, d_v), dtype=X.dtype, device=X.device)
    aq = ak = None
    if assign:
        aq = torch.empty((Bb, H, N), dtype=torch.int32, device=X.device)
        ak = torch.empty((Bb, H, N), dtype=torch.int32, device=X.device)
    B.gma_layer_forward(X, W_Q, W_K, W_V, d_model, mu, log_sigma2, log_pi, eps, int(causal),
                        out, dims, aq, ak, workspace, workspace.numel(), stream)
    return (out, aq, ak) if assign else out


def responsibilities(X: torch.Tensor, mu: torch.Tensor, log_sigma2: torch.Tensor,
                     log_pi: torch.Tensor, stream=None):
    """gamma [B,H,N,K] fp32 and z [B,H,N] int32 for X [B,H,N,d_r]."""
    _req(X.dim() == 4 and mu.dim() == 3, "X must be 4-D and mu 3-D")
    Bb, H, N, d_r = X.shape
    Kc = mu.shape[1]
    _check({"X": (X, (Bb, H, N, d_r))}, {"mu": mu, "log_sigma2": log_sigma2, "log_pi": log_pi},
           X.dtype, H, Kc, d_r)
    dims = B.make_dims(Bb, H, N, d_r, 16, Kc, torch_dtype_code(X))
    need = B.gma_forward_workspace_bytes(dims, 0)
    ws = alloc_workspace(need, X.device)
    gamma = torch.empty((Bb, H, N, Kc), dtype=torch.float32, device=X.device)
    assign = torch.empty((Bb, H, N), dtype=torch.int32, device=X.device)
    B.gma_responsibilities(X, mu, log_sigma2, log_pi, dims, gamma, assign, ws, ws.numel(),
                           stream)
    return gamma, assign


def prefix_state(K: torch.Tensor, V: torch.Tensor, mu: torch.Tensor, log_sigma2: torch.Tensor,
                 log_pi: torch.Tensor, assign: bool = False, stream=None):
    """Carried causal state (S [B,H,K,d_v], z [B,H,K], fp32) after the keys and
    values K [B,H,N,d_r], V [B,H,N,d_v]; optionally the key assignments."""
    _req(K.dim() == 4 and V.dim() == 4 and mu.dim() == 3, "K, V must be 4-D and mu 3-D")
    Bb, H, N, d_r = K.shape
    d_v = V.shape[-1]
    Kc = mu.shape[1]
    _check({"K": (K, (Bb, H, N, d_r)), "V": (V, (Bb, H, N, d_v))},
           {"mu": mu, "log_sigma2": log_sigma2, "log_pi": log_pi}, K.dtype, H, Kc, d_r)
    dims = B.make_dims(Bb, H, N, d_r, d_v, Kc, torch_dtype_code(K))
    ws = alloc_workspace(B.gma_forward_workspace_bytes(dims, 0), K.device)
    S = torch.empty((Bb, H, Kc, d_v), dtype=torch.float32, device=K.device)
    z = torch.empty((Bb, H, Kc), dtype=torch.float32, device=K.device)
    ak = torch.empty((Bb, H, N), dtype=torch.int32, device=K.device) if assign else None
    B.gma_prefix_state(K, V, mu, log_sigma2, log_pi, S, z, dims, ak, ws, ws.numel(), stream)
    return (S, z, ak) if assign else (S, z)


def decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, mu: torch.Tensor,
                log_sigma2: torch.Tensor, log_pi: torch.Tensor, S: torch.Tensor,
                z: torch.Tensor, eps: float = 1e-6, assign: bool = False,
                out: Optional[torch.Tensor] = None, stream=None):
    """One token per sequence, q, k [B,H,1,d_r], v [B,H,1,d_v]: returns o
    [B,H,1,d_v] and updates S, z in place (optionally z^Q, z^K [B,H])."""
    _req(q.dim() == 4 and v.dim() == 4 and mu.dim() == 3, "q, v must be 4-D and mu 3-D")
    Bb, H, _, d_r = q.shape
    d_v = v.shape[-1]
    Kc = mu.shape[1]
    _check({"q": (q, (Bb, H, 1, d_r)), "k": (k, (Bb, H, 1, d_r)), "v": (v, (Bb, H, 1, d_v)),
            "out": (out, (Bb, H, 1, d_v))},
           {"mu": mu, "log_sigma2": log_sigma2, "log_pi": log_pi}, q.dtype, H, Kc, d_r,
           {"S": (S, (Bb, H, Kc, d_v), torch.float32), "z": (z, (Bb, H, Kc), torch.float32)})
    dims = B.make_dims(Bb, H, 1, d_r, d_v, Kc, torch_dtype_code(q))
    if out is None:
        out = torch.empty((Bb, H, 1, d_v), dtype=v.dtype, device=v.device)
    aq = ak = None
    if assign:
        aq = torch.empty((Bb, H), dtype=torch.int32, device=q.device)
        ak = torch.empty((Bb, H), dtype=torch.int32, device=q.device)
    B.gma_decode_step(q, k, v, mu, log_sigma2, log_pi, eps, S, z, out, dims, aq, ak, stream)
    return (out, aq, ak) if assign else out


def reparameterize(omega: torch.Tensor, alpha: torch.Tensor, eps_sigma: float = 1e-4,
                   stream=None):
    """(log_sigma2 [H,K,d_r], log_pi [H,K]) from omega [H,K,d_r] and alpha [H,K]."""
    _req(omega.dim() == 3, "omega must be 3-D [H,K,d_r]")
    H, Kc, d_r = omega.shape
    _check({}, extra={"omega": (omega, (H, Kc, d_r), torch.float32),
                      "alpha": (alpha, (H, Kc), torch.float32)})
    ls2 = torch.empty_like(omega)
    lpi = torch.empty_like(alpha)
    B.gma_reparameterize(omega, alpha, eps_sigma, H, Kc, d_r, ls2, lpi, stream)
    return ls2, lpi


def usage_stats(X: torch.Tensor, mu: torch.Tensor, log_sigma2: torch.Tensor,
                log_pi: torch.Tensor, util_threshold: float = 0.1, stream=None):
    """Per-head component-usage diagnostics of the responsibilities of X
    [B,H,N,d_r]: dict(counts [H,K] int32, mean_gamma, utilization [H,K],
    token_entropy, usage_entropy, used [H])."""
    _req(X.dim() == 4 and mu.dim() == 3, "X must be 4-D and mu 3-D")
    Bb, H, N, d_r = X.shape
    Kc = mu.shape[1]
    _check({"X": (X, (Bb, H, N, d_r))}, {"mu": mu, "log_sigma2": log_sigma2, "log_pi": log_pi},
           X.dtype, H, Kc, d_r)
    dims = B.make_dims(Bb, H, N, d_r, 16, Kc, torch_dtype_code(X))
    ws = alloc_workspace(B.gma_usage_workspace_bytes(dims), X.device)
    counts = torch.empty((H, Kc), dtype=torch.int32, device=X.device)
    mg = torch.empty((H, Kc), dtype=torch.float32, device=X.device)
    ut = torch.empty((H, Kc), dtype=torch.float32, device=X.device)
    hs = torch.empty((H, 3), dtype=torch.float32, device=X.device)
    B.gma_usage_stats(X, mu, log_sigma2, log_pi, dims, util_threshold, counts, mg, ut, hs, ws,
                      ws.numel(), stream)
    return {"counts": counts, "mean_gamma": mg, "utilization": ut, "token_entropy": hs[:, 0],
            "usage_entropy": hs[:, 1], "used": hs[:, 2]}


def backward(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, mu: torch.Tensor,
             log_sigma2: torch.Tensor, log_pi: torch.Tensor, dO: torch.Tensor,
             eps: float = 1e-6, causal: bool = False, workspace: Optional[torch.Tensor] = None,
             stream=None):
    """Gradients of the forward given dO: dict(dQ, dK, dV in the input dtype;
    dmu, dlog_sigma2, dlog_pi fp32)."""
    _req(Q.dim() == 4 and V.dim() == 4 and mu.dim() == 3, "Q, V must be 4-D and mu 3-D")
    Bb, H, N, d_r = Q.shape
    d_v = V.shape[-1]
    Kc = mu.shape[1]
    _check({"Q": (Q, (Bb, H, N, d_r)), "K": (K, (Bb, H, N, d_r)), "V": (V, (Bb, H, N, d_v)),
            "dO": (dO, (Bb, H, N, d_v))},
           {"mu": mu, "log_sigma2": log_sigma2, "log_pi": log_pi}, Q.dtype, H, Kc, d_r,
           _ws(workspace))
    dims = B.make_dims(Bb, H, N, d_r, d_v, Kc, torch_dtype_code(Q))
    need = B.gma_backward_workspace_bytes(dims, int(causal))
    if workspace is None or workspace.numel() < need:
        workspace = alloc_workspace(need, Q.device)
    g = {"dQ": torch.empty_like(Q), "dK": torch.empty_like(K), "dV": torch.empty_like(V),
         "dmu": torch.empty_like(mu), "dlog_sigma2": torch.empty_like(log_sigma2),
         "dlog_pi": torch.empty_like(log_pi)}
    B.gma_backward(Q, K, V, mu, log_sigma2, log_pi, eps, int(causal), dO, dims, g["dQ"], g["dK"],
                   g["dV"], g["dmu"], g["dlog_sigma2"], g["dlog_pi"], workspace,
                   workspace.numel(), stream)
    return g
