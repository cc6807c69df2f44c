"""Convenience layer over the C ABI: derives gma_dims from tensor shapes and
allocates outputs and workspace with torch (device memory plumbing only).
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import binding as B


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
    Bb, H, N, d_r = Q.shape
    d_v = V.shape[-1]
    Kc = mu.shape[1]
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


def layer_forward(X: torch.Tensor, W_Q: torch.Tensor, W_K: torch.Tensor, W_V: torch.Tensor,
                  H: int, mu: torch.Tensor, log_sigma2: torch.Tensor, log_pi: torch.Tensor,
                  eps: float = 1e-6, causal: bool = True, assign: bool = False,
                  workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                  stream=None):
    Bb, N, d_model = X.shape
    d_r = W_Q.shape[1] // H
    d_v = W_V.shape[1] // H
    Kc = mu.shape[1]
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
    Bb, H, N, d_r = X.shape
    Kc = mu.shape[1]
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
    Bb, H, N, d_r = K.shape
    d_v = V.shape[-1]
    Kc = mu.shape[1]
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
    Bb, H, _, d_r = q.shape
    d_v = v.shape[-1]
    Kc = mu.shape[1]
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
    H, Kc, d_r = omega.shape
    ls2 = torch.empty_like(omega)
    lpi = torch.empty_like(alpha)
    B.gma_reparameterize(omega, alpha, eps_sigma, H, Kc, d_r, ls2, lpi, stream)
    return ls2, lpi


def usage_stats(X: torch.Tensor, mu: torch.Tensor, log_sigma2: torch.Tensor,
                log_pi: torch.Tensor, util_threshold: float = 0.1, stream=None):
    """Per-head component-usage diagnostics of the responsibilities of X
    [B,H,N,d_r]: dict(counts [H,K] int32, mean_gamma, utilization [H,K],
    token_entropy, usage_entropy, used [H])."""
    Bb, H, N, d_r = X.shape
    Kc = mu.shape[1]
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
    Bb, H, N, d_r = Q.shape
    d_v = V.shape[-1]
    Kc = mu.shape[1]
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
