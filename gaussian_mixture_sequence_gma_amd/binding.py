"""Thin ctypes binding of libgma.so (include/gma.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  Functions carry the C names; tensors are torch
tensors (device memory for the gma_* calls), or None for optional arguments.
A nonzero status raises GmaError with the library's message.  There is no
fallback: if libgma.so is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import List, Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
# GMA_LIBRARY names another build of the same library (e.g. one whose host
# code is compiled with sanitizers); the default is the in-tree build
LIB_PATH = os.environ.get("GMA_LIBRARY") or os.path.join(_HERE, "libgma.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "gma.h")

GMA_F32, GMA_BF16 = 0, 1
GMA_PROJ_F32, GMA_PROJ_SPLIT_BF16, GMA_PROJ_FUSED_BF16 = 0, 1, 2
GMA_OK, GMA_ERR_INVALID_ARG, GMA_ERR_UNSUPPORTED, GMA_ERR_WORKSPACE, GMA_ERR_HIP = range(5)


class GmaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s (%s)" % (message, status_name(status)))
        self.status = status


class gma_dims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("H", ctypes.c_int64), ("N", ctypes.c_int64),
                ("d_r", ctypes.c_int32), ("d_v", ctypes.c_int32), ("K", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("chunk", ctypes.c_int32)]


class gma_kernel_time(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int64),
                ("total_ms", ctypes.c_double)]


_lib = None


def load():
    """Load libgma.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libgma.so not found at %s; build it with "
                           "`python -m gaussian_mixture_sequence_gma_amd.build`" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P, S = ctypes.c_void_p, ctypes.c_size_t
    i32, f32 = ctypes.c_int, ctypes.c_float
    D = ctypes.POINTER(gma_dims)
    lib.gma_validate.argtypes = [D, f32, i32, ctypes.POINTER(P), i32, S, S]
    lib.gma_forward_workspace_bytes.argtypes = [D, i32, ctypes.POINTER(S)]
    lib.gma_forward.argtypes = [P, P, P, P, P, P, f32, i32, P, D, P, P, P, S, P]
    lib.gma_forward_noalloc.argtypes = [P, P, P, P, P, P, f32, i32, P, D, P, P, P]
    lib.gma_forward_reparam.argtypes = [P, P, P, P, P, P, f32, f32, i32, P, D, P, P, P, S, P]
    lib.gma_layer_workspace_bytes.argtypes = [D, ctypes.c_int32, i32, ctypes.POINTER(S)]
    lib.gma_layer_forward.argtypes = [P, P, P, P, ctypes.c_int32, P, P, P, f32, i32, P, D, P, P,
                                      P, S, P]
    lib.gma_layer_projection_layout.argtypes = [D, ctypes.c_int32, i32,
                                                ctypes.POINTER(ctypes.c_int32),
                                                ctypes.POINTER(S * 5)]
    lib.gma_responsibilities.argtypes = [P, P, P, P, D, P, P, P, S, P]
    lib.gma_prefix_state.argtypes = [P, P, P, P, P, P, P, D, P, P, S, P]
    lib.gma_decode_step.argtypes = [P, P, P, P, P, P, f32, P, P, P, D, P, P, P]
    lib.gma_reparameterize.argtypes = [P, P, f32, ctypes.c_int64, ctypes.c_int32,
                                       ctypes.c_int32, P, P, P]
    lib.gma_backward_workspace_bytes.argtypes = [D, i32, ctypes.POINTER(S)]
    lib.gma_backward.argtypes = [P, P, P, P, P, P, f32, i32, P, D, P, P, P, P, P, P, P, S, P]
    lib.gma_usage_workspace_bytes.argtypes = [D, ctypes.POINTER(S)]
    lib.gma_usage_stats.argtypes = [P, P, P, P, D, f32, P, P, P, P, P, S, P]
    lib.gma_status_string.argtypes = [i32]
    lib.gma_status_string.restype = ctypes.c_char_p
    lib.gma_last_error.argtypes = []
    lib.gma_last_error.restype = ctypes.c_char_p
    lib.gma_timing_enable.argtypes = [i32]
    lib.gma_timing_collect.argtypes = [ctypes.POINTER(gma_kernel_time), i32,
                                       ctypes.POINTER(ctypes.c_int)]
    for fn in ("gma_validate", "gma_forward_workspace_bytes", "gma_forward", "gma_forward_noalloc",
               "gma_forward_reparam",
               "gma_layer_workspace_bytes", "gma_layer_forward", "gma_layer_projection_layout",
               "gma_responsibilities", "gma_prefix_state", "gma_decode_step", "gma_reparameterize",
               "gma_usage_workspace_bytes", "gma_usage_stats",
               "gma_backward_workspace_bytes", "gma_backward",
               "gma_timing_enable", "gma_timing_collect"):
        getattr(lib, fn).restype = ctypes.c_int
    _lib = lib
    return lib


def declared_functions() -> List[str]:
    """Names of the functions include/gma.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w ]+?\*?\s*\b(gma_\w+)\s*\(", text, re.M)))


def status_name(status: int) -> str:
    return load().gma_status_string(int(status)).decode()


def _check(status: int):
    if status != GMA_OK:
        raise GmaError(status, load().gma_last_error().decode())


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_dims(B, H, N, d_r, d_v, K, dtype, chunk=0) -> gma_dims:
    return gma_dims(int(B), int(H), int(N), int(d_r), int(d_v), int(K), int(dtype), int(chunk))


# ---- C entry points ------------------------------------------------------------

def gma_validate(dims: gma_dims, eps: float, causal: int, ptrs=(), workspace_bytes: int = 0,
                 workspace_needed: int = 0) -> int:
    """Status of gma_validate (no exception): ptrs are tensors, ints or None."""
    arr = (ctypes.c_void_p * max(len(ptrs), 1))(*[_ptr(x) for x in ptrs])
    return load().gma_validate(ctypes.byref(dims), float(eps), int(causal),
                               arr if ptrs else None, len(ptrs), int(workspace_bytes),
                               int(workspace_needed))


def gma_forward_workspace_bytes(dims: gma_dims, causal: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load().gma_forward_workspace_bytes(ctypes.byref(dims), int(causal), ctypes.byref(n)))
    return n.value


def gma_forward(Q_X, K_X, V_X, mu, log_sigma2, log_pi, eps, causal, out, dims: gma_dims,
                assign_q=None, assign_k=None, workspace=None, workspace_bytes=0, stream=None):
    _check(load().gma_forward(_ptr(Q_X), _ptr(K_X), _ptr(V_X), _ptr(mu), _ptr(log_sigma2),
                              _ptr(log_pi), float(eps), int(causal), _ptr(out),
                              ctypes.byref(dims), _ptr(assign_q), _ptr(assign_k),
                              _ptr(workspace), int(workspace_bytes), _stream(stream)))


def gma_forward_reparam(Q_X, K_X, V_X, mu, omega, alpha, eps_sigma, eps, causal, out,
                        dims: gma_dims, assign_q=None, assign_k=None, workspace=None,
                        workspace_bytes=0, stream=None):
    _check(load().gma_forward_reparam(_ptr(Q_X), _ptr(K_X), _ptr(V_X), _ptr(mu), _ptr(omega),
                                      _ptr(alpha), float(eps_sigma), float(eps), int(causal),
                                      _ptr(out), ctypes.byref(dims), _ptr(assign_q),
                                      _ptr(assign_k), _ptr(workspace), int(workspace_bytes),
                                      _stream(stream)))


def gma_forward_noalloc(Q_X, K_X, V_X, mu, log_sigma2, log_pi, eps, causal, out, dims: gma_dims,
                        assign_q=None, assign_k=None, stream=None):
    _check(load().gma_forward_noalloc(_ptr(Q_X), _ptr(K_X), _ptr(V_X), _ptr(mu),
                                      _ptr(log_sigma2), _ptr(log_pi), float(eps), int(causal),
                                      _ptr(out), ctypes.byref(dims), _ptr(assign_q),
                                      _ptr(assign_k), _stream(stream)))


def gma_layer_workspace_bytes(dims: gma_dims, d_model: int, causal: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load().gma_layer_workspace_bytes(ctypes.byref(dims), int(d_model), int(causal),
                                            ctypes.byref(n)))
    return n.value


def gma_layer_forward(X, W_Q, W_K, W_V, d_model, mu, log_sigma2, log_pi, eps, causal, out,
                      dims: gma_dims, assign_q=None, assign_k=None, workspace=None,
                      workspace_bytes=0, stream=None):
    _check(load().gma_layer_forward(_ptr(X), _ptr(W_Q), _ptr(W_K), _ptr(W_V), int(d_model),
                                    _ptr(mu), _ptr(log_sigma2), _ptr(log_pi), float(eps),
                                    int(causal), _ptr(out), ctypes.byref(dims), _ptr(assign_q),
                                    _ptr(assign_k), _ptr(workspace), int(workspace_bytes),
                                    _stream(stream)))


def gma_layer_projection_layout(dims: gma_dims, d_model: int, causal: int):
    """(format, offsets): a GMA_PROJ_* code and the five byte offsets."""
    fmt = ctypes.c_int32(0)
    offs = (ctypes.c_size_t * 5)()
    _check(load().gma_layer_projection_layout(ctypes.byref(dims), int(d_model), int(causal),
                                              ctypes.byref(fmt), ctypes.byref(offs)))
    return fmt.value, list(offs)


def gma_responsibilities(X_r, mu, log_sigma2, log_pi, dims: gma_dims, gamma=None, assign=None,
                         workspace=None, workspace_bytes=0, stream=None):
    _check(load().gma_responsibilities(_ptr(X_r), _ptr(mu), _ptr(log_sigma2), _ptr(log_pi),
                                       ctypes.byref(dims), _ptr(gamma), _ptr(assign),
                                       _ptr(workspace), int(workspace_bytes), _stream(stream)))


def gma_prefix_state(K_X, V_X, mu, log_sigma2, log_pi, state_v, state_z, dims: gma_dims,
                     assign_k=None, workspace=None, workspace_bytes=0, stream=None):
    _check(load().gma_prefix_state(_ptr(K_X), _ptr(V_X), _ptr(mu), _ptr(log_sigma2),
                                   _ptr(log_pi), _ptr(state_v), _ptr(state_z),
                                   ctypes.byref(dims), _ptr(assign_k), _ptr(workspace),
                                   int(workspace_bytes), _stream(stream)))


def gma_decode_step(q, k, v, mu, log_sigma2, log_pi, eps, state_v, state_z, out,
                    dims: gma_dims, assign_q=None, assign_k=None, stream=None):
    _check(load().gma_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(mu), _ptr(log_sigma2),
                                  _ptr(log_pi), float(eps), _ptr(state_v), _ptr(state_z),
                                  _ptr(out), ctypes.byref(dims), _ptr(assign_q),
                                  _ptr(assign_k), _stream(stream)))


def gma_backward_workspace_bytes(dims: gma_dims, causal: int = 0) -> int:
    n = ctypes.c_size_t(0)
    _check(load().gma_backward_workspace_bytes(ctypes.byref(dims), int(causal), ctypes.byref(n)))
    return n.value


def gma_backward(Q_X, K_X, V_X, mu, log_sigma2, log_pi, eps, causal, dO, dims: gma_dims, dQ, dK,
                 dV, dmu, dlog_sigma2, dlog_pi, workspace=None, workspace_bytes=0, stream=None):
    _check(load().gma_backward(_ptr(Q_X), _ptr(K_X), _ptr(V_X), _ptr(mu), _ptr(log_sigma2),
                               _ptr(log_pi), float(eps), int(causal), _ptr(dO),
                               ctypes.byref(dims), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(dmu),
                               _ptr(dlog_sigma2), _ptr(dlog_pi), _ptr(workspace),
                               int(workspace_bytes), _stream(stream)))


def gma_usage_workspace_bytes(dims: gma_dims) -> int:
    n = ctypes.c_size_t(0)
    _check(load().gma_usage_workspace_bytes(ctypes.byref(dims), ctypes.byref(n)))
    return n.value


def gma_usage_stats(X_r, mu, log_sigma2, log_pi, dims: gma_dims, util_threshold, counts=None,
                    mean_gamma=None, utilization=None, head_stats=None, workspace=None,
                    workspace_bytes=0, stream=None):
    _check(load().gma_usage_stats(_ptr(X_r), _ptr(mu), _ptr(log_sigma2), _ptr(log_pi),
                                  ctypes.byref(dims), float(util_threshold), _ptr(counts),
                                  _ptr(mean_gamma), _ptr(utilization), _ptr(head_stats),
                                  _ptr(workspace), int(workspace_bytes), _stream(stream)))


def gma_reparameterize(omega, alpha, eps_sigma, H, K, d_r, log_sigma2, log_pi, stream=None):
    _check(load().gma_reparameterize(_ptr(omega), _ptr(alpha), float(eps_sigma), int(H), int(K),
                                     int(d_r), _ptr(log_sigma2), _ptr(log_pi), _stream(stream)))


def gma_status_string(status: int) -> str:
    return status_name(status)


def gma_last_error() -> str:
    return load().gma_last_error().decode()


def gma_timing_enable(enable: bool):
    _check(load().gma_timing_enable(1 if enable else 0))


def gma_timing_collect(max_entries: int = 32) -> List[Tuple[str, int, float]]:
    arr = (gma_kernel_time * max_entries)()
    cnt = ctypes.c_int(0)
    _check(load().gma_timing_collect(arr, max_entries, ctypes.byref(cnt)))
    return [(arr[i].name.decode(), int(arr[i].launches), float(arr[i].total_ms))
            for i in range(min(cnt.value, max_entries))]
