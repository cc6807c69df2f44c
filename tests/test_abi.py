"""C ABI checks that need no GPU: the library loads, exports what include/gma.h
declares, and rejects bad arguments before any launch."""
import ctypes
import math

import pytest

from gaussian_mixture_sequence_gma_amd import binding as B

pytestmark = pytest.mark.skipif(not __import__("os").path.exists(B.LIB_PATH),
                                reason="libgma.so not built")


def test_exports_every_declared_function():
    lib = B.load()
    names = B.declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n


def _dims(**kw):
    base = dict(B=1, H=2, N=100, d_r=64, d_v=64, K=64, dtype=B.GMA_BF16, chunk=0)
    base.update(kw)
    return B.make_dims(**base)


@pytest.mark.parametrize("kw,eps,causal,status", [
    ({}, 1e-6, 0, B.GMA_OK),
    ({}, 0.0, 1, B.GMA_OK),
    ({"B": 0}, 1e-6, 0, B.GMA_ERR_INVALID_ARG),
    ({"N": 0}, 1e-6, 0, B.GMA_ERR_INVALID_ARG),
    ({"K": 0}, 1e-6, 0, B.GMA_ERR_INVALID_ARG),
    ({"d_r": 0}, 1e-6, 0, B.GMA_ERR_INVALID_ARG),
    ({"dtype": 7}, 1e-6, 0, B.GMA_ERR_INVALID_ARG),
    ({"chunk": -1}, 1e-6, 0, B.GMA_ERR_INVALID_ARG),
    ({}, -1e-6, 0, B.GMA_ERR_INVALID_ARG),
    ({}, float("nan"), 0, B.GMA_ERR_INVALID_ARG),
    ({}, float("inf"), 0, B.GMA_ERR_INVALID_ARG),
    ({}, 1e-6, 2, B.GMA_ERR_INVALID_ARG),
    ({"d_r": 48}, 1e-6, 0, B.GMA_ERR_UNSUPPORTED),
    ({"d_v": 256}, 1e-6, 0, B.GMA_ERR_UNSUPPORTED),
    ({"K": 257}, 1e-6, 0, B.GMA_ERR_UNSUPPORTED),
    ({"K": 256}, 1e-6, 0, B.GMA_OK),
    ({"chunk": 32}, 1e-6, 1, B.GMA_ERR_UNSUPPORTED),
    ({"B": 300, "H": 300}, 1e-6, 0, B.GMA_ERR_UNSUPPORTED),
])
def test_validate(kw, eps, causal, status):
    assert B.gma_validate(_dims(**kw), eps, causal) == status
    if status != B.GMA_OK:
        assert B.gma_last_error() != ""


def test_validate_pointers_and_workspace():
    d = _dims()
    assert B.gma_validate(d, 1e-6, 0, ptrs=(1 << 20, 1 << 21), workspace_bytes=512,
                          workspace_needed=512) == B.GMA_OK
    assert B.gma_validate(d, 1e-6, 0, ptrs=(1 << 20, None)) == B.GMA_ERR_INVALID_ARG
    assert "pointer 1" in B.gma_last_error()
    assert B.gma_validate(d, 1e-6, 0, ptrs=((1 << 20) + 8,)) == B.GMA_ERR_INVALID_ARG
    assert B.gma_validate(d, 1e-6, 0, workspace_bytes=100,
                          workspace_needed=101) == B.GMA_ERR_WORKSPACE
    # the shape is checked first
    assert B.gma_validate(_dims(K=0), 1e-6, 0, ptrs=(None,)) == B.GMA_ERR_INVALID_ARG
    # fp32 causal beyond the scan kernel's LDS budget runs on the product path,
    # whose chunk products are batched over B*H*ceil(N/64) <= 65535
    big = B.make_dims(1, 1, 333, 64, 128, 128, B.GMA_F32)
    assert B.gma_validate(big, 1e-6, 1) == B.GMA_OK
    long = B.make_dims(1, 2, 64 * 40000, 64, 128, 128, B.GMA_F32)
    assert B.gma_validate(long, 1e-6, 1) == B.GMA_ERR_UNSUPPORTED
    assert "65535" in B.gma_last_error()
    assert B.gma_validate(long, 1e-6, 0) == B.GMA_OK


def test_workspace_query_and_errors():
    n0 = B.gma_forward_workspace_bytes(_dims(), 0)
    n1 = B.gma_forward_workspace_bytes(_dims(N=100000), 0)
    assert 0 < n0 < n1 and n0 % 256 == 0
    assert B.gma_forward_workspace_bytes(_dims(), 1) > 0
    with pytest.raises(B.GmaError) as ei:
        B.gma_forward_workspace_bytes(_dims(K=300), 0)
    assert ei.value.status == B.GMA_ERR_UNSUPPORTED
    assert B.gma_layer_workspace_bytes(_dims(), 1024, 1) > B.gma_forward_workspace_bytes(_dims(), 1)
    with pytest.raises(B.GmaError):
        B.gma_layer_workspace_bytes(_dims(), 1000, 1)


# Fake, never-dereferenced addresses: every call below must fail validation
# before any HIP call is made.
A16 = 1 << 20
MIS = A16 + 4


def _fwd(**over):
    args = dict(Q_X=A16, K_X=A16, V_X=A16, mu=A16, log_sigma2=A16, log_pi=A16, eps=1e-6,
                causal=0, out=A16, dims=_dims(), assign_q=None, assign_k=None,
                workspace=A16, workspace_bytes=0, stream=0)
    args.update(over)
    with pytest.raises(B.GmaError) as ei:
        B.gma_forward(**args)
    return ei.value.status


def test_forward_rejects_before_launch():
    assert _fwd(Q_X=None) == B.GMA_ERR_INVALID_ARG
    assert _fwd(out=None) == B.GMA_ERR_INVALID_ARG
    assert _fwd(workspace=None) == B.GMA_ERR_INVALID_ARG
    assert _fwd(V_X=MIS) == B.GMA_ERR_INVALID_ARG
    assert _fwd(eps=-1.0) == B.GMA_ERR_INVALID_ARG
    assert _fwd(dims=_dims(K=300)) == B.GMA_ERR_UNSUPPORTED
    assert _fwd(workspace_bytes=16) == B.GMA_ERR_WORKSPACE


def _fwd_reparam(**over):
    args = dict(Q_X=A16, K_X=A16, V_X=A16, mu=A16, omega=A16, alpha=A16, eps_sigma=1e-4,
                eps=1e-6, causal=0, out=A16, dims=_dims(), assign_q=None, assign_k=None,
                workspace=A16, workspace_bytes=0, stream=0)
    args.update(over)
    with pytest.raises(B.GmaError) as ei:
        B.gma_forward_reparam(**args)
    return ei.value.status


def test_forward_reparam_rejects_before_launch():
    assert _fwd_reparam(omega=None) == B.GMA_ERR_INVALID_ARG
    assert _fwd_reparam(alpha=None) == B.GMA_ERR_INVALID_ARG
    assert _fwd_reparam(eps_sigma=0.0) == B.GMA_ERR_INVALID_ARG
    assert _fwd_reparam(eps_sigma=float("nan")) == B.GMA_ERR_INVALID_ARG
    assert _fwd_reparam(omega=A16 + 2) == B.GMA_ERR_INVALID_ARG
    assert _fwd_reparam(dims=_dims(K=300)) == B.GMA_ERR_UNSUPPORTED
    assert _fwd_reparam(workspace_bytes=16) == B.GMA_ERR_WORKSPACE


def test_layer_and_resp_reject_before_launch():
    d = _dims()
    with pytest.raises(B.GmaError) as ei:
        B.gma_layer_forward(A16, A16, A16, A16, 1000, A16, A16, A16, 1e-6, 1, A16, d,
                            workspace=A16, workspace_bytes=1 << 40, stream=0)
    assert ei.value.status == B.GMA_ERR_UNSUPPORTED
    with pytest.raises(B.GmaError) as ei:
        B.gma_layer_forward(A16, A16, A16, A16, 1024, A16, A16, A16, 1e-6, 1, A16,
                            _dims(dtype=B.GMA_F32), workspace=A16, workspace_bytes=1 << 40,
                            stream=0)
    assert ei.value.status == B.GMA_ERR_UNSUPPORTED
    with pytest.raises(B.GmaError) as ei:
        B.gma_layer_forward(A16, A16, A16, A16, 1024, A16, A16, A16, 1e-6, 1, A16, d,
                            workspace=A16, workspace_bytes=64, stream=0)
    assert ei.value.status == B.GMA_ERR_WORKSPACE
    with pytest.raises(B.GmaError) as ei:
        B.gma_responsibilities(None, A16, A16, A16, d, workspace=A16, workspace_bytes=1 << 40,
                               stream=0)
    assert ei.value.status == B.GMA_ERR_INVALID_ARG


def test_status_strings():
    for s in range(5):
        assert B.gma_status_string(s).startswith("GMA_")
    assert "unknown" in B.gma_status_string(99)


def test_timing_collect_empty():
    B.gma_timing_enable(True)
    B.gma_timing_enable(False)
    assert B.gma_timing_collect() == []


@pytest.mark.parametrize("causal", [0, 1])
@pytest.mark.parametrize("kw,fmts", [
    # bf16 token-owner kernels take split routing vectors: split bf16
    # projections; d_r = 64 and at most 64 components: the projection
    # epilogue forms the responsibilities (only V_X is kept)
    ({}, (B.GMA_PROJ_FUSED_BF16, B.GMA_PROJ_FUSED_BF16)),
    ({"K": 32, "N": 16384}, (B.GMA_PROJ_FUSED_BF16, B.GMA_PROJ_FUSED_BF16)),
    ({"K": 128, "d_v": 128}, (B.GMA_PROJ_SPLIT_BF16, B.GMA_PROJ_SPLIT_BF16)),
    ({"d_r": 32, "K": 20}, (B.GMA_PROJ_SPLIT_BF16, B.GMA_PROJ_SPLIT_BF16)),
    # d_r = 128 exceeds the token-owner kernels: fp32 projections, fp32 path
    ({"d_r": 128}, (B.GMA_PROJ_F32, B.GMA_PROJ_F32)),
])
def test_layer_projection_layout(kw, fmts, causal):
    d = _dims(**kw)
    got, offs = B.gma_layer_projection_layout(d, 256, causal)
    total = B.gma_layer_workspace_bytes(d, 256, causal)
    assert got == fmts[causal]
    T = d.B * d.H * d.N
    if got == B.GMA_PROJ_F32:
        sizes = [4 * T * d.d_r, 4 * T * d.d_r, 4 * T * d.d_v]
        used = offs[:3]
        assert offs[3] == offs[4] == 0
    elif got == B.GMA_PROJ_FUSED_BF16:
        # V_X, then the queries' exponentials (32 or 64 components) at the tail
        sizes = [2 * T * d.d_v]
        used = offs[4:]
        assert offs[0] == offs[1] == offs[2] == offs[3] == 0
        kc = 32 if d.K <= 32 else 64
        assert used[0] > 0 and used[0] % 16 == 0
        assert total - (used[0] + sizes[0]) >= 2 * T * kc
        return
    else:
        sizes = [2 * T * d.d_r] * 4 + [2 * T * d.d_v]
        used = offs
    # arrays in order, 16-byte aligned, not overlapping, inside the workspace
    for i, (o, n) in enumerate(zip(used, sizes)):
        assert o % 16 == 0
        assert o + n <= total
        if i + 1 < len(used):
            assert o + n <= used[i + 1]
    # the projections fill the tail of the workspace, after the GMA part
    assert used[0] > 0
    assert total - (used[-1] + sizes[-1]) < 256


def test_layer_projection_layout_errors():
    fmt, offs = B.gma_layer_projection_layout(_dims(), 256, 0)
    assert fmt in (B.GMA_PROJ_F32, B.GMA_PROJ_SPLIT_BF16, B.GMA_PROJ_FUSED_BF16)
    with pytest.raises(B.GmaError) as ei:
        B.gma_layer_projection_layout(_dims(), 100, 0)          # d_model not a multiple of 64
    assert ei.value.status == B.GMA_ERR_UNSUPPORTED
    with pytest.raises(B.GmaError) as ei:
        B.gma_layer_projection_layout(_dims(dtype=B.GMA_F32), 256, 0)
    assert ei.value.status == B.GMA_ERR_UNSUPPORTED
    lib = B.load()
    out = (ctypes.c_size_t * 5)()
    assert lib.gma_layer_projection_layout(ctypes.byref(_dims()), 256, 0, None,
                                           ctypes.byref(out)) == B.GMA_ERR_INVALID_ARG


def _decode(**over):
    args = dict(q=A16, k=A16, v=A16, mu=A16, log_sigma2=A16, log_pi=A16, eps=1e-6,
                state_v=A16, state_z=A16, out=A16, dims=_dims(N=1), assign_q=None,
                assign_k=None, stream=0)
    args.update(over)
    with pytest.raises(B.GmaError) as ei:
        B.gma_decode_step(**args)
    return ei.value.status


def test_decode_step_rejects_before_launch():
    assert _decode(dims=_dims(N=2)) == B.GMA_ERR_INVALID_ARG      # one token per sequence
    assert _decode(q=None) == B.GMA_ERR_INVALID_ARG
    assert _decode(state_v=None) == B.GMA_ERR_INVALID_ARG
    assert _decode(state_z=None) == B.GMA_ERR_INVALID_ARG
    assert _decode(out=None) == B.GMA_ERR_INVALID_ARG
    assert _decode(state_v=A16 + 4) == B.GMA_ERR_INVALID_ARG     # 16-byte aligned
    assert _decode(assign_k=A16 + 2) == B.GMA_ERR_INVALID_ARG
    # the chunk length does not apply to a decode step: with chunk = 32 the
    # call fails on the NULL output, not on the chunk
    assert _decode(dims=_dims(N=1, chunk=32), out=None) == B.GMA_ERR_INVALID_ARG
    assert "NULL" in B.gma_last_error()
    assert _decode(eps=float("nan")) == B.GMA_ERR_INVALID_ARG
    assert _decode(dims=_dims(N=1, K=257)) == B.GMA_ERR_UNSUPPORTED
    assert _decode(dims=_dims(N=1, d_v=48)) == B.GMA_ERR_UNSUPPORTED
    assert "N = 1" in (lambda: (_decode(dims=_dims(N=3)), B.gma_last_error())[1])()


def _prefix(**over):
    args = dict(K_X=A16, V_X=A16, mu=A16, log_sigma2=A16, log_pi=A16, state_v=A16,
                state_z=A16, dims=_dims(), assign_k=None, workspace=A16,
                workspace_bytes=1 << 40, stream=0)
    args.update(over)
    with pytest.raises(B.GmaError) as ei:
        B.gma_prefix_state(**args)
    return ei.value.status


def test_prefix_state_rejects_before_launch():
    assert _prefix(K_X=None) == B.GMA_ERR_INVALID_ARG
    assert _prefix(state_z=None) == B.GMA_ERR_INVALID_ARG
    assert _prefix(workspace=None) == B.GMA_ERR_INVALID_ARG
    assert _prefix(state_v=A16 + 8) == B.GMA_ERR_INVALID_ARG
    assert _prefix(dims=_dims(K=0)) == B.GMA_ERR_INVALID_ARG
    assert _prefix(dims=_dims(d_r=8)) == B.GMA_ERR_UNSUPPORTED
    assert _prefix(workspace_bytes=32) == B.GMA_ERR_WORKSPACE
    # the forward's bidirectional workspace is enough
    n = B.gma_forward_workspace_bytes(_dims(), 0)
    assert _prefix(workspace_bytes=n - 1) == B.GMA_ERR_WORKSPACE


def test_reparameterize_rejects_before_launch():
    def st(**over):
        args = dict(omega=A16, alpha=A16, eps_sigma=1e-4, H=2, K=8, d_r=16, log_sigma2=A16,
                    log_pi=A16, stream=0)
        args.update(over)
        with pytest.raises(B.GmaError) as ei:
            B.gma_reparameterize(**args)
        return ei.value.status
    assert st(omega=None) == B.GMA_ERR_INVALID_ARG
    assert st(log_pi=None) == B.GMA_ERR_INVALID_ARG
    assert st(alpha=A16 + 2) == B.GMA_ERR_INVALID_ARG
    assert st(eps_sigma=0.0) == B.GMA_ERR_INVALID_ARG
    assert st(eps_sigma=float("inf")) == B.GMA_ERR_INVALID_ARG
    assert st(K=0) == B.GMA_ERR_INVALID_ARG
    assert st(H=70000) == B.GMA_ERR_UNSUPPORTED
    assert st(H=65535, K=4096, d_r=4096) == B.GMA_ERR_UNSUPPORTED


def test_backward_rejects_before_launch():
    def st(**over):
        args = dict(Q_X=A16, K_X=A16, V_X=A16, mu=A16, log_sigma2=A16, log_pi=A16, eps=1e-6,
                    causal=0, dO=A16, dims=_dims(), dQ=A16, dK=A16, dV=A16, dmu=A16,
                    dlog_sigma2=A16, dlog_pi=A16, workspace=A16, workspace_bytes=1 << 50,
                    stream=0)
        args.update(over)
        with pytest.raises(B.GmaError) as ei:
            B.gma_backward(**args)
        return ei.value.status
    assert st(causal=2) == B.GMA_ERR_INVALID_ARG
    assert st(causal=1, dims=_dims(B=64, H=64, N=4096)) == B.GMA_ERR_UNSUPPORTED
    assert st(dO=None) == B.GMA_ERR_INVALID_ARG
    assert st(dmu=None) == B.GMA_ERR_INVALID_ARG
    assert st(dQ=MIS) == B.GMA_ERR_INVALID_ARG
    assert st(workspace_bytes=1024) == B.GMA_ERR_WORKSPACE
    assert st(dims=_dims(N=65535 * 64 + 1)) == B.GMA_ERR_UNSUPPORTED
    n = B.gma_backward_workspace_bytes(_dims(), 0)
    assert n > B.gma_forward_workspace_bytes(_dims(), 0)
    assert st(workspace_bytes=n - 1) == B.GMA_ERR_WORKSPACE
    assert B.gma_backward_workspace_bytes(_dims(N=100), 1) > B.gma_backward_workspace_bytes(
        _dims(N=100), 0)


def test_usage_stats_rejects_before_launch():
    def st(**over):
        args = dict(X_r=A16, mu=A16, log_sigma2=A16, log_pi=A16, dims=_dims(),
                    util_threshold=0.1, counts=None, mean_gamma=None, utilization=None,
                    head_stats=None, workspace=A16, workspace_bytes=1 << 40, stream=0)
        args.update(over)
        with pytest.raises(B.GmaError) as ei:
            B.gma_usage_stats(**args)
        return ei.value.status
    assert st(X_r=None) == B.GMA_ERR_INVALID_ARG
    assert st(workspace=None) == B.GMA_ERR_INVALID_ARG
    assert st(X_r=MIS) == B.GMA_ERR_INVALID_ARG
    assert st(counts=A16 + 2) == B.GMA_ERR_INVALID_ARG
    assert st(util_threshold=float("nan")) == B.GMA_ERR_INVALID_ARG
    assert st(dims=_dims(K=0)) == B.GMA_ERR_INVALID_ARG
    assert st(dims=_dims(d_r=24)) == B.GMA_ERR_UNSUPPORTED
    assert st(dims=_dims(B=65535, H=1, N=32769)) == B.GMA_ERR_UNSUPPORTED       # B*N >= 2^31
    assert "2^31" in B.gma_last_error()
    n = B.gma_usage_workspace_bytes(_dims())
    assert n >= B.gma_forward_workspace_bytes(_dims(), 0)
    assert st(workspace_bytes=n - 1) == B.GMA_ERR_WORKSPACE
