"""Host-side argument checks of the Python entry points (no GPU needed).

Each call below has one inconsistency and must raise ValueError before
anything reaches the C library.  CPU tensors serve as stand-ins: shapes,
dtypes and contiguity are checked before the device, so a shape error is
reported as such; a call whose tensors are all consistent but on the CPU is
rejected for the device.
"""
import pytest
import torch

from gaussian_mixture_sequence_gma_amd import api

B, H, N, DR, DV, K = 2, 3, 10, 16, 32, 4
bf, f32 = torch.bfloat16, torch.float32


def t(*shape, dtype=f32):
    return torch.zeros(shape, dtype=dtype)


def fwd_args(**over):
    a = dict(Q=t(B, H, N, DR, dtype=bf), K=t(B, H, N, DR, dtype=bf), V=t(B, H, N, DV, dtype=bf),
             mu=t(H, K, DR), log_sigma2=t(H, K, DR), log_pi=t(H, K))
    a.update(over)
    return a


def bad_forward(**over):
    a = fwd_args(**over)
    kw = {k: a.pop(k) for k in ("out", "workspace") if k in a}
    with pytest.raises(ValueError) as e:
        api.forward(a["Q"], a["K"], a["V"], a["mu"], a["log_sigma2"], a["log_pi"], 1e-6, False,
                    **kw)
    return str(e.value)


@pytest.mark.parametrize("over,needle", [
    (dict(K=t(B, H, N - 1, DR, dtype=bf)), "K has shape"),
    (dict(V=t(B, H, N + 1, DV, dtype=bf)), "V has shape"),
    (dict(V=t(B, H, N, DV, dtype=f32)), "V has dtype"),
    (dict(Q=t(B, H, N, DR, dtype=torch.float16), K=t(B, H, N, DR, dtype=torch.float16),
          V=t(B, H, N, DV, dtype=torch.float16)), "unsupported dtype"),
    (dict(mu=t(H, K, DR, dtype=torch.float64)), "mu must be float32"),
    (dict(log_sigma2=t(H + 1, K, DR)), "log_sigma2 has shape"),
    (dict(log_pi=t(H, K + 1)), "log_pi has shape"),
    (dict(out=t(B, H, N, DV - 1, dtype=bf)), "out has shape"),
    (dict(out=t(B, H, N, DV, dtype=f32)), "out has dtype"),
    (dict(Q=t(B, H, DR, N, dtype=bf).transpose(2, 3)), "Q must be contiguous"),
    (dict(workspace=t(64, dtype=torch.float32)), "workspace has dtype"),
    (dict(), "must be a CUDA tensor"),
])
def test_forward_rejects(over, needle):
    assert needle in bad_forward(**over)


def test_layer_rejects():
    X = t(B, N, 64, dtype=bf)
    W = t(64, H * DR, dtype=bf)
    Wv = t(64, H * DV, dtype=bf)
    p = (t(H, K, DR), t(H, K, DR), t(H, K))
    with pytest.raises(ValueError, match="W_K has shape"):
        api.layer_forward(X, W, t(64, H * DR + 1, dtype=bf), Wv, H, *p)
    with pytest.raises(ValueError, match="multiples of H"):
        api.layer_forward(X, t(64, H * DR + 1, dtype=bf), W, Wv, H, *p)
    with pytest.raises(ValueError, match="W_V has dtype"):
        api.layer_forward(X, W, W, t(64, H * DV), H, *p)
    with pytest.raises(ValueError, match="CUDA"):
        api.layer_forward(X, W, W, Wv, H, *p)


def test_decode_rejects():
    q = t(B, H, 1, DR, dtype=bf)
    v = t(B, H, 1, DV, dtype=bf)
    p = (t(H, K, DR), t(H, K, DR), t(H, K))
    with pytest.raises(ValueError, match="S has shape"):
        api.decode_step(q, q, v, *p, t(B, H, K, DV + 1), t(B, H, K))
    with pytest.raises(ValueError, match="z has dtype"):
        api.decode_step(q, q, v, *p, t(B, H, K, DV), t(B, H, K, dtype=torch.float64))
    with pytest.raises(ValueError, match="k has shape"):
        api.decode_step(q, t(B, H, 2, DR, dtype=bf), v, *p, t(B, H, K, DV), t(B, H, K))


def test_other_entries_reject():
    p = (t(H, K, DR), t(H, K, DR), t(H, K))
    X = t(B, H, N, DR, dtype=bf)
    with pytest.raises(ValueError, match="log_pi has shape"):
        api.responsibilities(X, p[0], p[1], t(K, H))
    with pytest.raises(ValueError, match="mu has shape"):
        api.usage_stats(X, t(H, K, DR + 1), p[1], p[2])
    with pytest.raises(ValueError, match="V has shape"):
        api.prefix_state(X, t(B, H, N - 2, DV, dtype=bf), *p)
    with pytest.raises(ValueError, match="alpha has shape"):
        api.reparameterize(t(H, K, DR), t(H, K + 1))
    with pytest.raises(ValueError, match="dO has shape"):
        api.backward(X, X, t(B, H, N, DV, dtype=bf), *p, t(B, H, N, DV + 1, dtype=bf))
    with pytest.raises(ValueError, match="dO has dtype"):
        api.backward(X, X, t(B, H, N, DV, dtype=bf), *p, t(B, H, N, DV))


@pytest.mark.parametrize("over,needle", [
    (dict(omega=t(H, K + 1, DR)), "omega has shape"),
    (dict(alpha=t(H, K, dtype=torch.float64)), "alpha must be float32"),
    (dict(alpha=t(H + 1, K)), "alpha has shape"),
])
def test_forward_reparam_rejects(over, needle):
    a = dict(Q=t(B, H, N, DR, dtype=bf), K=t(B, H, N, DR, dtype=bf), V=t(B, H, N, DV, dtype=bf),
             mu=t(H, K, DR), omega=t(H, K, DR), alpha=t(H, K))
    a.update(over)
    with pytest.raises(ValueError) as e:
        api.forward_reparam(a["Q"], a["K"], a["V"], a["mu"], a["omega"], a["alpha"], 1e-4)
    assert needle in str(e.value)
