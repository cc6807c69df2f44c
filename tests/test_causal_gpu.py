"""GPU parity of the causal (prefix-scan) path against the fp64 oracle."""
import numpy as np
import pytest
import torch

from gaussian_mixture_sequence_gma_amd import api, inputs
from tests.parity import run_and_compare, rowwise_rel_err, upload

pytestmark = pytest.mark.gpu

W = inputs.WORKLOADS


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("name", ["tiny_bidir_f32", "lra_bidir_f32"])
def test_causal_variant_of_fp32_workloads(name):
    run_and_compare(W[name].with_(causal=True))


def test_lm_causal_bf16_full():
    run_and_compare(W["lm_causal_bf16"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_causal_several_chunks_per_span(dtype, seed):
    # B*H = 48 at N = 2048 gives spans of two 64-token chunks: the carried state
    # entering a span and the in-span update both matter (and the kernel's
    # start-of-span set-up runs concurrently with other waves' first chunk)
    w = W["lm_causal_bf16"].with_(N=2048, dtype=dtype)
    run_and_compare(w, seed=seed, heads=3)


def test_long_context_causal_bf16_heads_subset():
    w = W["long_bidir_bf16"].with_(causal=True)
    run_and_compare(w, rows=inputs.sample_rows(w.N, 512, seed=7), heads=4)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [1, 63, 65, 200, 1000, 3000])
def test_causal_ragged_lengths(dtype, N):
    run_and_compare(W["tiny_bidir_f32"].with_(N=N, dtype=dtype, B=2, H=3, causal=True))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("K", [1, 3, 17, 64, 100, 128])
def test_causal_component_counts(dtype, K):
    run_and_compare(W["tiny_bidir_f32"].with_(K=K, d_r=32, d_v=64, N=700, H=2, dtype=dtype,
                                              causal=True))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d_r,d_v,K", [(16, 16, 8), (16, 128, 40), (32, 32, 64),
                                       (128, 64, 40), (64, 128, 128), (128, 128, 64),
                                       (128, 64, 128)])
def test_causal_head_dims(dtype, d_r, d_v, K):
    # (fp32 with K > 64 and d_v = 128 exceeds the scan kernel's LDS and runs on
    # the product path)
    w = W["tiny_bidir_f32"].with_(d_r=d_r, d_v=d_v, K=K, N=333, dtype=dtype, causal=True)
    run_and_compare(w)


def test_causal_single_component_is_running_mean():
    w = W["tiny_bidir_f32"].with_(K=1, N=1500, H=2, causal=True)
    gen = inputs.generate(w, 3)
    dev = upload(gen)
    out = api.forward(dev["Q"], dev["K"], dev["V"], dev["mu"], dev["log_sigma2"],
                      dev["log_pi"], w.eps, True).cpu().numpy()
    V = gen["V"].f32.astype(np.float64)
    cnt = np.arange(1, w.N + 1, dtype=np.float64)[None, None, :, None]
    expect = np.cumsum(V, axis=2) / (cnt + w.eps)
    assert rowwise_rel_err(out, expect) < 1e-5


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_causal_ignores_future_tokens_bitwise(dtype):
    w = W["lm_causal_bf16"].with_(B=1, H=2, N=5000, dtype=dtype)
    gen = inputs.generate(w, 0)
    dev = upload(gen)
    base, aq0, _ = api.forward(dev["Q"], dev["K"], dev["V"], dev["mu"], dev["log_sigma2"],
                               dev["log_pi"], w.eps, True, assign=True)
    for i in (0, 63, 64, 1000, 4095, 4999):
        Q, K, V = dev["Q"].clone(), dev["K"].clone(), dev["V"].clone()
        g = torch.Generator(device="cuda").manual_seed(i)
        for t in (Q, K, V):
            t[:, :, i + 1:] = torch.randn(t[:, :, i + 1:].shape, generator=g, device="cuda",
                                          dtype=torch.float32).to(t.dtype)
        out, aq, _ = api.forward(Q, K, V, dev["mu"], dev["log_sigma2"], dev["log_pi"], w.eps,
                                 True, assign=True)
        assert torch.equal(out[:, :, :i + 1].view(torch.int16 if dtype == "bf16" else torch.int32),
                           base[:, :, :i + 1].view(torch.int16 if dtype == "bf16" else torch.int32))
        assert torch.equal(aq[:, :, :i + 1], aq0[:, :, :i + 1])


def test_causal_last_row_matches_bidirectional():
    w = W["lra_bidir_f32"].with_(B=1, H=4, N=3000)
    gen = inputs.generate(w, 2)
    dev = upload(gen)
    args = (dev["Q"], dev["K"], dev["V"], dev["mu"], dev["log_sigma2"], dev["log_pi"], w.eps)
    c = api.forward(*args, True).cpu().numpy()
    b = api.forward(*args, False).cpu().numpy()
    assert rowwise_rel_err(c[:, :, -1:], b[:, :, -1:]) < 1e-4


def test_causal_bitwise_deterministic():
    w = W["lm_causal_bf16"].with_(B=2, H=3, N=4000)
    gen = inputs.generate(w, 0)
    dev = upload(gen)
    outs = [api.forward(dev["Q"], dev["K"], dev["V"], dev["mu"], dev["log_sigma2"],
                        dev["log_pi"], w.eps, True).clone() for _ in range(3)]
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))
