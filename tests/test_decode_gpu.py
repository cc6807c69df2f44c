"""GPU parity of the causal decode step and the prefix state against the oracle.

gma_decode_step appends one token per sequence to a carried state (S, z)
("Causal GMA", the prefix memories and Eq. 8b); gma_prefix_state builds that
state from a prefix of keys and values (Eqs. 5-6 over the prefix).  Both go
through the C ABI; the oracle is oracle.decode_step and oracle.forward.

Tolerances: outputs as the forward (row-wise, fp32 1e-4, bf16 2e-2: the bf16
output is rounded to bf16); the fp32 state S' and z' row-wise 1e-4 (the step
adds gamma^K v^T to S in fp32); the prefix state from the bf16 write path
2e-2 (its key responsibilities enter the MFMA in bf16), fp32 1e-4.
"""
import numpy as np
import pytest
import torch

import oracle
from gaussian_mixture_sequence_gma_amd import api, inputs
from tests.parity import TOL, check_assign, rowwise_rel_err, upload

pytestmark = pytest.mark.gpu

STATE_TOL = 1e-4


def _wl(B, H, d_r, d_v, K, dtype, state_len=256, skew=False, N=1):
    kw = dict(mu_var=1.5, ls2_lo=-1.5, ls2_hi=0.5, logit_var=2.0) if skew else {}
    return inputs.Workload("decode_case", B, H, N, d_r, d_v, K, dtype, True,
                           state_len=state_len, **kw)


def _decode_once(w, seed):
    gen = inputs.generate(w, seed)
    dev = upload(gen)
    S = torch.from_numpy(gen["S"]).cuda()
    z = torch.from_numpy(gen["z"]).cuda()
    out, aq, ak = api.decode_step(dev["Q"], dev["K"], dev["V"], dev["mu"], dev["log_sigma2"],
                                  dev["log_pi"], S, z, w.eps, assign=True)
    torch.cuda.synchronize()
    ref = oracle.decode_step(gen["S"], gen["z"], gen["Q"].f32[:, :, 0], gen["K"].f32[:, :, 0],
                             gen["V"].f32[:, :, 0], gen["mu"], gen["log_sigma2"],
                             gen["log_pi"], w.eps)
    return gen, ref, out.float().cpu().numpy()[:, :, 0], S.cpu().numpy(), z.cpu().numpy(), \
        aq.cpu().numpy(), ak.cpu().numpy()


@pytest.mark.parametrize("B,H,d_r,d_v,K,dtype,skew", [
    (2, 3, 16, 32, 8, "f32", False),
    (3, 2, 64, 64, 64, "f32", False),
    (2, 2, 128, 16, 100, "f32", False),      # ragged K, eight lanes per component
    (1, 4, 32, 128, 1, "f32", False),        # one component: a running mean
    (2, 4, 64, 128, 128, "bf16", True),      # the long-context head shape
    (4, 2, 16, 64, 65, "bf16", False),       # K one past a wave's 64 components
    (1, 1, 128, 128, 128, "f32", True),
    (2, 2, 64, 64, 200, "f32", False),       # K above 128: four components per lane
    (2, 3, 64, 128, 256, "bf16", True),      # the language model's K = 256
    (1, 2, 32, 32, 129, "bf16", False),
])
def test_decode_step_matches_oracle(B, H, d_r, d_v, K, dtype, skew):
    w = _wl(B, H, d_r, d_v, K, dtype, skew=skew)
    gen, ref, out, S, z, aq, ak = _decode_once(w, 7)
    e_out = rowwise_rel_err(out, ref["out"])
    e_S = rowwise_rel_err(S, ref["S"])
    e_z = rowwise_rel_err(z, ref["z"])
    print("decode %s: out %.2e  S %.2e  z %.2e" % ((B, H, d_r, d_v, K, dtype), e_out, e_S, e_z))
    assert e_out <= TOL[dtype]
    assert e_S <= STATE_TOL
    assert e_z <= STATE_TOL
    check_assign(aq[:, :, None], ref["assign_q"][:, :, None], gen["Q"].f32, gen, dtype,
                 "decode assign_q")
    check_assign(ak[:, :, None], ref["assign_k"][:, :, None], gen["K"].f32, gen, dtype,
                 "decode assign_k")


def test_decode_full_size_serving_batch():
    """The decode workload as the benchmark launches it (B64 H32 d_r64 d_v128
    K128, bf16, carried state of a 4096-token prefix), every sequence checked."""
    w = inputs.WORKLOADS["decode_bf16"]
    gen, ref, out, S, z, aq, ak = _decode_once(w, 0)
    e_out = rowwise_rel_err(out, ref["out"])
    e_S = rowwise_rel_err(S, ref["S"])
    e_z = rowwise_rel_err(z, ref["z"])
    print("decode full size: out %.2e  S %.2e  z %.2e" % (e_out, e_S, e_z))
    assert e_out <= TOL["bf16"] and e_S <= STATE_TOL and e_z <= STATE_TOL
    check_assign(aq[:, :, None], ref["assign_q"][:, :, None], gen["Q"].f32, gen, "bf16",
                 "decode assign_q")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_from_empty_state_steps_through_causal_forward(dtype):
    """T steps from S = 0, z = 0 reproduce the causal forward's first T rows."""
    B, H, N, d_r, d_v, K = 2, 3, 24, 32, 64, 40
    w = inputs.Workload("steps", B, H, N, d_r, d_v, K, dtype, True)
    gen = inputs.generate(w, 3)
    dev = upload(gen)
    S = torch.zeros((B, H, K, d_v), dtype=torch.float32, device="cuda")
    z = torch.zeros((B, H, K), dtype=torch.float32, device="cuda")
    outs, aqs = [], []
    for i in range(N):
        o, aq, _ = api.decode_step(dev["Q"][:, :, i:i + 1].contiguous(),
                                   dev["K"][:, :, i:i + 1].contiguous(),
                                   dev["V"][:, :, i:i + 1].contiguous(), dev["mu"],
                                   dev["log_sigma2"], dev["log_pi"], S, z, w.eps, assign=True)
        outs.append(o)
        aqs.append(aq)
    torch.cuda.synchronize()
    got = torch.cat(outs, 2).float().cpu().numpy()
    ref = oracle.forward(gen["Q"].f32, gen["K"].f32, gen["V"].f32, gen["mu"], gen["log_sigma2"],
                         gen["log_pi"], w.eps, True, want_assign=True)
    e = rowwise_rel_err(got, ref["out"])
    print("decode steps %s: %.2e" % (dtype, e))
    assert e <= TOL[dtype]
    check_assign(torch.stack(aqs, 2).cpu().numpy(), ref["assign_q"], gen["Q"].f32, gen, dtype,
                 "steps assign_q")
    # the state after N steps is the latent memory of the whole sequence
    lat = oracle.forward(gen["Q"].f32, gen["K"].f32, gen["V"].f32, gen["mu"],
                         gen["log_sigma2"], gen["log_pi"], w.eps, False, want_latent=True)
    assert rowwise_rel_err(S.cpu().numpy(), lat["vtilde"]) <= STATE_TOL
    assert rowwise_rel_err(z.cpu().numpy(), lat["z"]) <= STATE_TOL


@pytest.mark.parametrize("B,H,N,d_r,d_v,K,dtype,skew", [
    (2, 3, 300, 32, 64, 40, "f32", False),
    (1, 2, 77, 16, 16, 1, "f32", False),
    (1, 4, 1000, 64, 128, 128, "bf16", True),
    (2, 2, 513, 128, 32, 100, "bf16", False),
    (1, 2, 5, 64, 64, 64, "bf16", False),
])
def test_prefix_state_matches_oracle_latent(B, H, N, d_r, d_v, K, dtype, skew):
    kw = dict(mu_var=1.5, ls2_lo=-1.5, ls2_hi=0.5, logit_var=2.0) if skew else {}
    w = inputs.Workload("prefix", B, H, N, d_r, d_v, K, dtype, False, **kw)
    gen = inputs.generate(w, 11)
    dev = upload(gen)
    S, z, ak = api.prefix_state(dev["K"], dev["V"], dev["mu"], dev["log_sigma2"],
                                dev["log_pi"], assign=True)
    torch.cuda.synchronize()
    ref = oracle.forward(gen["Q"].f32, gen["K"].f32, gen["V"].f32, gen["mu"], gen["log_sigma2"],
                         gen["log_pi"], w.eps, False, want_latent=True, want_assign=True)
    tol = TOL[dtype]
    e_S = rowwise_rel_err(S.cpu().numpy(), ref["vtilde"])
    e_z = rowwise_rel_err(z.cpu().numpy(), ref["z"])
    print("prefix %s: S %.2e  z %.2e" % ((B, H, N, d_r, d_v, K, dtype), e_S, e_z))
    assert e_S <= tol and e_z <= tol
    check_assign(ak.cpu().numpy(), ref["assign_k"], gen["K"].f32, gen, dtype, "prefix assign_k")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_then_decode_matches_causal_forward(dtype):
    """State of the first N-1 tokens, then one decode step at position N-1,
    equals the causal forward's last row."""
    B, H, N, d_r, d_v, K = 2, 4, 200, 64, 64, 64
    w = inputs.Workload("prefill", B, H, N, d_r, d_v, K, dtype, True)
    gen = inputs.generate(w, 5)
    dev = upload(gen)
    S, z = api.prefix_state(dev["K"][:, :, :N - 1].contiguous(),
                            dev["V"][:, :, :N - 1].contiguous(), dev["mu"], dev["log_sigma2"],
                            dev["log_pi"])
    o = api.decode_step(dev["Q"][:, :, N - 1:].contiguous(), dev["K"][:, :, N - 1:].contiguous(),
                        dev["V"][:, :, N - 1:].contiguous(), dev["mu"], dev["log_sigma2"],
                        dev["log_pi"], S, z, w.eps)
    torch.cuda.synchronize()
    ref = oracle.forward(gen["Q"].f32, gen["K"].f32, gen["V"].f32, gen["mu"], gen["log_sigma2"],
                         gen["log_pi"], w.eps, True)["out"][:, :, N - 1:]
    e = rowwise_rel_err(o.float().cpu().numpy(), ref)
    print("prefill + decode %s: %.2e" % (dtype, e))
    assert e <= TOL[dtype]


def test_prefix_state_full_size_sampled_heads():
    """The carried state of the long-context prefix (B1 H32 N32768 d_r64 d_v128
    K128, bf16) in one launch; heads 0 and 1 against the oracle's latent memory
    (heads are independent)."""
    w = inputs.WORKLOADS["long_bidir_bf16"]
    gen = inputs.generate(w, 0)
    dev = upload(gen)
    S, z = api.prefix_state(dev["K"], dev["V"], dev["mu"], dev["log_sigma2"], dev["log_pi"])
    torch.cuda.synchronize()
    hs = slice(0, 2)
    ref = oracle.forward(gen["Q"].f32[:, hs], gen["K"].f32[:, hs], gen["V"].f32[:, hs],
                         gen["mu"][hs], gen["log_sigma2"][hs], gen["log_pi"][hs], w.eps, False,
                         want_latent=True)
    e_S = rowwise_rel_err(S[:, hs].cpu().numpy(), ref["vtilde"])
    e_z = rowwise_rel_err(z[:, hs].cpu().numpy(), ref["z"])
    print("prefix full size: S %.2e  z %.2e" % (e_S, e_z))
    assert e_S <= TOL["bf16"] and e_z <= TOL["bf16"]
