"""The forward, the layer and the decode step captured in a HIP graph and replayed.

The library allocates nothing, never synchronises and records no memset, so a
caller can capture its launches (torch.cuda.graph drives hipStreamBeginCapture
on the capture stream, which the binding passes through the C ABI).  Each
replay is checked against the eager call on the same buffers: bit for bit,
since the kernels are the same and every reduction has a fixed order.  Eager
work and a synchronisation sit between replays, and the inputs are changed in
place between replays to show that the graph reads the live buffers.  One
replay per case is also checked against the oracle at the forward's tolerance.
"""
import pytest
import torch

import oracle
from gaussian_mixture_sequence_gma_amd import api, binding as B, inputs
from tests.parity import TOL, rowwise_rel_err, upload

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _fwd_ws(w):
    dims = B.make_dims(w.B, w.H, w.N, w.d_r, w.d_v, w.K, B.GMA_BF16 if w.dtype == "bf16"
                       else B.GMA_F32)
    return api.alloc_workspace(B.gma_forward_workspace_bytes(dims, int(w.causal)), "cuda")


@pytest.mark.parametrize("causal,dtype,d_v,K", [(False, "bf16", 128, 128), (True, "bf16", 128, 128),
                                                (False, "f32", 64, 64), (True, "f32", 64, 64)])
def test_forward_graph_replays_match_eager(causal, dtype, d_v, K):
    # N ragged against every tile and chunk size
    w = inputs.Workload("graph", 2, 4, 3001, 64, d_v, K, dtype, causal)
    gen = inputs.generate(w, 9)
    dev = upload(gen)
    ws = _fwd_ws(w)

    def run(out):
        return api.forward(dev["Q"], dev["K"], dev["V"], dev["mu"], dev["log_sigma2"],
                           dev["log_pi"], w.eps, causal, workspace=ws, out=out)

    eager = run(None)
    torch.cuda.synchronize()
    ref = oracle.forward(gen["Q"].f32, gen["K"].f32, gen["V"].f32, gen["mu"], gen["log_sigma2"],
                         gen["log_pi"], w.eps, causal)["out"]

    out = torch.empty_like(eager)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(out)
    V0 = dev["V"].clone()
    for r in range(REPLAYS):
        out.fill_(float("nan"))
        if r == REPLAYS - 1:
            # new values in place: the replay must see them
            dev["V"].copy_(torch.flip(V0, dims=[2]))
            expect = run(None)
        else:
            expect = eager
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, expect), "replay %d differs from the eager call" % r
        if r == 0:
            e = rowwise_rel_err(out.float().cpu().numpy(), ref)
            print("graph forward causal=%d %s: %.2e" % (causal, dtype, e))
            assert e <= TOL[dtype]


@pytest.mark.parametrize("causal", [True, False])
def test_layer_graph_replays_match_eager(causal):
    # the fused layer: projection with the responsibility epilogue, span
    # totals, then the scan (causal) or the reduction and read-out
    w = inputs.WORKLOADS["layer_causal_bf16"].with_(name="graph_layer", B=1, N=1000)
    gen = inputs.generate(w, 4)
    dev = upload(gen)

    def run(out):
        return api.layer_forward(dev["X"], dev["W_Q"], dev["W_K"], dev["W_V"], w.H, dev["mu"],
                                 dev["log_sigma2"], dev["log_pi"], w.eps, causal, out=out,
                                 workspace=ws)

    dims = B.make_dims(w.B, w.H, w.N, w.d_r, w.d_v, w.K, B.GMA_BF16)
    ws = api.alloc_workspace(B.gma_layer_workspace_bytes(dims, w.d_model, int(causal)), "cuda")
    eager = run(None)
    torch.cuda.synchronize()
    out = torch.empty_like(eager)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(out)
    for r in range(REPLAYS):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), "layer replay %d differs from the eager call" % r


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_loop_in_graph_matches_eager_steps(dtype):
    """A serving loop: one captured decode step, replayed once per token with
    the token copied into the graph's static input buffers; the outputs and the
    carried state match eager steps bit for bit and the causal forward within
    tolerance."""
    Bb, H, N, d_r, d_v, K = 3, 4, 12, 64, 128, 128
    w = inputs.Workload("graph_decode", Bb, H, N, d_r, d_v, K, dtype, True)
    gen = inputs.generate(w, 6)
    dev = upload(gen)
    tdt = dev["Q"].dtype

    # eager reference steps
    S_e = torch.zeros((Bb, H, K, d_v), dtype=torch.float32, device="cuda")
    z_e = torch.zeros((Bb, H, K), dtype=torch.float32, device="cuda")
    outs_e = []
    for i in range(N):
        outs_e.append(api.decode_step(dev["Q"][:, :, i:i + 1].contiguous(),
                                      dev["K"][:, :, i:i + 1].contiguous(),
                                      dev["V"][:, :, i:i + 1].contiguous(), dev["mu"],
                                      dev["log_sigma2"], dev["log_pi"], S_e, z_e, w.eps))
    torch.cuda.synchronize()

    # captured step on static buffers
    q = torch.zeros((Bb, H, 1, d_r), dtype=tdt, device="cuda")
    k = torch.zeros_like(q)
    v = torch.zeros((Bb, H, 1, d_v), dtype=tdt, device="cuda")
    o = torch.empty((Bb, H, 1, d_v), dtype=tdt, device="cuda")
    S = torch.zeros((Bb, H, K, d_v), dtype=torch.float32, device="cuda")
    z = torch.zeros((Bb, H, K), dtype=torch.float32, device="cuda")
    # one eager call before capture loads the library; then reset the state
    api.decode_step(q, k, v, dev["mu"], dev["log_sigma2"], dev["log_pi"], S, z, w.eps, out=o)
    torch.cuda.synchronize()
    S.zero_()
    z.zero_()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        api.decode_step(q, k, v, dev["mu"], dev["log_sigma2"], dev["log_pi"], S, z, w.eps, out=o)
    torch.cuda.synchronize()
    outs = []
    for i in range(N):
        q.copy_(dev["Q"][:, :, i:i + 1])
        k.copy_(dev["K"][:, :, i:i + 1])
        v.copy_(dev["V"][:, :, i:i + 1])
        g.replay()
        outs.append(o.clone())
        torch.cuda.synchronize()
        assert torch.equal(outs[-1], outs_e[i]), "decode replay at token %d differs" % i
    assert torch.equal(S, S_e) and torch.equal(z, z_e)
    ref = oracle.forward(gen["Q"].f32, gen["K"].f32, gen["V"].f32, gen["mu"], gen["log_sigma2"],
                         gen["log_pi"], w.eps, True)["out"]
    e = rowwise_rel_err(torch.cat(outs, 2).float().cpu().numpy(), ref)
    print("graph decode loop %s: %.2e" % (dtype, e))
    assert e <= TOL[dtype]
