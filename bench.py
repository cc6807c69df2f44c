#!/usr/bin/env python3
"""Throughput of the GMA forward pass on one MI355X.

One step = one gma_forward call (prologue, latent write, partial reduction and
fused responsibility + read-out; or the causal scan) over one batch of synthetic
inputs already resident in HBM.  Default workload: the long-context
bidirectional case (B1 H32 N32768 d_r64 d_v128 K128, bf16 inputs, skewed
parameters).  Prints one JSON line.

Timing: W untimed warm-up steps, then K steps timed with events on the stream
(ms_per_step and value), then the same K steps again with a hipEvent pair the
library records around each of its launches on the launch stream (per-kernel
durations; the events add a few microseconds between launches, so that pass's
step time is reported apart).  Unless --no-flush, a 512 MiB fill runs between
steps, outside the timed events, so that no workload is served from the 256 MB
Infinity Cache; each step then has its own event pair, and the median and the
minimum of the K step times are reported beside the mean (config.step_ms_*).

Roofline: the dominant kernel's algorithmic bytes (flops, for the MFMA-bound
projection GEMM of the layer workload) per launch divided by its average
duration from the instrumented pass, against MI355X's 8 TB/s HBM peak
(2.5 PFLOP/s dense bf16 MFMA).  cpu_baseline: the fp64 oracle on a bounded sample of the
same workload on this host's cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GMA fwd tokens·heads/s at N=32K,K=128; % of HBM/MFMA roofline"
UNIT = "tokens·heads/s"
HBM_PEAK_GBS = 8000.0


MFMA_BF16_PEAK_TFLOPS = 2500.0


def kernel_flops(name: str, w) -> int:
    """Algorithmic flops of one launch of an MFMA-bound kernel (0 for others):
    the three projections X W_Q, X W_K, X W_V of the layer workload."""
    if name == "gma_proj":
        return 2 * w.B * w.N * w.d_model * w.H * (2 * w.d_r + w.d_v)
    return 0


def kernel_bytes(name: str, w, s_r: int, s_v: int, s_out: int, kc: int = 0) -> int:
    """Algorithmic HBM bytes of one launch of `name` on workload w: s_r, s_v are
    the bytes per element of the routing vectors and values the GMA kernels
    read (a split routing vector is a bf16 pair, 4 bytes), s_out of O.  The
    layer's projection writes Q_X, K_X, V_X in the form the GMA kernels read;
    in the fused form (kc > 0) it writes V_X and, in place of Q_X and K_X, the
    queries' exponentials and the keys' responsibilities (kc bf16 each per
    token and head), which the span totals and the scan read."""
    T = w.B * w.H * w.N
    if kc:
        if name == "gma_proj":
            return 2 * (w.B * w.N * w.d_model + w.d_model * w.H * (2 * w.d_r + w.d_v)) + \
                T * (4 * kc + 2 * w.d_v)
        if name == "gma_span_state":
            return T * (2 * kc + 2 * w.d_v)
        if name == "gma_causal":
            return T * (4 * kc + 2 * w.d_v + w.d_v * s_out)
        if name == "gma_read":
            return T * (2 * kc + w.d_v * s_out)
    if name == "gma_proj":
        return 2 * (w.B * w.N * w.d_model + w.d_model * w.H * (2 * w.d_r + w.d_v)) + \
            T * (2 * w.d_r * s_r + w.d_v * s_v)
    if name in ("gma_write", "gma_span_state"):
        return T * (w.d_r * s_r + w.d_v * s_v)
    if name == "gma_read":
        return T * (w.d_r * s_r + w.d_v * s_out)
    if name == "gma_causal":
        return T * (2 * w.d_r * s_r + w.d_v * s_v + w.d_v * s_out)
    if name == "gma_backward":
        # the whole backward: Q_X, K_X, V_X and dO read, dQ, dK, dV written
        # (the responsibilities and their gradients are intermediates)
        return T * (4 * w.d_r + 3 * w.d_v) * s_out + w.H * w.K * (4 * w.d_r + 1) * 4
    if name == "gma_usage":
        return T * w.d_r * s_r
    if name == "gma_decode":
        # the fp32 state (S, z) read and written, the token's q, k, v and o,
        # and each head's mixture parameters once
        return w.B * w.H * (8 * w.K * (w.d_v + 1) + 2 * w.d_r * s_r + w.d_v * (s_v + s_out)) + \
            w.H * w.K * (2 * w.d_r + 1) * 4
    return 0


def profile_counters(kernel: str, workload: str, src_hash: str) -> dict:
    """The committed rocprofv3 counter summary of a kernel on a workload (HBM
    bytes per launch, MFMA busy fraction), if it was taken on the current
    kernel source; else {}."""
    path = os.path.join(ROOT, "profiles", "%s_%s_counters.json" % (kernel, workload))
    if not os.path.exists(path):
        return {}
    try:
        d = json.load(open(path))
    except ValueError:
        return {}
    if d.get("source_sha256") != src_hash:
        return {}
    return d


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gaussian_mixture_sequence_gma_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")):
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()


def cpu_baseline(w, gen, max_threads: int = 16, min_seconds: float = 10.0,
                 max_seconds: float = 30.0):
    """The fp64 oracle on this host: groups of 2*threads heads at full N (projection
    included for the layer workload), taken in order over (batch, head) and
    cycling, until min_seconds have passed (a group started later than
    max_seconds - last group's time is skipped)."""
    import oracle
    threads = max(1, min(max_threads, os.cpu_count() or 1))
    if w.state_len > 0:
        return cpu_baseline_decode(w, gen, min_seconds, max_seconds)
    per = min(w.H, 2 * threads)
    groups = [(b, h0) for b in range(w.B) for h0 in range(0, w.H, per)]
    done = 0
    t0 = time.perf_counter()
    last = 0.0
    gi = 0
    while True:
        b, h0 = groups[gi % len(groups)]
        h1 = min(w.H, h0 + per)
        sl = slice(h0, h1)
        bs = slice(b, b + 1)
        t1 = time.perf_counter()
        if w.d_model > 0:
            oracle.layer_forward(gen["X"].f32[bs], gen["W_Q"].f32[:, h0 * w.d_r:h1 * w.d_r],
                                 gen["W_K"].f32[:, h0 * w.d_r:h1 * w.d_r],
                                 gen["W_V"].f32[:, h0 * w.d_v:h1 * w.d_v], h1 - h0,
                                 gen["mu"][sl], gen["log_sigma2"][sl], gen["log_pi"][sl],
                                 w.eps, w.causal, nthreads=threads)
        else:
            oracle.forward(gen["Q"].f32[bs, sl], gen["K"].f32[bs, sl], gen["V"].f32[bs, sl],
                           gen["mu"][sl], gen["log_sigma2"][sl], gen["log_pi"][sl], w.eps,
                           w.causal, nthreads=threads)
        last = time.perf_counter() - t1
        done += (h1 - h0) * w.N
        gi += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or el + last > max_seconds:
            break
    dt = time.perf_counter() - t0
    what = "projection + GMA" if w.d_model > 0 else "GMA"
    return {"value": done / dt, "unit": UNIT, "cores": min(threads, per),
            "kind": "oracle",
            "sample": "%d groups of up to %d heads at full N=%d (%s %s, fp64), %d token-heads "
                      "of %d, %.1f s" % (gi, per, w.N, "causal" if w.causal else "bidirectional",
                                         what, done, w.tokens_heads, dt)}


def cpu_baseline_decode(w, gen, min_seconds: float, max_seconds: float):
    """The oracle's decode step over the whole batch (the carried state
    advancing from call to call), repeated until min_seconds have passed."""
    import oracle
    S, z = gen["S"], gen["z"]
    q, k, v = gen["Q"].f32[:, :, 0], gen["K"].f32[:, :, 0], gen["V"].f32[:, :, 0]
    calls = 0
    t0 = time.perf_counter()
    last = 0.0
    while True:
        t1 = time.perf_counter()
        r = oracle.decode_step(S, z, q, k, v, gen["mu"], gen["log_sigma2"], gen["log_pi"], w.eps)
        S, z = r["S"], r["z"]
        last = time.perf_counter() - t1
        calls += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or el + last > max_seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": calls * w.tokens_heads / dt, "unit": UNIT, "cores": 1, "kind": "oracle",
            "sample": "%d decode steps over the whole batch (%d sequences x heads, fp64, "
                      "numpy on one thread for the state update), %.1f s"
                      % (calls, w.B * w.H, dt)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="long_bidir_bf16")
    ap.add_argument("--causal", type=int, default=None, help="override the workload's variant")
    ap.add_argument("--reparam", action="store_true",
                    help="each step derives log sigma^2 and log pi on the device from "
                         "unconstrained parameters (the workload's log sigma^2 and log pi "
                         "arrays stand in for omega and alpha): inside the forward's prologue "
                         "(gma_forward_reparam) for gma_forward workloads, else by "
                         "gma_reparameterize before the step")
    ap.add_argument("--usage-stats", action="store_true",
                    help="time gma_usage_stats (component-usage diagnostics) over the "
                         "workload's queries instead of the forward")
    ap.add_argument("--backward", action="store_true",
                    help="time gma_backward (gradients of the bidirectional forward, dL/dO "
                         "standard normal) instead of the forward")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flush", dest="flush", action="store_false",
                    help="do not evict the Infinity Cache between timed steps")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run a plain 1 GiB device-to-device copy `steps` times (reference "
                         "kernel of known traffic for scaling HBM byte counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(--gpus %d requested; run with --gpus 1)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from gaussian_mixture_sequence_gma_amd import api, binding, inputs

    if args.calibrate_copy:
        nbytes = 1 << 30
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record()
        for _ in range(args.steps):
            dst.copy_(src)
        ev1.record()
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1) / args.steps
        print(json.dumps({"calibrate_copy_bytes_read": nbytes, "bytes_written": nbytes,
                          "ms_per_copy": ms, "GBps_read_plus_write": 2 * nbytes / ms / 1e6}))
        return

    w = inputs.WORKLOADS[args.workload]
    if args.causal is not None:
        w = w.with_(causal=bool(args.causal))
    binding.load()
    dev = torch.device("cuda:0")
    gen = inputs.generate(w, 0)
    s_out = 2 if w.dtype == "bf16" else 4
    s_r = s_v = s_out
    kc = 0                                 # fused layer: components formed

    decode = w.state_len > 0
    if w.d_model > 0:
        X = api.host_tensor_to_device(gen["X"], dev)
        WQ = api.host_tensor_to_device(gen["W_Q"], dev)
        WK = api.host_tensor_to_device(gen["W_K"], dev)
        WV = api.host_tensor_to_device(gen["W_V"], dev)
    else:
        Q = api.host_tensor_to_device(gen["Q"], dev)
        K = api.host_tensor_to_device(gen["K"], dev)
        V = api.host_tensor_to_device(gen["V"], dev)
    mu = torch.from_numpy(gen["mu"]).to(dev)
    ls2 = torch.from_numpy(gen["log_sigma2"]).to(dev)
    lpi = torch.from_numpy(gen["log_pi"]).to(dev)
    out_dtype = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    out = torch.empty((w.B, w.H, w.N, w.d_v), dtype=out_dtype, device=dev)
    dims = binding.make_dims(w.B, w.H, w.N, w.d_r, w.d_v, w.K,
                             binding.GMA_BF16 if w.dtype == "bf16" else binding.GMA_F32,
                             w.chunk)
    if w.d_model > 0:
        nbytes = binding.gma_layer_workspace_bytes(dims, w.d_model, int(w.causal))
        # the projections reach the GMA kernels as bf16 pairs (Q_X, K_X) and
        # bf16 (V_X), or all in fp32
        fmt, _ = binding.gma_layer_projection_layout(dims, w.d_model, int(w.causal))
        s_r, s_v = (4, 2) if fmt in (binding.GMA_PROJ_SPLIT_BF16,
                                     binding.GMA_PROJ_FUSED_BF16) else (4, 4)
        if fmt == binding.GMA_PROJ_FUSED_BF16:
            kc = 32 if w.K <= 32 else 64
    elif decode:
        nbytes = 0
        # the carried state, advanced in place by every step
        S_state = torch.from_numpy(gen["S"]).to(dev)
        z_state = torch.from_numpy(gen["z"]).to(dev)
    else:
        nbytes = binding.gma_forward_workspace_bytes(dims, int(w.causal))
    ws = api.alloc_workspace(nbytes, dev)

    if args.reparam:
        omega, alpha = ls2, lpi
        ls2, lpi = torch.empty_like(omega), torch.empty_like(alpha)

    if args.usage_stats:
        if decode or w.d_model > 0:
            sys.exit("--usage-stats takes a workload with routing vectors (not decode or layer)")
        ws = api.alloc_workspace(binding.gma_usage_workspace_bytes(dims), dev)
        u_counts = torch.empty((w.H, w.K), dtype=torch.int32, device=dev)
        u_f = torch.empty((3, w.H, w.K), dtype=torch.float32, device=dev)
        u_hs = torch.empty((w.H, 3), dtype=torch.float32, device=dev)

    if args.backward:
        if decode or w.d_model > 0:
            sys.exit("--backward takes a workload with routing vectors (not decode or layer)")
        ws = api.alloc_workspace(binding.gma_backward_workspace_bytes(dims, int(w.causal)), dev)
        dO = torch.randn((w.B, w.H, w.N, w.d_v), device=dev).to(out_dtype)
        grads = [torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V),
                 torch.empty_like(mu), torch.empty_like(ls2), torch.empty_like(lpi)]

    def step():
        if args.backward:
            binding.gma_backward(Q, K, V, mu, ls2, lpi, w.eps, int(w.causal), dO, dims, *grads,
                                 ws, ws.numel())
            return
        if args.usage_stats:
            binding.gma_usage_stats(Q, mu, ls2, lpi, dims, 0.1, u_counts, u_f[0], u_f[1], u_hs,
                                    ws, ws.numel())
            return
        if args.reparam and (decode or w.d_model > 0):
            binding.gma_reparameterize(omega, alpha, 1e-4, w.H, w.K, w.d_r, ls2, lpi)
        elif args.reparam:
            binding.gma_forward_reparam(Q, K, V, mu, omega, alpha, 1e-4, w.eps, int(w.causal),
                                        out, dims, None, None, ws, ws.numel())
            return
        if decode:
            binding.gma_decode_step(Q, K, V, mu, ls2, lpi, w.eps, S_state, z_state, out, dims)
        elif w.d_model > 0:
            binding.gma_layer_forward(X, WQ, WK, WV, w.d_model, mu, ls2, lpi, w.eps,
                                      int(w.causal), out, dims, None, None, ws, ws.numel())
        else:
            binding.gma_forward(Q, K, V, mu, ls2, lpi, w.eps, int(w.causal), out, dims,
                                None, None, ws, ws.numel())

    # Between timed steps a 512 MiB fill evicts the 256 MB Infinity Cache (and
    # L2), so a workload whose tensors would fit there is still read from HBM;
    # each step is then timed by its own event pair, the fill outside it.
    flush_buf = torch.empty(512 << 20, dtype=torch.uint8, device=dev) if args.flush else None

    def flush():
        if flush_buf is not None:
            flush_buf.fill_(1)

    for _ in range(args.warmup):
        flush()
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def timed(k):
        """Mean ms per step over k steps (event pairs on the launch stream),
        and the per-step times where each step has its own pair."""
        if flush_buf is None:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(k):
                step()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / k, []
        pairs = []
        torch.cuda.synchronize()
        for _ in range(k):
            flush()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step()
            e1.record(stream)
            pairs.append((e0, e1))
        torch.cuda.synchronize()
        per = [a.elapsed_time(b) for a, b in pairs]
        return sum(per) / k, per

    # timed region 1: K steps as a user runs them -> ms_per_step and value
    binding.gma_timing_enable(False)
    ms, per_step = timed(args.steps)
    value = w.tokens_heads / (ms * 1e-3)
    # timed region 2: the same K steps with a hipEvent pair around every launch
    # (recorded by the library on the launch stream) -> per-kernel durations;
    # the events themselves add a few microseconds between launches, so this
    # region's step time is reported separately
    binding.gma_timing_collect()            # discard anything left over
    binding.gma_timing_enable(True)
    ms_instrumented = timed(args.steps)[0]
    binding.gma_timing_enable(False)
    kt = binding.gma_timing_collect()

    kernels = {name: {"launches": n, "avg_us": 1e3 * tot / max(n, 1)} for name, n, tot in kt}
    dom = max(kernels, key=lambda k: kernels[k]["avg_us"] * kernels[k]["launches"])
    if args.backward:
        # the backward is a chain of passes over fp32 intermediates: its
        # roofline is taken for the whole step against its algorithmic bytes
        kernels["gma_backward"] = {"launches": args.steps, "avg_us": 1e3 * ms}
        dom = "gma_backward"
    dom_bytes = kernel_bytes(dom, w, s_r, s_v, s_out, kc)
    dom_flops = kernel_flops(dom, w)
    prof = profile_counters(dom, w.name, kernel_source_hash())
    traffic = prof.get("hbm_bytes_per_launch")
    t_dom = kernels[dom]["avg_us"] * 1e-6
    if dom_flops:
        achieved = dom_flops / t_dom / 1e12
        roofline = {"bound": "mfma", "kernel": dom, "achieved": achieved,
                    "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": achieved / MFMA_BF16_PEAK_TFLOPS, "traffic": traffic,
                    "mfma_busy": prof.get("mfma_busy"),
                    "alg_flops_per_launch": dom_flops, "alg_bytes_per_launch": dom_bytes}
    else:
        achieved = dom_bytes / t_dom / 1e9 if dom_bytes else None
        roofline = {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": (achieved / HBM_PEAK_GBS) if achieved else None,
                    "traffic": traffic, "mfma_busy": prof.get("mfma_busy"),
                    "alg_bytes_per_launch": dom_bytes}
    # the counters' HBM bytes over the same measured duration
    roofline["traffic_gbs"] = traffic / t_dom / 1e9 if traffic else None
    step_bytes = sum(kernel_bytes(k, w, s_r, s_v, s_out, kc) for k in kernels)

    cpu = None
    if not args.no_cpu_baseline and not args.usage_stats and not args.backward:
        cpu = cpu_baseline(w, gen)

    cfg = {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d_r": w.d_r, "d_v": w.d_v,
           "K": w.K, "causal": bool(w.causal), "inputs": w.dtype, "eps": w.eps,
           "kernel_avg_us": {k: round(v["avg_us"], 2) for k, v in kernels.items()},
           "kernel_timing": "second pass of the K steps with a hipEvent pair around each launch "
                            "(%.4f ms/step in that pass)" % ms_instrumented,
           "cache_flush": "512 MiB fill between timed steps" if args.flush else None,
           "step_ms_median": statistics.median(per_step) if per_step else None,
           "step_ms_min": min(per_step) if per_step else None,
           "step_hbm_frac": (step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS) if step_bytes else None}
    if w.d_model:
        cfg["d_model"] = w.d_model
    if args.usage_stats:
        cfg["step"] = "gma_usage_stats over the queries (threshold 0.1) in place of the forward"
    if args.backward:
        cfg["step"] = "gma_backward (all gradients, forward recomputed) in place of the forward"
    if args.reparam:
        cfg["reparam"] = ("log sigma^2 and log pi from omega and alpha (Eqs. 14-15, eps_sigma 1e-4) "
                          "in every step: " + ("gma_reparameterize before it" if (decode or w.d_model > 0)
                                               else "inside gma_forward_reparam's prologue"))
    if decode:
        cfg["step"] = "one decode token per sequence against a carried fp32 state"
        cfg["state_len"] = w.state_len
    line = {"metric": METRIC, "value": value, "unit": UNIT, "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
            "data": "synthetic (seeded normal routing vectors/values, random mixture parameters)",
            "config": cfg, "roofline": roofline, "cpu_baseline": cpu}
    print(json.dumps(line))


if __name__ == "__main__":
    main()
