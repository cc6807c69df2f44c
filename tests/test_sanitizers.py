"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The oracle's C core, built with gcc and both sanitizers, runs the forward
  (both variants, row subsets, assignments, the latent state, ragged lengths,
  K = 1) and the responsibilities in a child process with the sanitizer runtime
  preloaded.  Its results must equal the regular build's bit for bit, and the
  sanitizers must report nothing.
* The library's host code (argument checks, planning, workspace sizing, the
  C ABI), built by build_host_sanitized, runs the CPU ABI and validation tests
  in a child process with clang's ASan runtime preloaded.

Both children run with leak detection off (the interpreter itself holds
allocations to exit) and halt on the first UBSan report.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

_ORACLE_CHILD = r"""
import sys
import numpy as np
sys.path.insert(0, ROOT)
import oracle
from gaussian_mixture_sequence_gma_amd import inputs

def cases():
    for (B, H, N, d_r, d_v, K, causal, rows) in [
            (1, 2, 37, 8, 5, 3, False, None),
            (2, 1, 70, 16, 8, 1, True, None),
            (1, 1, 129, 4, 3, 7, True, [0, 5, 64, 128]),
            (1, 2, 65, 8, 4, 5, False, [1, 64])]:
        w = inputs.Workload("san", B, H, N, d_r, d_v, K, "f32", causal)
        yield w, inputs.generate(w, 3), (None if rows is None else np.array(rows, dtype=np.int64))

def run():
    out = []
    for w, g, rows in cases():
        r = oracle.forward(g["Q"].f32, g["K"].f32, g["V"].f32, g["mu"], g["log_sigma2"],
                           g["log_pi"], w.eps, w.causal, rows=rows, want_assign=True,
                           want_latent=not w.causal, nthreads=2)
        out.extend(np.asarray(v) for v in r.values())
        rr = oracle.responsibilities(g["Q"].f32, g["mu"], g["log_sigma2"], g["log_pi"])
        out.extend(np.asarray(v) for v in rr.values())
    return out

ref = run()
with oracle.using_library(SAN):
    got = run()
assert len(ref) == len(got)
for a, b in zip(ref, got):
    assert a.shape == b.shape and np.array_equal(a, b), "sanitized oracle differs"
print("oracle under sanitizers: %d arrays equal" % len(ref))
"""


def _asan_env(preload: str) -> dict:
    env = dict(os.environ)
    env["LD_PRELOAD"] = preload
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    return env


def _check_child(r: subprocess.CompletedProcess):
    text = r.stdout + r.stderr
    assert "AddressSanitizer" not in text, text[-4000:]
    assert "runtime error" not in text, text[-4000:]
    assert r.returncode == 0, text[-4000:]


def test_oracle_under_asan_ubsan(tmp_path):
    import oracle
    oracle.build(force=False)                     # the regular build the child compares with
    san = str(tmp_path / "gma_oracle_san.so")
    src = os.path.join(ROOT, "oracle", "gma_oracle.c")
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-Wall",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                           "-fno-omit-frame-pointer", "-o", san, src, "-lm", "-lpthread"])
    libasan = subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
    code = "ROOT = %r\nSAN = %r\n" % (ROOT, san) + _ORACLE_CHILD
    r = subprocess.run([sys.executable, "-c", code], env=_asan_env(libasan), capture_output=True,
                       text=True, timeout=600)
    _check_child(r)
    assert "arrays equal" in r.stdout


def _clang_asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_library_host_code_under_asan_ubsan():
    from gaussian_mixture_sequence_gma_amd import build
    rt = _clang_asan_runtime()
    if rt is None:
        pytest.skip("clang ASan runtime not found")
    objs = [os.path.join(build.OBJDIR, os.path.splitext(s)[0] + ".o") for s in build.SOURCES[1:]]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("library objects not built (run the build first)")
    lib = build.build_host_sanitized()
    env = _asan_env(rt)
    env["GMA_LIBRARY"] = lib
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py"),
                        os.path.join(ROOT, "tests", "test_api_validation.py")],
                       env=env, capture_output=True, text=True, timeout=900, cwd=ROOT)
    _check_child(r)
    assert " passed" in r.stdout and "failed" not in r.stdout, r.stdout[-3000:]
