"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer:
every entry point runs on small seeded inputs (decode, hierarchical,
prefill, block-shared prefill, fp8), in a child process that preloads the
ASan runtime, and any report fails the test. Host code only; no GPU."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "lsa_oracle.c")

DRIVER = r"""
import sys
sys.path.insert(0, ROOT)
import numpy as np
import oracle
from indexer_driven_sparse_amd import synth
oracle.set_threads(2)
rng = np.random.default_rng(7)
bf = lambda a: synth.to_bf16_bits(np.asarray(a, np.float32))
N, Hq, Hkv, T, d, r, B = 2, 8, 2, 300, 64, 16, 37
Q, K, V = bf(rng.standard_normal((N, Hq, d))), bf(rng.standard_normal((N, T, Hkv, d))), bf(rng.standard_normal((N, T, Hkv, d)))
W = (rng.standard_normal((d, r)) / 8).astype(np.float32)
kd = oracle.project_keys(K, W, oracle.BF16)
k8 = oracle.project_keys(K, W, oracle.FP8)
out = oracle.decode_step(Q, W, kd, K, V, B)
out8 = oracle.decode_step(Q, W, k8, K, V, B)
cen = oracle.centroids(kd, 16)
hi = oracle.hierarchical_decode_step(Q, W, kd, cen, K, V, 16, 5, B)
qi = oracle.query_prep(Q, Hkv, W)
sc = oracle.scores(qi, kd)
idx, osc, cnt = oracle.topk(sc.reshape(N * Hkv, T), B, n_valid=np.array([T, 5, 0, T - 1], np.int32))
att, lse = oracle.attention(Q, K, V, out["idx"])
L = 200
qp, kp = bf(rng.standard_normal((L, 1, 64))), bf(rng.standard_normal((L, 1, 64)))
pi, ps = oracle.prefill_topk(qp, kp, 50)
pf = oracle.prefill_scores(qp, kp)
bi, bs, bsc = oracle.prefill_block_topk(qp, kp, 50, 16, want_scores=True)
Qp, Kp, Vp = bf(rng.standard_normal((L, 8, d))), bf(rng.standard_normal((1, L, 1, d))), bf(rng.standard_normal((1, L, 1, d)))
pa, pl = oracle.attention(Qp, Kp, Vp, pi, prefill=True)
ba, bl = oracle.attention(Qp, Kp, Vp, bi, prefill=True, query_block=16)
for x in (0.1, -3.0, 1e30, float("nan")):
    oracle.round_bf16(x); oracle.round_fp8(x)
print("driver ok", int(out["idx"].sum()), int(pi.sum()), flush=True)
"""


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("the gcc AddressSanitizer runtime is not installed")
    lib = str(tmp_path / "liblsa_oracle_san.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                           "-fno-omit-frame-pointer", SRC, "-o", lib, "-lm"])
    env = dict(os.environ)
    env.update({"LD_PRELOAD": asan, "LSA_ORACLE_LIB": lib,
                "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1",
                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1", "OMP_NUM_THREADS": "2"})
    res = subprocess.run([sys.executable, "-c", f"ROOT = {ROOT!r}\n" + DRIVER], env=env,
                         capture_output=True, text=True, timeout=600)
    report = res.stdout[-3000:] + res.stderr[-6000:]
    assert res.returncode == 0, report
    assert "driver ok" in res.stdout, report
    assert "AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr, report
