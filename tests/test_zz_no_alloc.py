"""lsa_indexed_attention_noalloc: the attention call whose split partials
live in the library's static per-GPU scratch instead of a caller workspace,
for callers that cannot allocate. Through the C ABI it must give exactly
what lsa_indexed_attention gives with a workspace, call after call on the
same scratch (a larger call, then smaller ones), on both attention paths."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from indexer_driven_sparse_amd import synth
from tests.helpers import ATTN_ATOL, LSE_ATOL, dev, host

pytestmark = pytest.mark.gpu


def _case(N, Hq, Hkv, T, B, dtype, seed):
    rng = np.random.default_rng(seed)
    d = 128
    Q = rng.standard_normal((N, Hq, d), dtype=np.float32)
    K = rng.standard_normal((N, T, Hkv, d), dtype=np.float32)
    V = rng.standard_normal((N, T, Hkv, d), dtype=np.float32)
    if dtype == synth.BF16:
        Q, K, V = synth.to_bf16_bits(Q), synth.to_bf16_bits(K), synth.to_bf16_bits(V)
    idx = np.full((N, Hkv, B), -1, dtype=np.int32)
    for n in range(N):
        for g in range(Hkv):
            c = B - (7 if (n + g) % 3 == 0 else 0)        # some rows padded with -1
            idx[n, g, :c] = np.sort(rng.choice(T, size=c, replace=False))
    return Q, K, V, idx


def _both(lsa, Q, K, V, idx, Hq):
    q, k, v, ix = dev(Q), dev(K), dev(V), dev(idx)
    N = Q.shape[0]
    outs = []
    for fn in ("ws", "noalloc"):
        out = torch.full((N, Hq, Q.shape[2]), float("nan"), device="cuda")
        lse = torch.full((N, Hq), float("nan"), device="cuda")
        if fn == "ws":
            lsa.lsa_indexed_attention(q, k, v, ix, out, lse=lse)
        else:
            lsa.lsa_indexed_attention_noalloc(q, k, v, ix, out, lse=lse)
        torch.cuda.synchronize()
        outs.append((host(out), host(lse)))
    return outs


def test_noalloc_attention_equals_workspace_attention():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from indexer_driven_sparse_amd import lsa
    shapes = [
        # (N, Hq, Hkv, T, B, dtype): matrix-core decode, 8 splits of 256 entries
        (4, 32, 8, 20000, 2048, synth.BF16),
        # a smaller call on the same scratch: 3 splits, the last one ragged
        (2, 16, 4, 5000, 700, synth.BF16),
        # the vector path (fp32), many splits of one long list
        (1, 4, 1, 4096, 256, synth.F32),
        # and the first shape again, after the smaller ones
        (4, 32, 8, 20000, 2048, synth.BF16),
    ]
    for i, (N, Hq, Hkv, T, B, dt) in enumerate(shapes):
        print("[case] noalloc attention", i, N, Hq, Hkv, T, B, dt, flush=True)
        need = lsa.attention_workspace_bytes_for(N, Hq, Hkv, 128, B, T, dt)
        assert 0 < need <= lsa.NOALLOC_SCRATCH_BYTES     # partials really go through the scratch
        Q, K, V, idx = _case(N, Hq, Hkv, T, B, dt, seed=100 + i)
        (o_ws, l_ws), (o_na, l_na) = _both(lsa, Q, K, V, idx, Hq)
        np.testing.assert_array_equal(o_na.view(np.int32), o_ws.view(np.int32))
        np.testing.assert_array_equal(l_na.view(np.int32), l_ws.view(np.int32))
        ro, rl = oracle.attention(Q, K, V, idx)
        np.testing.assert_allclose(o_na, ro, rtol=0, atol=ATTN_ATOL)
        np.testing.assert_allclose(l_na, rl, rtol=0, atol=LSE_ATOL)


def test_noalloc_attention_rejects_a_shape_beyond_the_scratch():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from indexer_driven_sparse_amd import lsa
    # 1024 sequences x 8 KV heads x 4 query heads, B = 2048: 33 MB of partials
    N, Hq, Hkv, T, B = 1024, 32, 8, 64, 2048
    print("[case] noalloc attention over the scratch limit", N, Hq, Hkv, B, flush=True)
    q = torch.zeros(N, Hq, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(N, T, Hkv, 128, dtype=torch.bfloat16, device="cuda")
    idx = torch.full((N, Hkv, B), -1, dtype=torch.int32, device="cuda")
    out = torch.empty(N, Hq, 128, device="cuda")
    with pytest.raises(lsa.LsaError) as e:
        lsa.lsa_indexed_attention_noalloc(q, k, k, idx, out)
    assert e.value.status == -6
