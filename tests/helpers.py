"""Comparison helpers for the GPU parity tests (test infrastructure).

Tolerances (the targets the path is built to):
  * indexer scores: |gpu - ref| <= 1e-3 |ref| + 1e-5 sum_j |q_j k_j|; the
    second term guards cancellation and is ~2.6x the fp32 bound for a
    64-term dot product (gamma_64 ~ 3.8e-6);
  * top-B sets: identical, except positions whose oracle score lies within
    1e-4 * max(|s_B|, rms of the row's scores) of the oracle's B-th score
    (near-ties that fp32 scoring may legitimately order differently);
    identical outright when the scores handed to the selection are the same;
  * attention output: within 2e-3 absolute; lse within 2e-3 absolute.
"""
from __future__ import annotations

import numpy as np
import torch

from indexer_driven_sparse_amd import synth

ATTN_ATOL = 2e-3
LSE_ATOL = 2e-3


def dev(a: np.ndarray) -> torch.Tensor:
    """Host array -> device tensor (uint16 arrays are bf16 bits, uint8
    arrays OCP E4M3 bits)."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    if a.dtype == np.uint8:
        return torch.from_numpy(np.ascontiguousarray(a)).view(torch.float8_e4m3fn).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> host array (bf16 comes back as uint16 bits, fp8 as
    uint8 bits)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()


_FP8 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def decoded(a: np.ndarray) -> np.ndarray:
    """Stored values as float64 (bf16 bits, E4M3 bits or fp32)."""
    if a.dtype == np.uint16:
        return synth.bf16_bits_to_f32(a).astype(np.float64)
    if a.dtype == np.uint8:
        return _FP8[a]
    return a.astype(np.float64)


def assert_scores_close(gpu: np.ndarray, ref: np.ndarray, q: np.ndarray, k: np.ndarray) -> None:
    """gpu/ref [rows, n]; q [rows, r] (double); k [rows, n, r] (decoded)."""
    guard = np.einsum("ir,inr->in", np.abs(q), np.abs(k))
    fin = np.isfinite(ref)
    np.testing.assert_array_equal(np.isneginf(gpu), np.isneginf(ref))
    err = np.abs(gpu[fin] - ref[fin])
    bound = 1e-3 * np.abs(ref[fin]) + 1e-5 * guard[fin]
    bad = err > bound
    assert not bad.any(), f"{bad.sum()} scores out of tolerance; worst {np.max(err - bound)}"


def check_index_sets(gpu: np.ndarray, ref: np.ndarray, ref_scores: list, B: int):
    """gpu/ref [rows, B] ascending, -1 padded; ref_scores[row] maps position
    -> oracle score for that row (array over positions). Returns a list of
    rows whose sets differ (by tolerated near-ties only)."""
    differing = []
    for i in range(gpu.shape[0]):
        g, r = gpu[i], ref[i]
        gv, rv = g[g >= 0], r[r >= 0]
        assert len(gv) == len(rv), f"row {i}: {len(gv)} vs {len(rv)} selected"
        assert (g[len(gv):] == -1).all(), f"row {i}: padding"
        assert np.all(np.diff(gv) > 0), f"row {i}: not strictly ascending"
        if np.array_equal(gv, rv):
            continue
        sc = ref_scores[i]
        sel = sc[rv]
        s_b = np.min(sel)
        tol = 1e-4 * max(abs(s_b), float(np.sqrt(np.mean(sc[np.isfinite(sc)] ** 2))))
        sym = np.setxor1d(gv, rv)
        assert np.all(np.abs(sc[sym] - s_b) <= tol), \
            f"row {i}: {len(sym)} differing positions beyond the near-tie tolerance"
        differing.append(i)
    return differing
