"""Seeded synthetic workloads shared by the tests, the smoke check and the
benchmark.

This module only draws random inputs and encodes them (fp32, or bf16 bits
by round-to-nearest-even). It computes nothing the method computes: no
projection, no score, no selection, no attention. Both the CPU oracle and the
GPU library receive exactly the arrays built here.

Shapes follow the decode and prefill workloads of the pages: GQA 32 query /
8 KV heads with head_dim 128 (the LLaMA-3.1-8B attention shape the JSSA
figures use), projected rank 64, budgets B = T/64 (the fixed 1.5625% budget
of JSSA Fig. 3) and B = 2048 (JSSA Figs. 4 and 6). The pages' accuracy
datasets and models are not reproduced; these draws stand in for their
context shapes.

bf16 arrays are returned as numpy.uint16 raw bits; fp32 arrays as float32.
"""
from __future__ import annotations

import dataclasses

import numpy as np

F32 = 0
BF16 = 1


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Encode finite float32 values as bf16 bits, round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + (((u >> 16) & 1) + 0x7FFF)) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact decode of bf16 bits to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _encode(x: np.ndarray, dtype: int) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32) if dtype == F32 else to_bf16_bits(x)


def _streams(seed: int):
    """Independent generators, spawned in a fixed order:
    Q, K, V, W, indexer noise, plant positions."""
    kids = np.random.SeedSequence(seed).spawn(6)
    return [np.random.Generator(np.random.PCG64(k)) for k in kids]


@dataclasses.dataclass
class DecodeCase:
    """A decode workload: one layer's cache plus one step's queries."""
    name: str
    N: int
    Hq: int
    Hkv: int
    T: int
    d: int
    r: int
    B: int
    dtype: int           # storage dtype of Q, K, V and the projected-key cache
    Q: np.ndarray        # [N, Hq, d]
    K: np.ndarray        # [N, T, Hkv, d]  (standard GQA cache layout)
    V: np.ndarray        # [N, T, Hkv, d]
    W: np.ndarray        # [d, r] float32
    planted: list | None = None   # per (n, g): sorted planted positions
    block: int = 64      # hierarchical block size
    B_coarse: int = 0    # hierarchical: blocks kept by the coarse pass (0 = flat)
    seed: int = 0        # SeedSequence root of the draws

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv


def make_decode_case(N: int, Hq: int, Hkv: int, T: int, d: int = 128, r: int = 64,
                     B: int = 256, dtype: int = BF16, plant: str | None = None,
                     plant_sigma: float = 4.0, hitter_frac: float = 0.01,
                     n_spans: int = 64, span: int = 32, seed: int = 0,
                     name: str = "decode", B_coarse: int = 0, block: int = 64) -> DecodeCase:
    """Draw Q, K, V ~ N(0,1) and W ~ N(0, 1/d).

    plant=None: nothing planted.
    plant="hitters": round(hitter_frac*T) positions per (sequence, KV head),
      drawn independently, get plant_sigma standard deviations added along
      the direction of the group's summed query (heavy hitters aligned with
      the mean query).
    plant="spans": n_spans non-overlapping spans of `span` contiguous tokens
      per (sequence, KV head) get the same shift; span starts are a sorted
      sample of n_spans distinct values from [0, T - n_spans*span], spread by
      span*rank so they never overlap.
    The shift is applied before the storage cast.
    """
    sq, sk, sv, sw, _snoise, sp = _streams(seed)
    G = Hq // Hkv
    Qf = sq.standard_normal((N, Hq, d), dtype=np.float32)
    W = (sw.standard_normal((d, r), dtype=np.float32) / np.float32(np.sqrt(d))).astype(np.float32)
    K = np.empty((N, T, Hkv, d), dtype=np.float32 if dtype == F32 else np.uint16)
    V = np.empty_like(K)
    planted = [] if plant else None
    for n in range(N):
        Kn = sk.standard_normal((T, Hkv, d), dtype=np.float32)
        if plant:
            for g in range(Hkv):
                direction = Qf[n, g * G:(g + 1) * G].astype(np.float64).sum(axis=0)
                direction /= np.linalg.norm(direction)
                if plant == "hitters":
                    cnt = int(round(hitter_frac * T))
                    pos = np.sort(sp.choice(T, size=cnt, replace=False))
                elif plant == "spans":
                    hi = T - n_spans * span
                    if hi < 0:
                        raise ValueError("spans do not fit in T")
                    starts = np.sort(sp.choice(hi + 1, size=n_spans, replace=False))
                    starts = starts + span * np.arange(n_spans)
                    pos = (starts[:, None] + np.arange(span)[None, :]).reshape(-1)
                else:
                    raise ValueError(f"unknown plant {plant!r}")
                Kn[pos, g, :] += np.float32(plant_sigma) * direction.astype(np.float32)
                planted.append(pos.astype(np.int64))
        K[n] = _encode(Kn, dtype)
        del Kn
        V[n] = _encode(sv.standard_normal((T, Hkv, d), dtype=np.float32), dtype)
    return DecodeCase(name=name, N=N, Hq=Hq, Hkv=Hkv, T=T, d=d, r=r, B=B, dtype=dtype,
                      Q=_encode(Qf, dtype), K=K, V=V, W=W, planted=planted,
                      B_coarse=B_coarse, block=block, seed=seed)


@dataclasses.dataclass
class PrefillCase:
    """A causal prefill workload: indexer vectors drawn directly, plus the
    full-width Q/K/V of one KV group."""
    name: str
    L: int
    Hq: int
    Hkv: int
    d: int
    r: int
    B: int
    q_idx: np.ndarray    # [L, Hkv, r] bf16 bits
    k_idx: np.ndarray    # [L, Hkv, r] bf16 bits
    Q: np.ndarray        # [L, Hq, d] bf16 bits
    K: np.ndarray        # [1, L, Hkv, d] bf16 bits
    V: np.ndarray        # [1, L, Hkv, d] bf16 bits


def sinusoid(L: int, width: int) -> np.ndarray:
    """Position component pe(p)[2m] = cos(p*th_m), pe(p)[2m+1] = sin(p*th_m),
    th_m = 10000^(-2m/width): a RoPE-like sinusoid added to the draws."""
    m = np.arange(width // 2, dtype=np.float64)
    th = 10000.0 ** (-2.0 * m / width)
    ang = np.arange(L, dtype=np.float64)[:, None] * th[None, :]
    pe = np.empty((L, width), dtype=np.float64)
    pe[:, 0::2] = np.cos(ang)
    pe[:, 1::2] = np.sin(ang)
    return pe.astype(np.float32)


def make_prefill_case(L: int, Hq: int = 8, Hkv: int = 1, d: int = 128, r: int = 64,
                      B: int = 2048, seed: int = 3, name: str = "prefill") -> PrefillCase:
    """N(0,1) draws plus an amplitude-1 sinusoidal position component, all
    stored as bf16."""
    sq, sk, sv, _sw, snoise, _sp = _streams(seed)
    pe_r = sinusoid(L, r)[:, None, :]
    pe_d = sinusoid(L, d)[:, None, :]
    q_idx = to_bf16_bits(snoise.standard_normal((L, Hkv, r), dtype=np.float32) + pe_r)
    k_idx = to_bf16_bits(snoise.standard_normal((L, Hkv, r), dtype=np.float32) + pe_r)
    Q = to_bf16_bits(sq.standard_normal((L, Hq, d), dtype=np.float32) + pe_d)
    K = to_bf16_bits(sk.standard_normal((L, Hkv, d), dtype=np.float32) + pe_d)[None]
    V = to_bf16_bits(sv.standard_normal((L, Hkv, d), dtype=np.float32))[None]
    return PrefillCase(name=name, L=L, Hq=Hq, Hkv=Hkv, d=d, r=r, B=B, q_idx=q_idx,
                       k_idx=k_idx, Q=Q, K=K, V=V)


# The five named workloads. Seeds are the workload's ordinal.
WORKLOADS = {
    "decode_t4k_fp32": "decode, 1 sequence, T=4096, 1 KV head / 4 query heads, d=128, r=64, "
                       "B=256, all fp32",
    "decode_t32k_hitters": "decode, 1 sequence, T=32768, GQA 32/8, d=128, r=64, B=1024, bf16, "
                           "1% heavy hitters planted +4 sigma along the mean query",
    "decode_t128k_b2048": "decode, 4 sequences, T=131072, GQA 32/8, d=128, r=64, B=2048, bf16, "
                          "64 hot spans of 32 tokens per KV head",
    "prefill_l64k": "causal prefill indexer + sparse attention, L=65536, 1 KV head / 8 query "
                    "heads, d=128, r=64, top-2048, bf16, sinusoidal position component",
    "hier_t1m": "hierarchical decode, 1 sequence, T=1048576, GQA 32/8, d=128, r=64, block 64, "
                "top-128 blocks, B=2048, bf16, hot spans",
}


def workload(name: str, **over):
    """Build one of the named workloads (keyword overrides shrink it for
    tests, e.g. T=...)."""
    if name == "decode_t4k_fp32":
        kw = dict(N=1, Hq=4, Hkv=1, T=4096, B=256, dtype=F32, seed=0)
    elif name == "decode_t32k_hitters":
        kw = dict(N=1, Hq=32, Hkv=8, T=32768, B=1024, dtype=BF16, plant="hitters", seed=1)
    elif name == "decode_t128k_b2048":
        kw = dict(N=4, Hq=32, Hkv=8, T=131072, B=2048, dtype=BF16, plant="spans", seed=2)
    elif name == "prefill_l64k":
        kw = dict(L=65536, Hq=8, Hkv=1, B=2048, seed=3)
        kw.update(over)
        return make_prefill_case(name=name, **kw)
    elif name == "hier_t1m":
        kw = dict(N=1, Hq=32, Hkv=8, T=1048576, B=2048, dtype=BF16, plant="spans", seed=4,
                  B_coarse=128, block=64)
    else:
        raise KeyError(name)
    kw.update(over)
    return make_decode_case(name=name, **kw)
