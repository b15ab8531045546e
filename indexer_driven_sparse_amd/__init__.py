"""Indexer-driven sparse attention for AMD MI355X (gfx950).

The compute path is the C-ABI library ``liblsa.so`` (hand-written HIP
kernels); :mod:`indexer_driven_sparse_amd.lsa` is its thin ctypes binding and
:mod:`indexer_driven_sparse_amd.synth` draws the seeded synthetic workloads.
"""
__all__ = ["lsa", "synth"]
