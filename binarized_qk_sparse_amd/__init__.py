"""Binarized-QK sparse attention for MI355X (gfx950).

The compute path is ``libhad.so`` (hand-written HIP kernels behind the C ABI of
``include/had.h``); :mod:`binarized_qk_sparse_amd.ops` is the thin torch
binding, :mod:`binarized_qk_sparse_amd.synth` draws the seeded workloads.
"""
__all__ = ["ops", "synth", "build"]
