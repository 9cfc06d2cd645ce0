"""Seeded synthetic workloads for binarized-QK attention.

This module only draws random tensors; it holds none of the attention
arithmetic. Both the HIP path and the CPU oracle are fed from here, so the
tests compare them on identical inputs.

Workloads (shapes and value laws stand in for the datasets the pages evaluate
on, which are not available here):

* ``c1`` HAD top-N toy: batch 1, 3 heads, n=197, d=64, fp32 Q/K/V iid N(0,1),
  plain sign, no bias, N=30, fp32 A*V.  (HAD summary, method: N around 30 for
  DeiT at context 197.)
* ``c2`` BERT-base shape: batch 16, 12 heads, n=256, d=64, bf16 Q/K/V iid N(0,1),
  per-head relative-position table over 2n-1 offsets ~ N(0, 0.02^2), plain sign,
  N=30.  (HAD summary, method: BERT at 256 tokens with top 30.)
* ``c3`` T5-base long-context sweep: batch 4, 12 heads, d=64,
  n in {128, 256, 512, 1024}, N = 15*n/128; Q and K are N(0,1) times a
  per-(head, channel) std drawn U(0.5, 2), separately for Q and K; V N(0,1);
  bf16; plain sign; no bias.  (HAD summary, method: N grows linearly from 15 at
  128 tokens to 120 at 1024 tokens.)
* ``c4`` BinaryAttention dense, DeiT-B shape: batch 64, 12 heads, n=197, d=64,
  Q/K = N(0,1) + per-(head, channel) mean ~ N(0, 0.5^2), separately for Q and K;
  V N(0,1); bf16; mean-centred scaled sign; relative-position table; dense
  softmax; uint8 A x int8 V.  (BinaryAttention, sections 2.2-2.4.)
* ``c5`` high-resolution ViT: 1024x1024 image at patch 8 -> n=16384; batch 1,
  16 heads, d=64, bf16 Q/K/V iid N(0,1); mean-centred scaled sign;
  relative-position table; top-256; uint8 A x int8 V over the kept set.
  ``c5q4`` is the same with 4-bit V (7 levels each side of zero).
* ``c4@n``: the DeiT-B dense workload at another length (same batch, heads and laws;
  the relative-position table grows to 2n-1 offsets): the sweep of the dense
  kernel over sequence lengths that BinaryAttention's kernel-speed figure runs.
* ``c4d128`` (and ``c4d128@n``): the dense workload's laws at head_dim 128, the head
  size of BinaryAttention's kernel-speed figure: batch 8, 12 heads, n=1024.
* ``c4b2d``, ``c5b2d``: c4 and c5 with the two-dimensional decomposable bias
  (row and column offset tables ~ N(0, 0.02^2) per head, tensor id 7, over
  the 14 x 14 grid after DeiT's class token and the 128 x 128 grid).

Second arguments of N(., .) are standard deviations.  Generation: NumPy
``default_rng([config_index, n, tensor_id])`` in float32, tensor ids Q=1, K=2,
V=3, bias table=4, per-channel std/mean for Q=5 and for K=6.  Tensors marked
bf16 are rounded to bfloat16 by torch (round to nearest even); the oracle
reads the same bf16 values widened exactly to float32.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np
import torch

SIGN = 0
MEAN_SIGN = 1
AV_F32 = 0
AV_Q8 = 1
AV_Q4 = 2


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int
    B: int
    H: int
    n: int
    d: int
    top_n: Optional[int]  # None -> dense (every key kept)
    dtype: str  # "f32" or "bf16"
    mode: int  # SIGN or MEAN_SIGN
    bias: bool
    av_mode: int  # AV_F32, AV_Q8 or AV_Q4
    qk_law: str  # "iid", "chan_std", "chan_mean"
    grid: Optional[tuple] = None  # (gh, gw): two-dimensional decomposable bias over a patch grid

    @property
    def pairs(self) -> int:
        return self.B * self.H * self.n * self.n

    @property
    def kept(self) -> int:
        return self.n if self.top_n is None else min(self.top_n, self.n)

    def with_n(self, n: int) -> "Workload":
        top = None if self.top_n is None else (15 * n) // 128 if self.name.startswith("c3") else self.top_n
        return dataclasses.replace(self, n=n, top_n=top, name=f"{self.name.split('@')[0]}@{n}")


WORKLOADS: Dict[str, Workload] = {
    "c1": Workload("c1", 0, 1, 3, 197, 64, 30, "f32", SIGN, False, AV_F32, "iid"),
    "c2": Workload("c2", 1, 16, 12, 256, 64, 30, "bf16", SIGN, True, AV_F32, "iid"),
    "c3": Workload("c3", 2, 4, 12, 1024, 64, 120, "bf16", SIGN, False, AV_F32, "chan_std"),
    "c4": Workload("c4", 3, 64, 12, 197, 64, None, "bf16", MEAN_SIGN, True, AV_Q8, "chan_mean"),
    "c5": Workload("c5", 4, 1, 16, 16384, 64, 256, "bf16", MEAN_SIGN, True, AV_Q8, "iid"),
    # c5 with 4-bit V (the next step BinaryAttention's conclusion names); same draws as c5
    "c5q4": Workload("c5q4", 4, 1, 16, 16384, 64, 256, "bf16", MEAN_SIGN, True, AV_Q4, "iid"),
    # c4 and c5 with the two-dimensional decomposable bias in place of the 1-D table:
    # DeiT-B's class token plus 14 x 14 patches, and the 128 x 128 patch grid
    "c4b2d": Workload("c4b2d", 3, 64, 12, 197, 64, None, "bf16", MEAN_SIGN, True, AV_Q8, "chan_mean", (14, 14)),
    "c5b2d": Workload("c5b2d", 4, 1, 16, 16384, 64, 256, "bf16", MEAN_SIGN, True, AV_Q8, "iid", (128, 128)),
    # the long-context sweep at head_dim 128 (the kernel shape of BinaryAttention's
    # speed-versus-length figure); "c3d128@n" scales N = 15 n / 128 like c3
    "c3d128": Workload("c3d128", 5, 4, 12, 1024, 128, 120, "bf16", SIGN, False, AV_F32, "chan_std"),
    # the dense forward at head_dim 128 with c4's inputs, 8 x 12 heads of 1024 tokens
    # ("c4d128@n" for the other lengths of that figure)
    "c4d128": Workload("c4d128", 6, 8, 12, 1024, 128, None, "bf16", MEAN_SIGN, True, AV_Q8, "chan_mean"),
}

C3_SWEEP = (128, 256, 512, 1024)


def c3(n: int) -> Workload:
    """The long-context sweep point at ``n`` tokens (N = 15*n/128)."""
    return WORKLOADS["c3"].with_n(n)


def workload(name: str) -> Workload:
    if "@" in name:
        base, n = name.split("@")
        return WORKLOADS[base].with_n(int(n))
    return WORKLOADS[name]


def _rng(w: Workload, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng([w.index, w.n, tensor_id])


def _round(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def generate(w: Workload, *, B: Optional[int] = None, H: Optional[int] = None) -> Dict[str, object]:
    """Draw Q, K, V (and the bias table) for workload ``w`` on the CPU.

    ``B``/``H`` may shrink the batch or head count (the first B batches and the
    first H heads of the same draw are NOT guaranteed; a smaller shape is a
    separate seeded draw) for parity cases that the oracle must finish fast.

    Returns torch CPU tensors ``q, k, v`` of shape [B, H, n, d] in the
    workload's dtype, ``bias`` as float32 [H, 2n-1] or None, plus the
    workload fields needed by a caller.
    """
    Bv = w.B if B is None else B
    Hv = w.H if H is None else H
    shape = (Bv, Hv, w.n, w.d)
    q = _rng(w, 1).standard_normal(shape, dtype=np.float32)
    k = _rng(w, 2).standard_normal(shape, dtype=np.float32)
    v = _rng(w, 3).standard_normal(shape, dtype=np.float32)
    if w.qk_law == "chan_std":
        q *= _rng(w, 5).uniform(0.5, 2.0, size=(1, Hv, 1, w.d)).astype(np.float32)
        k *= _rng(w, 6).uniform(0.5, 2.0, size=(1, Hv, 1, w.d)).astype(np.float32)
    elif w.qk_law == "chan_mean":
        q += (0.5 * _rng(w, 5).standard_normal((1, Hv, 1, w.d))).astype(np.float32)
        k += (0.5 * _rng(w, 6).standard_normal((1, Hv, 1, w.d))).astype(np.float32)
    bias = bias2d = None
    if w.bias and w.grid is None:
        bias = torch.from_numpy((0.02 * _rng(w, 4).standard_normal((Hv, 2 * w.n - 1))).astype(np.float32))
    elif w.bias:
        gh, gw = w.grid
        g = _rng(w, 7)
        bias2d = {"grid": (gh, gw),
                  "row": torch.from_numpy((0.02 * g.standard_normal((Hv, 2 * gh - 1))).astype(np.float32)),
                  "col": torch.from_numpy((0.02 * g.standard_normal((Hv, 2 * gw - 1))).astype(np.float32))}
        if w.n == gh * gw + 1:
            bias2d["cls"] = torch.from_numpy((0.02 * g.standard_normal((Hv, 3))).astype(np.float32))
    return {
        "q": _round(q, w.dtype),
        "k": _round(k, w.dtype),
        "v": _round(v, w.dtype),
        "bias": bias,
        "bias2d": bias2d,
        "workload": w,
        "B": Bv,
        "H": Hv,
    }


def random_bits(B: int, H: int, n: int, d: int, seed: int) -> np.ndarray:
    """Uniformly random packed codes uint32[B, H, n, d/32] (for kernel-level cases)."""
    g = np.random.default_rng([1000, seed, n, d])
    return g.integers(0, 2**32, size=(B, H, n, d // 32), dtype=np.uint64).astype(np.uint32)


def random_alpha(B: int, H: int, n: int, seed: int) -> np.ndarray:
    """Positive per-token scales float32[B, H, n] around 0.8 (for kernel-level cases)."""
    g = np.random.default_rng([1001, seed, n])
    return (0.8 + 0.1 * g.standard_normal((B, H, n))).astype(np.float32).clip(0.05, None)
