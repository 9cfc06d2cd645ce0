"""Shared helpers of the GPU parity tests: seeded inputs, oracle references, tolerances."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from binarized_qk_sparse_amd import ops, synth

RTOL = 1e-3  # fp32 output tolerance: relative
ATOL = 1e-4  # fp32 output tolerance: absolute


def f32(t: torch.Tensor) -> np.ndarray:
    """CPU float32 copy (bf16 widens exactly)."""
    return t.detach().float().cpu().numpy()


def u32(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().view(np.uint32)


def assert_close(got: np.ndarray, want: np.ndarray, what: str, rtol=RTOL, atol=ATOL):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    excess = np.abs(got - want) - (atol + rtol * np.abs(want))
    if excess.max() > 0:
        k = np.unravel_index(np.argmax(excess), excess.shape)
        raise AssertionError(f"{what}: worst element {k}: got {got[k]!r} want {want[k]!r} "
                             f"(|diff| {abs(got[k] - want[k]):.3e}, {int((excess > 0).sum())} elements out)")


def sample_rows(total: int, count: int, seed: int) -> np.ndarray:
    if count >= total:
        return np.arange(total, dtype=np.int64)
    g = np.random.default_rng([77, seed, total])
    return np.sort(g.choice(total, size=count, replace=False)).astype(np.int64)


def rows_per_head(BH: int, n: int, per_head: int, seed: int) -> np.ndarray:
    """A seeded sample of ``per_head`` query rows from every (batch, head) slice, flat and sorted."""
    g = np.random.default_rng([78, seed, BH, n])
    take = min(per_head, n)
    return np.concatenate([bh * n + np.sort(g.choice(n, size=take, replace=False)) for bh in range(BH)]).astype(np.int64)


def packed_inputs(w: synth.Workload, B=None, H=None, dev="cuda"):
    """Seeded inputs plus the oracle's codes/scales; the GPU copies go to `dev`."""
    g = synth.generate(w, B=B, H=H)
    qb, aq, mq = oracle.pack(f32(g["q"]), w.mode)
    kb, ak, mk = oracle.pack(f32(g["k"]), w.mode)
    res = dict(g)
    res.update(oq=qb, ok=kb, oaq=aq, oak=ak, omq=mq, omk=mk)
    res["dq"] = torch.from_numpy(qb.view(np.int32)).to(dev)
    res["dk"] = torch.from_numpy(kb.view(np.int32)).to(dev)
    res["dv"] = g["v"].to(dev)
    if w.mode == synth.MEAN_SIGN:
        res["daq"] = torch.from_numpy(aq).to(dev)
        res["dak"] = torch.from_numpy(ak).to(dev)
    else:
        res["daq"] = res["dak"] = None
        res["oaq"] = res["oak"] = None
    res["dbias"] = None if g["bias"] is None else g["bias"].to(dev)
    res["obias"] = None if g["bias"] is None else g["bias"].numpy()
    return res


def q8_tolerance(vscale: np.ndarray, rows: np.ndarray, n: int) -> np.ndarray:
    """One int8 LSB of V per output element: the scale of its channel."""
    bh = rows // n
    return vscale.reshape(-1, vscale.shape[-1])[bh]


def unpack_q4(packed: np.ndarray) -> np.ndarray:
    """int8 codes [..., 2m] from bytes [..., m] that hold two 4-bit two's-complement codes
    each (channel 2b in the low nibble of byte b, channel 2b + 1 in the high nibble)."""
    p = packed.astype(np.uint8)
    nib = np.stack([p & 0xF, p >> 4], axis=-1).astype(np.int8)
    nib = np.where(nib >= 8, nib - 16, nib).astype(np.int8)
    return nib.reshape(packed.shape[:-1] + (2 * packed.shape[-1],))


def ws_vq(ws: torch.Tensor, B: int, H: int, n: int, d: int, av: int):
    """(V codes int8 [B,H,n,d], scales f32 [B,H,d]) as CPU tensors from a workspace after a
    quantized call, the 4-bit codes unpacked."""
    vq, sc = ops.workspace_view(ws, B, H, n, d, av_mode=av)
    vq = vq.cpu()
    if av == synth.AV_Q4:
        vq = torch.from_numpy(unpack_q4(vq.numpy()))
    return vq, sc.cpu()
