"""Python binding of the C ABI: marshals torch device tensors into pointers.

Every function here only checks shapes/dtypes, allocates outputs with torch
and calls the same-named entry point of ``libhad.so`` on the current HIP
stream.  All arithmetic runs in the library's gfx950 kernels.
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import _lib
from ._lib import (HAD_AV_F32, HAD_AV_Q4, HAD_AV_Q8, HAD_BF16, HAD_F32, HAD_MEAN_SIGN,  # noqa: F401
                   HAD_SIGN, HadError)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return HAD_F32
    if t.dtype == torch.bfloat16:
        return HAD_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, name: str) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def workspace_bytes(B: int, H: int, n: int, d: int) -> int:
    return int(_lib.load().had_workspace_bytes(B, H, n, d))


def workspace(B: int, H: int, n: int, d: int, device=None) -> torch.Tensor:
    """A device byte buffer large enough for any entry point at these sizes."""
    return torch.empty(max(workspace_bytes(B, H, n, d), 256), dtype=torch.uint8, device=device or "cuda")


def had_pack(x: torch.Tensor, mode: int = HAD_SIGN, ws: Optional[torch.Tensor] = None
             ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """x [B,H,n,d] fp32/bf16 -> (bits int32 [B,H,n,d/32] holding uint32 words,
    alpha f32 [B,H,n], mu f32 [B,H,d])."""
    _dev(x, "x")
    B, H, n, d = x.shape
    bits = torch.empty((B, H, n, d // 32), dtype=torch.int32, device=x.device)
    alpha = torch.empty((B, H, n), dtype=torch.float32, device=x.device)
    mu = torch.empty((B, H, d), dtype=torch.float32, device=x.device)
    if mode == HAD_MEAN_SIGN and ws is None:
        ws = workspace(B, H, n, d, x.device)
    wsz = 0 if ws is None else ws.numel()
    st = _lib.load().had_pack(x.data_ptr(), _dtype_code(x), B, H, n, d, mode, bits.data_ptr(),
                              alpha.data_ptr(), mu.data_ptr(), _ptr(ws), wsz, _stream())
    _lib.check("had_pack", st)
    return bits, alpha, mu


def had_pack_qk(q: torch.Tensor, k: torch.Tensor, mode: int = HAD_SIGN, ws: Optional[torch.Tensor] = None):
    """Q and K [B,H,n,d] (same dtype and shape) -> ((qbits, alpha_q, mu_q), (kbits, alpha_k, mu_k)),
    each exactly what had_pack gives for that tensor, from one set of launches."""
    _dev(q, "q")
    _dev(k, "k")
    if q.shape != k.shape or q.dtype != k.dtype:
        raise ValueError("q and k must share shape and dtype")
    B, H, n, d = q.shape
    outs = []
    for _ in range(2):
        outs.append((torch.empty((B, H, n, d // 32), dtype=torch.int32, device=q.device),
                     torch.empty((B, H, n), dtype=torch.float32, device=q.device),
                     torch.empty((B, H, d), dtype=torch.float32, device=q.device)))
    if mode == HAD_MEAN_SIGN and ws is None:
        ws = workspace(B, H, n, d, q.device)
    wsz = 0 if ws is None else ws.numel()
    (qb, aq, mq), (kb, ak, mk) = outs
    st = _lib.load().had_pack_qk(q.data_ptr(), k.data_ptr(), _dtype_code(q), B, H, n, d, mode, qb.data_ptr(),
                                 kb.data_ptr(), aq.data_ptr(), ak.data_ptr(), mq.data_ptr(), mk.data_ptr(),
                                 _ptr(ws), wsz, _stream())
    _lib.check("had_pack_qk", st)
    return outs[0], outs[1]


def _bias2d(bias2d):
    """(row, col, cls, grid_h, grid_w) pointers and sizes of a two-dimensional bias dict
    {"grid": (gh, gw), "row": [H, 2gh-1], "col": [H, 2gw-1], optional "cls": [H, 3]} (device float32)."""
    gh, gw = (int(x) for x in bias2d["grid"])
    for nm in ("row", "col", "cls"):
        if bias2d.get(nm) is not None:
            _dev(bias2d[nm], nm)
    return _ptr(bias2d["row"]), _ptr(bias2d["col"]), _ptr(bias2d.get("cls")), gh, gw


def had_attention_topn(qbits: torch.Tensor, kbits: torch.Tensor, v: torch.Tensor, top_n: int, *,
                       alpha_q: Optional[torch.Tensor] = None, alpha_k: Optional[torch.Tensor] = None,
                       bias: Optional[torch.Tensor] = None, bias2d: Optional[dict] = None, av_mode: int = HAD_AV_F32,
                       want_idx: bool = False, ws: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None):
    """Top-N attention; returns out f32 [B,H,n,d] (and idx int32 [B,H,n,min(N,n)] if asked).
    ``bias2d`` (see ``_bias2d``) selects had_attention_topn_2d in place of the 1-D ``bias``."""
    for t, nm in ((qbits, "qbits"), (kbits, "kbits"), (v, "v")):
        _dev(t, nm)
    B, H, n, d = v.shape
    keep = min(int(top_n), n)
    if out is None:
        out = torch.empty((B, H, n, d), dtype=torch.float32, device=v.device)
    idx = torch.empty((B, H, n, keep), dtype=torch.int32, device=v.device) if want_idx else None
    if av_mode != HAD_AV_F32 and ws is None:
        ws = workspace(B, H, n, d, v.device)
    wsz = 0 if ws is None else ws.numel()
    if bias2d is not None:
        if bias is not None:
            raise ValueError("give bias or bias2d, not both")
        st = _lib.load().had_attention_topn_2d(qbits.data_ptr(), kbits.data_ptr(), _ptr(alpha_q), _ptr(alpha_k),
                                               *_bias2d(bias2d), v.data_ptr(), _dtype_code(v), B, H, n, d,
                                               int(top_n), av_mode, out.data_ptr(), _ptr(idx), _ptr(ws), wsz,
                                               _stream())
        _lib.check("had_attention_topn_2d", st)
        return (out, idx) if want_idx else out
    st = _lib.load().had_attention_topn(qbits.data_ptr(), kbits.data_ptr(), _ptr(alpha_q), _ptr(alpha_k),
                                        _ptr(bias), v.data_ptr(), _dtype_code(v), B, H, n, d, int(top_n),
                                        av_mode, out.data_ptr(), _ptr(idx), _ptr(ws), wsz, _stream())
    _lib.check("had_attention_topn", st)
    return (out, idx) if want_idx else out


def binattn_dense_q8(qbits: torch.Tensor, kbits: torch.Tensor, v: torch.Tensor, *,
                     alpha_q: Optional[torch.Tensor] = None, alpha_k: Optional[torch.Tensor] = None,
                     bias: Optional[torch.Tensor] = None, bias2d: Optional[dict] = None,
                     ws: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Dense softmax, uint8 A x per-channel int8 V; returns out f32 [B,H,n,d].
    ``bias2d`` selects binattn_dense_q8_2d in place of the 1-D ``bias``."""
    for t, nm in ((qbits, "qbits"), (kbits, "kbits"), (v, "v")):
        _dev(t, nm)
    B, H, n, d = v.shape
    if out is None:
        out = torch.empty((B, H, n, d), dtype=torch.float32, device=v.device)
    if ws is None:
        ws = workspace(B, H, n, d, v.device)
    if bias2d is not None:
        if bias is not None:
            raise ValueError("give bias or bias2d, not both")
        st = _lib.load().binattn_dense_q8_2d(qbits.data_ptr(), kbits.data_ptr(), _ptr(alpha_q), _ptr(alpha_k),
                                             *_bias2d(bias2d), v.data_ptr(), _dtype_code(v), B, H, n, d,
                                             out.data_ptr(), ws.data_ptr(), ws.numel(), _stream())
        _lib.check("binattn_dense_q8_2d", st)
        return out
    st = _lib.load().binattn_dense_q8(qbits.data_ptr(), kbits.data_ptr(), _ptr(alpha_q), _ptr(alpha_k),
                                      _ptr(bias), v.data_ptr(), _dtype_code(v), B, H, n, d, out.data_ptr(),
                                      ws.data_ptr(), ws.numel(), _stream())
    _lib.check("binattn_dense_q8", st)
    return out


def binattn_dense_q8_fused(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, mode: int = HAD_MEAN_SIGN, *,
                           bias: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Binarize Q, K and quantize V on chip, then dense q8 attention, in one launch (n <= 256);
    returns out f32 [B,H,n,d], the same bits as had_pack_qk followed by binattn_dense_q8."""
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, nm)
    if q.shape != k.shape or q.dtype != k.dtype or v.shape != q.shape:
        raise ValueError("q, k and v must share a shape, and q and k a dtype")
    B, H, n, d = v.shape
    if out is None:
        out = torch.empty((B, H, n, d), dtype=torch.float32, device=v.device)
    st = _lib.load().binattn_dense_q8_fused(q.data_ptr(), k.data_ptr(), _dtype_code(q), int(mode), _ptr(bias),
                                            v.data_ptr(), _dtype_code(v), B, H, n, d, out.data_ptr(), _stream())
    _lib.check("binattn_dense_q8_fused", st)
    return out


def workspace_view(ws: torch.Tensor, B: int, H: int, n: int, d: int):
    """(vq int8 [B,H,n,d], vscale f32 [B,H,d]) views of a workspace after a quantized call."""
    import math

    def a256(x):
        return (x + 255) // 256 * 256

    chunks = math.ceil(n / 256)
    off_vq = a256(8 * B * H * chunks * d)
    off_sc = a256(off_vq + B * H * n * d)
    vq = ws[off_vq:off_vq + B * H * n * d].view(torch.int8).view(B, H, n, d)
    sc = ws[off_sc:off_sc + 4 * B * H * d].view(torch.float32).view(B, H, d)
    return vq, sc
