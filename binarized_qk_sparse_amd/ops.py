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
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _check(t: Optional[torch.Tensor], name: str, device: torch.device, dtypes, shape=None) -> None:
    """An optional tensor argument: on ``device``, contiguous, of one of ``dtypes`` and, when
    given, exactly ``shape``.  Raises before anything reaches the library, so a caller's
    mistake never becomes an out-of-bounds access on the device."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {' or '.join(str(x) for x in dtypes)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


_FLOATS = (torch.float32, torch.bfloat16)


def _check_input(x: torch.Tensor, name: str, device: torch.device):
    """A [B,H,n,d] float32/bfloat16 input; returns (B, H, n, d)."""
    _check(x, name, device, _FLOATS)
    if x.dim() != 4:
        raise ValueError(f"{name} must be [B, H, n, d], got shape {tuple(x.shape)}")
    return tuple(int(s) for s in x.shape)


def _check_ws(ws: Optional[torch.Tensor], device: torch.device, B: int, H: int, n: int, d: int) -> None:
    _check(ws, "ws", device, (torch.uint8,))
    if ws is not None and ws.numel() < workspace_bytes(B, H, n, d):
        raise ValueError(f"ws holds {ws.numel()} bytes, the call needs {workspace_bytes(B, H, n, d)}")


def _check_attention_args(qbits, kbits, v, device, *, alpha_q=None, alpha_k=None, bias=None, bias2d=None,
                          out=None, ws=None):
    """Every tensor argument of the attention entry points against V's [B,H,n,d]: codes int32
    [B,H,n,d/32], alpha float32 [B,H,n], the 1-D bias float32 [H,2n-1], the two-dimensional
    tables against their grid, out float32 [B,H,n,d], the workspace at least
    had_workspace_bytes.  Returns (B, H, n, d)."""
    B, H, n, d = _check_input(v, "v", device)
    if d % 32 != 0:
        raise ValueError(f"head_dim {d} is not a multiple of 32")
    for t, nm in ((qbits, "qbits"), (kbits, "kbits")):
        if t is None:
            raise ValueError(f"{nm} is required")
        _check(t, nm, device, (torch.int32,), (B, H, n, d // 32))
    _check(alpha_q, "alpha_q", device, (torch.float32,), (B, H, n))
    _check(alpha_k, "alpha_k", device, (torch.float32,), (B, H, n))
    _check(bias, "bias", device, (torch.float32,), (H, 2 * n - 1))
    if bias2d is not None:
        if bias is not None:
            raise ValueError("give bias or bias2d, not both")
        gh, gw = (int(x) for x in bias2d["grid"])
        if gh < 1 or gw < 1:
            raise ValueError("bias2d grid sizes must be positive")
        cls = bias2d.get("cls")
        if n != gh * gw + (0 if cls is None else 1):
            raise ValueError(f"n = {n} does not match a {gh} x {gw} grid{'' if cls is None else ' plus a class token'}")
        for nm, shp in (("row", (H, 2 * gh - 1)), ("col", (H, 2 * gw - 1))):
            if bias2d.get(nm) is None:
                raise ValueError(f"bias2d needs '{nm}'")
            _check(bias2d[nm], nm, device, (torch.float32,), shp)
        _check(cls, "cls", device, (torch.float32,), (H, 3))
    _check(out, "out", device, (torch.float32,), (B, H, n, d))
    _check_ws(ws, device, B, H, n, d)
    return B, H, n, d


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
    B, H, n, d = _check_input(x, "x", x.device)
    _check_ws(ws, x.device, B, H, n, d)
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
    B, H, n, d = _check_input(q, "q", q.device)
    _check_input(k, "k", q.device)
    if q.shape != k.shape or q.dtype != k.dtype:
        raise ValueError("q and k must share shape and dtype")
    _check_ws(ws, q.device, B, H, n, d)
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
    return _ptr(bias2d["row"]), _ptr(bias2d["col"]), _ptr(bias2d.get("cls")), gh, gw


def had_attention_topn(qbits: torch.Tensor, kbits: torch.Tensor, v: torch.Tensor, top_n: int, *,
                       alpha_q: Optional[torch.Tensor] = None, alpha_k: Optional[torch.Tensor] = None,
                       bias: Optional[torch.Tensor] = None, bias2d: Optional[dict] = None, av_mode: int = HAD_AV_F32,
                       want_idx: bool = False, ws: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None):
    """Top-N attention; returns out f32 [B,H,n,d] (and idx int32 [B,H,n,min(N,n)] if asked).
    ``bias2d`` (see ``_bias2d``) selects had_attention_topn_2d in place of the 1-D ``bias``."""
    _dev(v, "v")
    B, H, n, d = _check_attention_args(qbits, kbits, v, v.device, alpha_q=alpha_q, alpha_k=alpha_k, bias=bias,
                                       bias2d=bias2d, out=out, ws=ws)
    if int(top_n) < 1:
        raise ValueError("top_n must be at least 1")
    keep = min(int(top_n), n)
    if out is None:
        out = torch.empty((B, H, n, d), dtype=torch.float32, device=v.device)
    idx = torch.empty((B, H, n, keep), dtype=torch.int32, device=v.device) if want_idx else None
    if av_mode != HAD_AV_F32 and ws is None:
        ws = workspace(B, H, n, d, v.device)
    wsz = 0 if ws is None else ws.numel()
    if bias2d is not None:
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
    _dev(v, "v")
    B, H, n, d = _check_attention_args(qbits, kbits, v, v.device, alpha_q=alpha_q, alpha_k=alpha_k, bias=bias,
                                       bias2d=bias2d, out=out, ws=ws)
    if out is None:
        out = torch.empty((B, H, n, d), dtype=torch.float32, device=v.device)
    if ws is None:
        ws = workspace(B, H, n, d, v.device)
    if bias2d is not None:
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


def binattn_dense_q8_noalloc(qbits: torch.Tensor, kbits: torch.Tensor, v: torch.Tensor, *,
                             alpha_q: Optional[torch.Tensor] = None, alpha_k: Optional[torch.Tensor] = None,
                             bias: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """binattn_dense_q8 without a workspace: the library's static device scratch holds the
    integer V (sizes up to HAD_NOALLOC_SCRATCH_BYTES of workspace); returns out f32 [B,H,n,d].
    Calls that overlap on one GPU share that scratch and must be ordered by the caller."""
    _dev(v, "v")
    B, H, n, d = _check_attention_args(qbits, kbits, v, v.device, alpha_q=alpha_q, alpha_k=alpha_k, bias=bias,
                                       out=out)
    if out is None:
        out = torch.empty((B, H, n, d), dtype=torch.float32, device=v.device)
    st = _lib.load().binattn_dense_q8_noalloc(qbits.data_ptr(), kbits.data_ptr(), _ptr(alpha_q), _ptr(alpha_k),
                                              _ptr(bias), v.data_ptr(), _dtype_code(v), B, H, n, d, out.data_ptr(),
                                              _stream())
    _lib.check("binattn_dense_q8_noalloc", st)
    return out


def had_attention_topn_fused(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, top_n: int, mode: int = HAD_SIGN, *,
                             bias: Optional[torch.Tensor] = None, want_idx: bool = False,
                             out: Optional[torch.Tensor] = None):
    """Binarize Q and K on chip and run the top-N attention (fp32 A*V) in one launch, for
    sequences one workgroup holds; returns out f32 [B,H,n,d] (and idx int32 [B,H,n,min(N,n)])."""
    _dev(v, "v")
    B, H, n, d = _check_input(v, "v", v.device)
    _check_input(q, "q", v.device)
    _check_input(k, "k", v.device)
    if q.shape != k.shape or q.dtype != k.dtype or v.shape != q.shape:
        raise ValueError("q, k and v must share a shape, and q and k a dtype")
    if int(top_n) < 1:
        raise ValueError("top_n must be at least 1")
    _check(bias, "bias", v.device, (torch.float32,), (H, 2 * n - 1))
    _check(out, "out", v.device, (torch.float32,), (B, H, n, d))
    keep = min(int(top_n), n)
    if out is None:
        out = torch.empty((B, H, n, d), dtype=torch.float32, device=v.device)
    idx = torch.empty((B, H, n, keep), dtype=torch.int32, device=v.device) if want_idx else None
    st = _lib.load().had_attention_topn_fused(q.data_ptr(), k.data_ptr(), _dtype_code(q), int(mode), _ptr(bias),
                                              v.data_ptr(), _dtype_code(v), B, H, n, d, int(top_n), out.data_ptr(),
                                              _ptr(idx), _stream())
    _lib.check("had_attention_topn_fused", st)
    return (out, idx) if want_idx else out


def binattn_dense_q8_fused(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, mode: int = HAD_MEAN_SIGN, *,
                           bias: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Binarize Q, K and quantize V on chip, then dense q8 attention, in one launch (n <= 256);
    returns out f32 [B,H,n,d], the same bits as had_pack_qk followed by binattn_dense_q8."""
    _dev(v, "v")
    B, H, n, d = _check_input(v, "v", v.device)
    _check_input(q, "q", v.device)
    _check_input(k, "k", v.device)
    if q.shape != k.shape or q.dtype != k.dtype or v.shape != q.shape:
        raise ValueError("q, k and v must share a shape, and q and k a dtype")
    _check(bias, "bias", v.device, (torch.float32,), (H, 2 * n - 1))
    _check(out, "out", v.device, (torch.float32,), (B, H, n, d))
    if out is None:
        out = torch.empty((B, H, n, d), dtype=torch.float32, device=v.device)
    st = _lib.load().binattn_dense_q8_fused(q.data_ptr(), k.data_ptr(), _dtype_code(q), int(mode), _ptr(bias),
                                            v.data_ptr(), _dtype_code(v), B, H, n, d, out.data_ptr(), _stream())
    _lib.check("binattn_dense_q8_fused", st)
    return out


def workspace_view(ws: torch.Tensor, B: int, H: int, n: int, d: int, av_mode: int = HAD_AV_Q8):
    """(vq, vscale f32 [B,H,d]) views of a workspace after a quantized call, at the offsets
    the library reports (had_workspace_region).  vq is int8 [B,H,n,d] after HAD_AV_Q8, and
    uint8 [B,H,n,d/2] after HAD_AV_Q4: two 4-bit two's-complement codes per byte, channel 2b
    in the low nibble of byte b and channel 2b + 1 in the high nibble."""
    import ctypes

    lib = _lib.load()
    views = []
    for region in (_lib.HAD_WS_VQ, _lib.HAD_WS_VSCALE):
        off, nb = ctypes.c_size_t(0), ctypes.c_size_t(0)
        _lib.check("had_workspace_region",
                   lib.had_workspace_region(B, H, n, d, region, ctypes.byref(off), ctypes.byref(nb)))
        if off.value + nb.value > ws.numel():
            raise ValueError("workspace smaller than the region it should hold")
        views.append(ws[off.value:off.value + nb.value])
    if av_mode == HAD_AV_Q4:
        vq = views[0][:B * H * n * (d // 2)].view(torch.uint8).view(B, H, n, d // 2)
    else:
        vq = views[0].view(torch.int8).view(B, H, n, d)
    sc = views[1].view(torch.float32).view(B, H, d)
    return vq, sc
