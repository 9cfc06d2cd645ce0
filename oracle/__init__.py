"""CPU oracle for binarized-QK attention (TEST INFRASTRUCTURE).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It wraps ``libhad_oracle.so`` (plain C, built from
``had_oracle.c`` by :func:`build`) with NumPy-array functions.  It shares no
code with the GPU library and imports nothing from it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "had_oracle.c")
_SO = os.path.join(_HERE, "libhad_oracle.so")

SIGN = 0
MEAN_SIGN = 1
AV_F32 = 0
AV_Q8 = 1
AV_Q4 = 2  # 4-bit V: 7 levels each side of zero, stored as int8

_lib = None


def build() -> str:
    """Compile the oracle with gcc (-O2, no FP contraction, OpenMP)."""
    tmp = _SO + ".tmp"
    cmd = ["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_SO)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.oracle_pack.argtypes = [P, I64, I64, I64, I64, ctypes.c_int, P, P, P]
    lib.oracle_pack.restype = None
    lib.oracle_logits.argtypes = [P, P, P, P, P, P, P, P, I64, I64, I64, I64, I64, I64, I64, P, P]
    lib.oracle_logits.restype = None
    lib.oracle_vquant.argtypes = [P, I64, I64, I64, I64, P, P]
    lib.oracle_vquant.restype = None
    lib.oracle_vquant_levels.argtypes = [P, I64, I64, I64, I64, ctypes.c_int, P, P]
    lib.oracle_vquant_levels.restype = None
    lib.oracle_attention.argtypes = [P, P, P, P, P, P, P, P, I64, I64, I64, P, P, P, I64, I64, I64, I64, I64,
                                     ctypes.c_int, P, I64, P, P, P]
    lib.oracle_attention.restype = ctypes.c_int
    lib.oracle_threads.argtypes = []
    lib.oracle_threads.restype = ctypes.c_int
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_threads.restype = None
    _lib = lib
    return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def threads() -> int:
    return _load().oracle_threads()


def set_threads(t: int) -> None:
    _load().oracle_set_threads(int(t))


def pack(x: np.ndarray, mode: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """x float32 [B,H,n,d] -> (bits uint32 [B,H,n,d/32], alpha f32 [B,H,n], mu f32 [B,H,d])."""
    x = _c(x, np.float32)
    B, H, n, d = x.shape
    assert d % 32 == 0
    bits = np.zeros((B, H, n, d // 32), np.uint32)
    alpha = np.zeros((B, H, n), np.float32)
    mu = np.zeros((B, H, d), np.float32)
    _load().oracle_pack(_ptr(x), B, H, n, d, mode, _ptr(bits), _ptr(alpha), _ptr(mu))
    return bits, alpha, mu


def _bias2d_args(bias2d, n):
    """(R, C, X, gh, gw, cls) of a two-dimensional decomposable bias, or the absent form.

    ``bias2d`` is None or a dict: ``grid`` (gh, gw), ``row`` float32 [H, 2gh-1], ``col``
    float32 [H, 2gw-1] and, with a leading class token, ``cls`` float32 [H, 3]
    (class->patch, patch->class, class->class); n must be gh*gw (+1 with a class token)."""
    if bias2d is None:
        return None, None, None, 0, 0, 0
    gh, gw = (int(x) for x in bias2d["grid"])
    X = _c(bias2d.get("cls"), np.float32)
    cls = 0 if X is None else 1
    assert n == cls + gh * gw, "n must be the grid size plus the class token"
    return _c(bias2d["row"], np.float32), _c(bias2d["col"], np.float32), X, gh, gw, cls


def logits(qbits, kbits, alpha_q=None, alpha_k=None, bias=None, bias2d=None):
    """Full (hamming int32, logits float32) matrices [B,H,n,n]."""
    qbits = _c(qbits, np.uint32)
    kbits = _c(kbits, np.uint32)
    B, H, n, W = qbits.shape
    d = 32 * W
    ham = np.zeros((B, H, n, n), np.int32)
    lg = np.zeros((B, H, n, n), np.float32)
    aq, ak, T = _c(alpha_q, np.float32), _c(alpha_k, np.float32), _c(bias, np.float32)
    R, C, X, gh, gw, cls = _bias2d_args(bias2d, n)
    _load().oracle_logits(_ptr(qbits), _ptr(kbits), _ptr(aq), _ptr(ak), _ptr(T), _ptr(R), _ptr(C), _ptr(X), gh, gw,
                          cls, B, H, n, d, _ptr(ham), _ptr(lg))
    return ham, lg


def vquant(v: np.ndarray, levels: int = 127):
    """v float32 [B,H,n,d] -> (vq int8 [B,H,n,d], scale float32 [B,H,d]); ``levels`` 127 (int8)
    or 7 (4-bit V)."""
    v = _c(v, np.float32)
    B, H, n, d = v.shape
    vq = np.zeros((B, H, n, d), np.int8)
    sc = np.zeros((B, H, d), np.float32)
    _load().oracle_vquant_levels(_ptr(v), B, H, n, d, int(levels), _ptr(vq), _ptr(sc))
    return vq, sc


def attention(qbits, kbits, v, *, alpha_q=None, alpha_k=None, bias=None, bias2d=None, top_n=None,
              av_mode=AV_F32, rows=None, want_idx=False, want_aq8=False):
    """Attention for the given flat query rows (all rows if ``rows`` is None).

    ``bias`` is the 1-D offset table [H, 2n-1]; ``bias2d`` the two-dimensional
    decomposable form (see ``_bias2d_args``); at most one of them is given.

    ``top_n=None`` keeps every key.  Returns a dict with ``out`` float32
    [nrows, d] (or [B,H,n,d] when rows is None), and optionally ``idx`` and
    ``aq8`` int32 [.., min(N,n)].
    """
    qbits = _c(qbits, np.uint32)
    kbits = _c(kbits, np.uint32)
    v = _c(v, np.float32)
    B, H, n, W = qbits.shape
    d = 32 * W
    assert v.shape == (B, H, n, d)
    N = n if top_n is None else int(top_n)
    keep = min(N, n)
    r = None if rows is None else _c(rows, np.int64)
    nrows = B * H * n if r is None else r.shape[0]
    out = np.zeros((nrows, d), np.float32)
    idx = np.zeros((nrows, keep), np.int32) if want_idx else None
    quant = av_mode in (AV_Q8, AV_Q4)
    a8 = np.zeros((nrows, keep), np.int32) if (want_aq8 and quant) else None
    vq = sc = None
    if quant:
        vq, sc = vquant(v, 127 if av_mode == AV_Q8 else 7)
    aq, ak, T = _c(alpha_q, np.float32), _c(alpha_k, np.float32), _c(bias, np.float32)
    assert bias is None or bias2d is None
    R, C, X, gh, gw, cls = _bias2d_args(bias2d, n)
    rc = _load().oracle_attention(_ptr(qbits), _ptr(kbits), _ptr(aq), _ptr(ak), _ptr(T), _ptr(R), _ptr(C), _ptr(X),
                                  gh, gw, cls, _ptr(v),
                                  _ptr(vq), _ptr(sc), B, H, n, d, N, av_mode, _ptr(r), nrows,
                                  _ptr(out), _ptr(idx), _ptr(a8))
    if rc != 0:
        raise OverflowError("int32 accumulator overflow in the quantized A*V")
    res = {"out": out if rows is not None else out.reshape(B, H, n, d)}
    if idx is not None:
        res["idx"] = idx if rows is not None else idx.reshape(B, H, n, keep)
    if a8 is not None:
        res["aq8"] = a8 if rows is not None else a8.reshape(B, H, n, keep)
    if quant:
        res["vq"], res["vscale"] = vq, sc
    return res
