"""ctypes loader for ``libhad.so`` (the C ABI declared in include/had.h).

Loading the library does not touch the GPU; the HIP runtime initialises on the
first kernel launch.  If the library has not been built the import of the
ops fails loudly: there is no other execution path.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhad.so")

# Constants of include/had.h
HAD_OK = 0
HAD_ERR_INVALID_ARG = 1
HAD_ERR_UNSUPPORTED = 2
HAD_ERR_WORKSPACE = 3
HAD_ERR_HIP = 4
HAD_F32 = 0
HAD_BF16 = 1
HAD_SIGN = 0
HAD_MEAN_SIGN = 1
HAD_AV_F32 = 0
HAD_AV_Q8 = 1
HAD_AV_Q4 = 2
HAD_WS_VQ = 0
HAD_WS_VSCALE = 1
HAD_ABI_VERSION = 1
HAD_NOALLOC_SCRATCH_BYTES = 64 << 20

EXPORTS = (
    "had_abi_version",
    "had_status_str",
    "had_workspace_bytes",
    "had_workspace_region",
    "had_pack",
    "had_pack_qk",
    "had_attention_topn",
    "binattn_dense_q8",
    "binattn_dense_q8_fused",
    "had_attention_topn_2d",
    "binattn_dense_q8_2d",
    "binattn_dense_q8_noalloc",
    "had_attention_topn_fused",
)

_lib = None


class HadError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status_str(status)} ({status})")
        self.status = status


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m binarized_qk_sparse_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, I64, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    lib.had_abi_version.argtypes = []
    lib.had_abi_version.restype = I
    lib.had_status_str.argtypes = [I]
    lib.had_status_str.restype = ctypes.c_char_p
    lib.had_workspace_bytes.argtypes = [I64, I64, I64, I64]
    lib.had_workspace_bytes.restype = SZ
    lib.had_workspace_region.argtypes = [I64, I64, I64, I64, I, ctypes.POINTER(SZ), ctypes.POINTER(SZ)]
    lib.had_workspace_region.restype = I
    lib.had_pack.argtypes = [P, I, I64, I64, I64, I64, I, P, P, P, P, SZ, P]
    lib.had_pack.restype = I
    lib.had_pack_qk.argtypes = [P, P, I, I64, I64, I64, I64, I, P, P, P, P, P, P, P, SZ, P]
    lib.had_pack_qk.restype = I
    lib.had_attention_topn.argtypes = [P, P, P, P, P, P, I, I64, I64, I64, I64, I64, I, P, P, P, SZ, P]
    lib.had_attention_topn.restype = I
    lib.binattn_dense_q8.argtypes = [P, P, P, P, P, P, I, I64, I64, I64, I64, P, P, SZ, P]
    lib.binattn_dense_q8.restype = I
    lib.binattn_dense_q8_fused.argtypes = [P, P, I, I, P, P, I, I64, I64, I64, I64, P, P]
    lib.binattn_dense_q8_fused.restype = I
    lib.had_attention_topn_2d.argtypes = [P, P, P, P, P, P, P, I64, I64, P, I, I64, I64, I64, I64, I64, I, P, P, P,
                                          SZ, P]
    lib.had_attention_topn_2d.restype = I
    lib.binattn_dense_q8_2d.argtypes = [P, P, P, P, P, P, P, I64, I64, P, I, I64, I64, I64, I64, P, P, SZ, P]
    lib.binattn_dense_q8_2d.restype = I
    lib.binattn_dense_q8_noalloc.argtypes = [P, P, P, P, P, P, I, I64, I64, I64, I64, P, P]
    lib.binattn_dense_q8_noalloc.restype = I
    lib.had_attention_topn_fused.argtypes = [P, P, I, I, P, P, I, I64, I64, I64, I64, I64, P, P, P]
    lib.had_attention_topn_fused.restype = I
    if lib.had_abi_version() != HAD_ABI_VERSION:
        raise ImportError("libhad.so ABI version mismatch")
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load().had_status_str(int(status)).decode()


def check(fn: str, status: int) -> None:
    if status != HAD_OK:
        raise HadError(fn, status)
