"""The C-ABI library loads without a GPU, exports every declared entry point,
and rejects bad arguments before touching the HIP runtime."""
import ctypes
import os
import re

import pytest

from binarized_qk_sparse_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    with open(os.path.join(ROOT, "include", "had.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(had_\w+|binattn_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    names = _declared_functions()
    assert set(names) == set(_lib.EXPORTS)
    for name in names:
        assert hasattr(lib, name), name


def test_ceiling_library_loads_and_exports():
    """libhad_ubench.so (the measured VALU, v_exp, co-issue and copy ceilings bench.py reports) is
    built beside libhad.so and exports its three launchers; they reject bad sizes before any launch."""
    lib = ctypes.CDLL(os.path.join(ROOT, "binarized_qk_sparse_amd", "libhad_ubench.so"))
    for name in ("hub_xor_bcnt", "hub_exp"):
        f = getattr(lib, name)
        f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        assert f(None, 1, 1, None) == 1
        assert f(ctypes.c_void_p(256), 0, 1, None) == 1
    f = lib.hub_coissue
    f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    assert f(None, 1, 1, 1, None) == 1
    assert f(ctypes.c_void_p(256), 1, 0, 0, None) == 1


def test_header_constants_match_binding():
    with open(os.path.join(ROOT, "include", "had.h")) as f:
        text = f.read()
    defs = dict(re.findall(r"#define\s+(HAD_\w+)\s+(\d+)", text))
    for k, v in defs.items():
        if hasattr(_lib, k):
            assert getattr(_lib, k) == int(v), k


def test_status_strings_and_version():
    assert _lib.load().had_abi_version() == _lib.HAD_ABI_VERSION
    for code, name in [(0, "HAD_OK"), (1, "HAD_ERR_INVALID_ARG"), (2, "HAD_ERR_UNSUPPORTED"),
                       (3, "HAD_ERR_WORKSPACE"), (4, "HAD_ERR_HIP"), (99, "HAD_ERR_UNKNOWN")]:
        assert _lib.status_str(code) == name


def test_workspace_bytes():
    lib = _lib.load()
    a = lib.had_workspace_bytes(1, 1, 100, 64)
    b = lib.had_workspace_bytes(2, 1, 100, 64)
    assert a > 0 and a % 256 == 0 and b > a
    assert lib.had_workspace_bytes(0, 1, 100, 64) == 0
    # c5 shape: int8 V plus scales and partials
    assert lib.had_workspace_bytes(1, 16, 16384, 64) >= 16 * 16384 * 64


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


@pytest.mark.parametrize("args,want", [
    (dict(x=None), _lib.HAD_ERR_INVALID_ARG),
    (dict(bits=None), _lib.HAD_ERR_INVALID_ARG),
    (dict(B=0), _lib.HAD_ERR_INVALID_ARG),
    (dict(n=-1), _lib.HAD_ERR_INVALID_ARG),
    (dict(dtype=7), _lib.HAD_ERR_INVALID_ARG),
    (dict(mode=5), _lib.HAD_ERR_INVALID_ARG),
    (dict(d=48), _lib.HAD_ERR_UNSUPPORTED),
    (dict(d=256), _lib.HAD_ERR_UNSUPPORTED),
    (dict(n=70000), _lib.HAD_ERR_UNSUPPORTED),
    (dict(n=65537), _lib.HAD_ERR_UNSUPPORTED),
    (dict(mode=1, alpha=None), _lib.HAD_ERR_INVALID_ARG),
    (dict(mode=1, ws=None), _lib.HAD_ERR_WORKSPACE),
    (dict(mode=1, wsz=16), _lib.HAD_ERR_WORKSPACE),
])
def test_pack_validation(args, want):
    a = dict(x=FAKE, dtype=_lib.HAD_BF16, B=1, H=1, n=64, d=64, mode=0, bits=FAKE, alpha=FAKE, mu=FAKE,
             ws=FAKE, wsz=1 << 30)
    a.update(args)
    st = _lib.load().had_pack(a["x"], a["dtype"], a["B"], a["H"], a["n"], a["d"], a["mode"], a["bits"],
                              a["alpha"], a["mu"], a["ws"], a["wsz"], None)
    assert st == want


@pytest.mark.parametrize("args,want", [
    (dict(q=None), _lib.HAD_ERR_INVALID_ARG),
    (dict(k=None), _lib.HAD_ERR_INVALID_ARG),
    (dict(kbits=None), _lib.HAD_ERR_INVALID_ARG),
    (dict(H=0), _lib.HAD_ERR_INVALID_ARG),
    (dict(mode=3), _lib.HAD_ERR_INVALID_ARG),
    (dict(d=96), _lib.HAD_ERR_UNSUPPORTED),
    (dict(mode=1, mu_k=None), _lib.HAD_ERR_INVALID_ARG),
    (dict(mode=1, ws=None), _lib.HAD_ERR_WORKSPACE),
    (dict(mode=1, wsz=64), _lib.HAD_ERR_WORKSPACE),
])
def test_pack_qk_validation(args, want):
    a = dict(q=FAKE, k=FAKE, dtype=_lib.HAD_F32, B=1, H=2, n=64, d=64, mode=0, qbits=FAKE, kbits=FAKE,
             alpha_q=FAKE, alpha_k=FAKE, mu_q=FAKE, mu_k=FAKE, ws=FAKE, wsz=1 << 30)
    a.update(args)
    st = _lib.load().had_pack_qk(a["q"], a["k"], a["dtype"], a["B"], a["H"], a["n"], a["d"], a["mode"],
                                 a["qbits"], a["kbits"], a["alpha_q"], a["alpha_k"], a["mu_q"], a["mu_k"],
                                 a["ws"], a["wsz"], None)
    assert st == want


@pytest.mark.parametrize("args,want", [
    (dict(q=None), _lib.HAD_ERR_INVALID_ARG),
    (dict(v=None), _lib.HAD_ERR_INVALID_ARG),
    (dict(out=None), _lib.HAD_ERR_INVALID_ARG),
    (dict(top_n=0), _lib.HAD_ERR_INVALID_ARG),
    (dict(av=3), _lib.HAD_ERR_INVALID_ARG),
    (dict(vdt=9), _lib.HAD_ERR_INVALID_ARG),
    (dict(H=0), _lib.HAD_ERR_INVALID_ARG),
    (dict(d=32), _lib.HAD_ERR_UNSUPPORTED),
    (dict(d=256), _lib.HAD_ERR_UNSUPPORTED),
    (dict(n=1 << 20), _lib.HAD_ERR_UNSUPPORTED),
    (dict(n=65537), _lib.HAD_ERR_UNSUPPORTED),
    (dict(av=1, ws=None), _lib.HAD_ERR_WORKSPACE),
    (dict(av=1, wsz=100), _lib.HAD_ERR_WORKSPACE),
    (dict(av=1, ws=ctypes.c_void_p(0x1001)), _lib.HAD_ERR_WORKSPACE),
])
def test_attention_validation(args, want):
    a = dict(q=FAKE, k=FAKE, aq=None, ak=None, bias=None, v=FAKE, vdt=_lib.HAD_BF16, B=1, H=1, n=256, d=64,
             top_n=30, av=0, out=FAKE, idx=None, ws=FAKE, wsz=1 << 30)
    a.update(args)
    st = _lib.load().had_attention_topn(a["q"], a["k"], a["aq"], a["ak"], a["bias"], a["v"], a["vdt"], a["B"],
                                        a["H"], a["n"], a["d"], a["top_n"], a["av"], a["out"], a["idx"], a["ws"],
                                        a["wsz"], None)
    assert st == want


@pytest.mark.parametrize("args,want", [
    (dict(k=None), _lib.HAD_ERR_INVALID_ARG),
    (dict(n=0), _lib.HAD_ERR_INVALID_ARG),
    (dict(d=32), _lib.HAD_ERR_UNSUPPORTED),
    (dict(n=65537), _lib.HAD_ERR_UNSUPPORTED),
    (dict(ws=None), _lib.HAD_ERR_WORKSPACE),
    (dict(wsz=0), _lib.HAD_ERR_WORKSPACE),
])
def test_dense_validation(args, want):
    a = dict(q=FAKE, k=FAKE, v=FAKE, B=2, H=3, n=197, d=64, out=FAKE, ws=FAKE, wsz=1 << 30)
    a.update(args)
    st = _lib.load().binattn_dense_q8(a["q"], a["k"], None, None, None, a["v"], _lib.HAD_BF16, a["B"], a["H"],
                                      a["n"], a["d"], a["out"], a["ws"], a["wsz"], None)
    assert st == want


@pytest.mark.parametrize("args,want", [
    (dict(q=None), _lib.HAD_ERR_INVALID_ARG),
    (dict(v=None), _lib.HAD_ERR_INVALID_ARG),
    (dict(out=None), _lib.HAD_ERR_INVALID_ARG),
    (dict(B=0), _lib.HAD_ERR_INVALID_ARG),
    (dict(qkdt=5), _lib.HAD_ERR_INVALID_ARG),
    (dict(vdt=5), _lib.HAD_ERR_INVALID_ARG),
    (dict(mode=2), _lib.HAD_ERR_INVALID_ARG),
    (dict(d=32), _lib.HAD_ERR_UNSUPPORTED),
    (dict(n=257), _lib.HAD_ERR_UNSUPPORTED),
])
def test_dense_fused_validation(args, want):
    a = dict(q=FAKE, k=FAKE, qkdt=_lib.HAD_BF16, mode=_lib.HAD_MEAN_SIGN, v=FAKE, vdt=_lib.HAD_BF16, B=2, H=3, n=197,
             d=64, out=FAKE)
    a.update(args)
    st = _lib.load().binattn_dense_q8_fused(a["q"], a["k"], a["qkdt"], a["mode"], None, a["v"], a["vdt"], a["B"],
                                            a["H"], a["n"], a["d"], a["out"], None)
    assert st == want


@pytest.mark.parametrize("args,want", [
    (dict(q=None), _lib.HAD_ERR_INVALID_ARG),
    (dict(k=None), _lib.HAD_ERR_INVALID_ARG),
    (dict(out=None), _lib.HAD_ERR_INVALID_ARG),
    (dict(H=0), _lib.HAD_ERR_INVALID_ARG),
    (dict(qkdt=5), _lib.HAD_ERR_INVALID_ARG),
    (dict(vdt=5), _lib.HAD_ERR_INVALID_ARG),
    (dict(mode=7), _lib.HAD_ERR_INVALID_ARG),
    (dict(top_n=0), _lib.HAD_ERR_INVALID_ARG),
    (dict(d=96), _lib.HAD_ERR_UNSUPPORTED),
    (dict(n=257), _lib.HAD_ERR_UNSUPPORTED),                            # mean-centred: n <= 256
    (dict(mode=_lib.HAD_SIGN, vdt=_lib.HAD_F32, n=513), _lib.HAD_ERR_UNSUPPORTED),
    (dict(mode=_lib.HAD_SIGN, n=1025), _lib.HAD_ERR_UNSUPPORTED),
    (dict(mode=_lib.HAD_SIGN, d=128, n=513), _lib.HAD_ERR_UNSUPPORTED),
])
def test_topn_fused_validation(args, want):
    a = dict(q=FAKE, k=FAKE, qkdt=_lib.HAD_F32, mode=_lib.HAD_MEAN_SIGN, v=FAKE, vdt=_lib.HAD_BF16, B=2, H=3, n=197,
             d=64, top_n=30, out=FAKE)
    a.update(args)
    st = _lib.load().had_attention_topn_fused(a["q"], a["k"], a["qkdt"], a["mode"], None, a["v"], a["vdt"], a["B"],
                                              a["H"], a["n"], a["d"], a["top_n"], a["out"], None, None)
    assert st == want


@pytest.mark.parametrize("args,want", [
    (dict(row=None), _lib.HAD_ERR_INVALID_ARG),
    (dict(col=None), _lib.HAD_ERR_INVALID_ARG),
    (dict(gh=0), _lib.HAD_ERR_INVALID_ARG),
    (dict(n=196), _lib.HAD_ERR_INVALID_ARG),                 # class token given: n must be 197
    (dict(cls=None), _lib.HAD_ERR_INVALID_ARG),              # no class token: n must be 196
    (dict(gh=1, gw=5000, n=5001), _lib.HAD_ERR_UNSUPPORTED),  # long sequence, tables above its LDS space
    (dict(gh=40000, gw=1, n=40001), _lib.HAD_ERR_UNSUPPORTED),
    (dict(q=None), _lib.HAD_ERR_INVALID_ARG),
])
def test_attention_2d_validation(args, want):
    a = dict(q=FAKE, k=FAKE, row=FAKE, col=FAKE, cls=FAKE, gh=14, gw=14, v=FAKE, vdt=_lib.HAD_BF16, B=1, H=1, n=197,
             d=64, top_n=30, av=0, out=FAKE, ws=FAKE, wsz=1 << 30)
    a.update(args)
    st = _lib.load().had_attention_topn_2d(a["q"], a["k"], None, None, a["row"], a["col"], a["cls"], a["gh"], a["gw"],
                                           a["v"], a["vdt"], a["B"], a["H"], a["n"], a["d"], a["top_n"], a["av"],
                                           a["out"], None, a["ws"], a["wsz"], None)
    assert st == want


def test_dense_2d_validation():
    lib = _lib.load()
    st = lib.binattn_dense_q8_2d(FAKE, FAKE, None, None, FAKE, FAKE, None, 14, 14, FAKE, _lib.HAD_BF16, 1, 1, 197, 64,
                                 FAKE, FAKE, 1 << 30, None)
    assert st == _lib.HAD_ERR_INVALID_ARG  # 14 x 14 without a class token is 196 tokens
    st = lib.binattn_dense_q8_2d(FAKE, FAKE, None, None, FAKE, None, FAKE, 14, 14, FAKE, _lib.HAD_BF16, 1, 1, 197, 64,
                                 FAKE, FAKE, 1 << 30, None)
    assert st == _lib.HAD_ERR_INVALID_ARG


@pytest.mark.parametrize("args,want", [
    (dict(q=None), _lib.HAD_ERR_INVALID_ARG),
    (dict(out=None), _lib.HAD_ERR_INVALID_ARG),
    (dict(n=0), _lib.HAD_ERR_INVALID_ARG),
    (dict(vdt=4), _lib.HAD_ERR_INVALID_ARG),
    (dict(d=32), _lib.HAD_ERR_UNSUPPORTED),
    # a workspace of more than the static scratch: 256 x 16 heads x 256 tokens x 64 channels of int8 V
    (dict(B=256, H=16, n=256), _lib.HAD_ERR_UNSUPPORTED),
])
def test_dense_noalloc_validation(args, want):
    # every rejection happens before any HIP call (none is possible on this host)
    a = dict(q=FAKE, k=FAKE, v=FAKE, vdt=_lib.HAD_BF16, B=2, H=3, n=197, d=64, out=FAKE)
    a.update(args)
    st = _lib.load().binattn_dense_q8_noalloc(a["q"], a["k"], None, None, None, a["v"], a["vdt"], a["B"], a["H"],
                                              a["n"], a["d"], a["out"], None)
    assert st == want


def test_noalloc_scratch_limit_matches_header():
    with open(os.path.join(ROOT, "include", "had.h")) as f:
        text = f.read()
    m = re.search(r"#define\s+HAD_NOALLOC_SCRATCH_BYTES\s+\(\(size_t\)(\d+)\s*<<\s*(\d+)\)", text)
    assert m is not None
    assert int(m.group(1)) << int(m.group(2)) == _lib.HAD_NOALLOC_SCRATCH_BYTES
    lib = _lib.load()
    assert lib.had_workspace_bytes(256, 16, 256, 64) > _lib.HAD_NOALLOC_SCRATCH_BYTES
    assert lib.had_workspace_bytes(64, 12, 197, 64) <= _lib.HAD_NOALLOC_SCRATCH_BYTES  # the DeiT-B dense workload
