"""The Python binding rejects malformed tensor arguments before anything reaches the library.

These run on the CPU: the argument checks take the device to compare against as a
parameter, so CPU tensors stand in for device tensors here; the public functions
themselves refuse host tensors outright.
"""
import numpy as np
import pytest
import torch

from binarized_qk_sparse_amd import ops

CPU = torch.device("cpu")
B, H, n, d = 2, 3, 17, 64


def _good(**over):
    args = dict(
        qbits=torch.zeros((B, H, n, d // 32), dtype=torch.int32),
        kbits=torch.zeros((B, H, n, d // 32), dtype=torch.int32),
        v=torch.zeros((B, H, n, d), dtype=torch.bfloat16),
        alpha_q=torch.ones((B, H, n), dtype=torch.float32),
        alpha_k=torch.ones((B, H, n), dtype=torch.float32),
        bias=torch.zeros((H, 2 * n - 1), dtype=torch.float32),
        out=torch.empty((B, H, n, d), dtype=torch.float32),
        ws=torch.empty(ops.workspace_bytes(B, H, n, d), dtype=torch.uint8),
    )
    args.update(over)
    return args


def _call(args):
    a = dict(args)
    return ops._check_attention_args(a.pop("qbits"), a.pop("kbits"), a.pop("v"), CPU, **a)


def test_well_formed_arguments_pass():
    assert _call(_good()) == (B, H, n, d)
    assert _call(_good(alpha_q=None, alpha_k=None, bias=None, out=None, ws=None)) == (B, H, n, d)


@pytest.mark.parametrize("name,bad", [
    ("qbits", torch.zeros((B, H, n, 1), dtype=torch.int32)),           # d/32 words wrong
    ("qbits", torch.zeros((B, H, n, 2), dtype=torch.int64)),           # wrong dtype
    ("kbits", torch.zeros((B, H, n + 1, 2), dtype=torch.int32)),       # wrong n
    ("kbits", None),                                                   # required
    ("alpha_q", torch.ones((B, H, n), dtype=torch.float64)),           # float64 alpha
    ("alpha_q", torch.ones((B, H, n), dtype=torch.bfloat16)),          # bf16 alpha
    ("alpha_k", torch.ones((B, H, n - 1), dtype=torch.float32)),       # short alpha
    ("bias", torch.zeros((H, 2 * n), dtype=torch.float32)),            # wrong table length
    ("bias", torch.zeros((H + 1, 2 * n - 1), dtype=torch.float32)),    # wrong head count
    ("out", torch.empty((B, H, n, d), dtype=torch.bfloat16)),          # out must be float32
    ("out", torch.empty((B, H, n, d // 2), dtype=torch.float32)),      # mis-shaped out
    ("ws", torch.empty(16, dtype=torch.uint8)),                        # workspace too small
    ("ws", torch.empty(ops.workspace_bytes(B, H, n, d), dtype=torch.int8)),  # wrong dtype
    ("v", torch.zeros((B, H, n, d), dtype=torch.float16)),             # unsupported V dtype
    ("v", torch.zeros((B, H, n, 48), dtype=torch.float32)),            # d not a multiple of 32
    ("v", torch.zeros((H, n, d), dtype=torch.float32)),                # not 4-D
])
def test_malformed_argument_is_rejected(name, bad):
    with pytest.raises((ValueError, TypeError)):
        _call(_good(**{name: bad}))


def test_non_contiguous_tensors_are_rejected():
    t = torch.ones((B, H, 2 * n), dtype=torch.float32)[:, :, ::2]
    with pytest.raises(ValueError, match="contiguous"):
        _call(_good(alpha_q=t))
    o = torch.empty((B, H, d, n), dtype=torch.float32).transpose(2, 3)
    with pytest.raises(ValueError, match="contiguous"):
        _call(_good(out=o))


def test_tensor_on_another_device_is_rejected():
    meta = torch.ones((B, H, n), dtype=torch.float32, device="meta")
    with pytest.raises(ValueError, match="expected cpu"):
        _call(_good(alpha_k=meta))


def _bias2d(gh=3, gw=5, with_cls=True, **over):
    b = {"grid": (gh, gw),
         "row": torch.zeros((H, 2 * gh - 1), dtype=torch.float32),
         "col": torch.zeros((H, 2 * gw - 1), dtype=torch.float32)}
    if with_cls:
        b["cls"] = torch.zeros((H, 3), dtype=torch.float32)
    b.update(over)
    return b


def test_two_dimensional_bias_tables_are_checked_against_the_grid():
    ok = _good(bias=None)
    ok["v"] = torch.zeros((B, H, 16, d), dtype=torch.bfloat16)
    ok["qbits"] = ok["kbits"] = torch.zeros((B, H, 16, 2), dtype=torch.int32)
    ok.update(alpha_q=None, alpha_k=None, out=None, ws=None)
    assert _call({**ok, "bias2d": _bias2d()}) == (B, H, 16, d)
    bad = [
        _bias2d(gh=4),                                                        # n != grid + class token
        _bias2d(with_cls=False),                                              # n != grid
        _bias2d(row=torch.zeros((H, 4), dtype=torch.float32)),                # row table length
        _bias2d(col=torch.zeros((H, 9), dtype=torch.float64)),                # column table dtype
        _bias2d(cls=torch.zeros((H, 2), dtype=torch.float32)),                # class values
    ]
    for b in bad:
        with pytest.raises(ValueError):
            _call({**ok, "bias2d": b})
    with pytest.raises(ValueError, match="not both"):
        _call({**ok, "bias2d": _bias2d(), "bias": torch.zeros((H, 31), dtype=torch.float32)})


def test_public_entry_points_refuse_host_tensors():
    a = _good()
    with pytest.raises(ValueError, match="GPU tensor"):
        ops.had_attention_topn(a["qbits"], a["kbits"], a["v"], 5)
    with pytest.raises(ValueError, match="GPU tensor"):
        ops.binattn_dense_q8(a["qbits"], a["kbits"], a["v"])
    with pytest.raises(ValueError, match="GPU tensor"):
        ops.had_pack(a["v"])
    with pytest.raises(ValueError, match="GPU tensor"):
        ops.binattn_dense_q8_fused(a["v"], a["v"], a["v"])


def test_workspace_regions_come_from_the_library():
    from binarized_qk_sparse_amd import _lib
    import ctypes

    lib = _lib.load()
    off, nb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert lib.had_workspace_region(B, H, n, d, _lib.HAD_WS_VQ, ctypes.byref(off), ctypes.byref(nb)) == 0
    assert nb.value == B * H * n * d and off.value % 256 == 0
    vq_end = off.value + nb.value
    assert lib.had_workspace_region(B, H, n, d, _lib.HAD_WS_VSCALE, ctypes.byref(off), ctypes.byref(nb)) == 0
    assert nb.value == 4 * B * H * d and off.value >= vq_end and off.value % 256 == 0
    assert off.value + nb.value <= ops.workspace_bytes(B, H, n, d)
    assert lib.had_workspace_region(B, H, n, d, 7, ctypes.byref(off), ctypes.byref(nb)) == _lib.HAD_ERR_INVALID_ARG
    assert lib.had_workspace_region(0, H, n, d, 0, ctypes.byref(off), ctypes.byref(nb)) == _lib.HAD_ERR_INVALID_ARG
    ws = torch.zeros(ops.workspace_bytes(B, H, n, d), dtype=torch.uint8)
    vq, sc = ops.workspace_view(ws, B, H, n, d)
    assert vq.shape == (B, H, n, d) and vq.dtype == torch.int8
    assert sc.shape == (B, H, d) and sc.dtype == torch.float32
    # 4-bit V: two codes per byte in the same region
    vq4, _ = ops.workspace_view(ws, B, H, n, d, av_mode=ops.HAD_AV_Q4)
    assert vq4.shape == (B, H, n, d // 2) and vq4.dtype == torch.uint8


def test_unpack_q4_reads_two_codes_per_byte():
    from parity_util import unpack_q4

    codes = np.array([[-7, 7, 0, -1, 3, -4, 1, 2]], np.int8)
    packed = np.array([[(int(c0) & 0xF) | ((int(c1) & 0xF) << 4) for c0, c1 in zip(codes[0, 0::2], codes[0, 1::2])]],
                      np.uint8)
    assert packed.tolist() == [[0x79, 0xF0, 0xC3, 0x21]]
    assert np.array_equal(unpack_q4(packed), codes)
