"""GPU parity of binattn_dense_q8_fused (binarize, quantize and dense q8 attention in one launch).

Bar: the same bits as had_pack_qk followed by binattn_dense_q8 on the same
device inputs, and the oracle's pack + dense q8 attention within one int8 LSB of
V per output element (the quantized path's tolerance).
"""
import numpy as np
import pytest
import torch

import oracle
from binarized_qk_sparse_amd import ops, synth
from parity_util import f32, q8_tolerance, sample_rows

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    ops._lib.load()


def _inputs(B, H, n, d, qk_dtype, v_dtype, bias, seed):
    g = np.random.default_rng([31, B, H, n, d, seed])
    xq = (g.standard_normal((B, H, n, d)) + 0.5 * g.standard_normal((1, H, 1, d))).astype(np.float32)
    xk = (g.standard_normal((B, H, n, d)) - 0.5 * g.standard_normal((1, H, 1, d))).astype(np.float32)
    xq[0, 0, :, 1] = 0.75  # a constant channel: x - mu is exactly 0 there
    xk[-1, -1, 0, :8] = -0.0
    v = (g.standard_normal((B, H, n, d)) * g.uniform(0.2, 3.0, (1, H, 1, d))).astype(np.float32)
    v[0, -1, :, 2] = 0.0  # an all-zero channel: scale 0, int8 codes 0
    T = (0.02 * g.standard_normal((H, 2 * n - 1))).astype(np.float32) if bias else None
    return (torch.from_numpy(xq).to(qk_dtype), torch.from_numpy(xk).to(qk_dtype), torch.from_numpy(v).to(v_dtype),
            None if T is None else torch.from_numpy(T))


def _unfused(q, k, v, mode, T):
    B, H, n, d = q.shape
    ws = ops.workspace(B, H, n, d)
    (qb, aq, _), (kb, ak, _) = ops.had_pack_qk(q, k, mode, ws=ws)
    if mode == ops.HAD_SIGN:
        aq = ak = None
    return ops.binattn_dense_q8(qb, kb, v, alpha_q=aq, alpha_k=ak, bias=T, ws=ws)


CASES = [  # n, d, mode, qk dtype, v dtype, bias
    (1, 64, synth.MEAN_SIGN, torch.bfloat16, torch.bfloat16, True),
    (17, 64, synth.SIGN, torch.float32, torch.float32, False),
    (100, 64, synth.MEAN_SIGN, torch.float32, torch.bfloat16, True),
    (197, 64, synth.MEAN_SIGN, torch.bfloat16, torch.bfloat16, True),
    (197, 64, synth.SIGN, torch.bfloat16, torch.float32, True),
    (256, 64, synth.MEAN_SIGN, torch.bfloat16, torch.float32, False),
    (33, 128, synth.MEAN_SIGN, torch.bfloat16, torch.bfloat16, True),
    (197, 128, synth.SIGN, torch.float32, torch.bfloat16, True),
    (256, 128, synth.MEAN_SIGN, torch.float32, torch.float32, True),
]


@pytest.mark.parametrize("n,d,mode,qk_dtype,v_dtype,bias", CASES)
def test_fused_equals_separate_passes(n, d, mode, qk_dtype, v_dtype, bias):
    q, k, v, T = _inputs(2, 3, n, d, qk_dtype, v_dtype, bias, seed=1)
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    dT = None if T is None else T.to(DEV)
    fused = ops.binattn_dense_q8_fused(q, k, v, mode, bias=dT)
    separate = _unfused(q, k, v, mode, dT)
    torch.cuda.synchronize()
    assert torch.equal(fused, separate), f"n={n} d={d}: {int((fused != separate).sum())} elements differ"


@pytest.mark.parametrize("n,d,mode,qk_dtype,v_dtype,bias", CASES[::2])
def test_fused_matches_oracle(n, d, mode, qk_dtype, v_dtype, bias):
    q, k, v, T = _inputs(2, 3, n, d, qk_dtype, v_dtype, bias, seed=2)
    out = ops.binattn_dense_q8_fused(q.to(DEV), k.to(DEV), v.to(DEV), mode, bias=None if T is None else T.to(DEV))
    torch.cuda.synchronize()
    qb, aq, _ = oracle.pack(f32(q), mode)
    kb, ak, _ = oracle.pack(f32(k), mode)
    if mode == synth.SIGN:
        aq = ak = None
    ref = oracle.attention(qb, kb, f32(v), alpha_q=aq, alpha_k=ak, bias=None if T is None else T.numpy(),
                           top_n=None, av_mode=oracle.AV_Q8)
    rows = np.arange(2 * 3 * n)
    tol = q8_tolerance(ref["vscale"], rows, n)
    diff = np.abs(out.cpu().numpy().reshape(-1, d) - ref["out"].reshape(-1, d))
    assert np.all(diff <= tol + 1e-6), f"{int((diff > tol + 1e-6).sum())} elements beyond one int8 LSB"


def test_fused_c4_full_size():
    w = synth.workload("c4")
    g = synth.generate(w)
    q, k, v, T = g["q"].to(DEV), g["k"].to(DEV), g["v"].to(DEV), g["bias"].to(DEV)
    fused = ops.binattn_dense_q8_fused(q, k, v, w.mode, bias=T)
    separate = _unfused(q, k, v, w.mode, T)
    torch.cuda.synchronize()
    assert torch.equal(fused, separate)
    # and the oracle end to end on sampled query rows
    qb, aq, _ = oracle.pack(f32(g["q"]), w.mode)
    kb, ak, _ = oracle.pack(f32(g["k"]), w.mode)
    rows = sample_rows(w.B * w.H * w.n, 3000, 6)
    ref = oracle.attention(qb, kb, f32(g["v"]), alpha_q=aq, alpha_k=ak, bias=g["bias"].numpy(), top_n=None,
                           av_mode=oracle.AV_Q8, rows=rows)
    diff = np.abs(fused.cpu().numpy().reshape(-1, 64)[rows] - ref["out"])
    assert np.all(diff <= q8_tolerance(ref["vscale"], rows, w.n) + 1e-6)


def test_fused_rejects_bad_arguments():
    x = torch.zeros((1, 1, 300, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ops.HadError) as e:
        ops.binattn_dense_q8_fused(x, x, x, synth.MEAN_SIGN)
    assert e.value.status == ops._lib.HAD_ERR_UNSUPPORTED
