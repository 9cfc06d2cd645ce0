"""GPU parity of the two-dimensional decomposable bias entry points (had_attention_topn_2d,
binattn_dense_q8_2d) against the oracle.

Bar: kept index sets bit-exact; fp32 outputs within 1e-3 relative + 1e-4 absolute; the
quantized paths within one int8 LSB of V per output element.
"""
import numpy as np
import pytest
import torch

import oracle
from binarized_qk_sparse_amd import ops, synth
from parity_util import assert_close, f32, q8_tolerance, rows_per_head, sample_rows, ws_vq

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    ops._lib.load()


def _case(B, H, gh, gw, cls, d, mode, vdtype, seed):
    n = cls + gh * gw
    g = np.random.default_rng([51, B, H, gh, gw, cls, d, seed])
    xq = (g.standard_normal((B, H, n, d)) + 0.3 * g.standard_normal((1, H, 1, d))).astype(np.float32)
    xk = (g.standard_normal((B, H, n, d)) + 0.3 * g.standard_normal((1, H, 1, d))).astype(np.float32)
    v = torch.from_numpy(g.standard_normal((B, H, n, d)).astype(np.float32)).to(vdtype)
    b2 = {"grid": (gh, gw), "row": (0.2 * g.standard_normal((H, 2 * gh - 1))).astype(np.float32),
          "col": (0.2 * g.standard_normal((H, 2 * gw - 1))).astype(np.float32)}
    if cls:
        b2["cls"] = (0.2 * g.standard_normal((H, 3))).astype(np.float32)
    qb, aq, _ = oracle.pack(xq, mode)
    kb, ak, _ = oracle.pack(xk, mode)
    if mode == synth.SIGN:
        aq = ak = None
    return n, qb, kb, aq, ak, b2, v


def _dev2d(b2):
    return {k: (torch.from_numpy(x).to(DEV) if isinstance(x, np.ndarray) else x) for k, x in b2.items()}


def _dt(a):
    return None if a is None else torch.from_numpy(a).to(DEV)


@pytest.mark.parametrize("gh,gw,cls,N,d,mode,vdtype", [
    (8, 8, 1, 10, 64, synth.MEAN_SIGN, torch.bfloat16),   # resident kernel, class token
    (16, 16, 0, 30, 64, synth.SIGN, torch.float32),       # resident kernel, plain sign
    (3, 7, 1, 5, 128, synth.MEAN_SIGN, torch.bfloat16),   # resident kernel, head_dim 128
    (1, 40, 0, 12, 64, synth.SIGN, torch.bfloat16),       # one grid row: the 1-D table's case
    (40, 40, 1, 64, 64, synth.MEAN_SIGN, torch.bfloat16),  # long-sequence kernel (n = 1601)
    (20, 30, 0, 100, 128, synth.SIGN, torch.bfloat16),     # long-sequence kernel at head_dim 128
    (1, 1, 0, 3, 64, synth.SIGN, torch.float32),           # a single token
    (1, 1, 1, 1, 64, synth.MEAN_SIGN, torch.bfloat16),     # class token and one patch
    (2, 1, 1, 5, 64, synth.MEAN_SIGN, torch.bfloat16),     # one grid column, N >= n
])
def test_topn_bias2d_matches_oracle(gh, gw, cls, N, d, mode, vdtype):
    n, qb, kb, aq, ak, b2, v = _case(1, 2, gh, gw, cls, d, mode, vdtype, seed=1)
    out, idx = ops.had_attention_topn(_dt(qb.view(np.int32)), _dt(kb.view(np.int32)), v.to(DEV), N, alpha_q=_dt(aq),
                                      alpha_k=_dt(ak), bias2d=_dev2d(b2), want_idx=True)
    torch.cuda.synchronize()
    rows = sample_rows(2 * n, 500, n)
    ref = oracle.attention(qb, kb, f32(v), alpha_q=aq, alpha_k=ak, bias2d=b2, top_n=N, rows=rows, want_idx=True)
    keep = min(N, n)
    assert np.array_equal(idx.cpu().numpy().reshape(-1, keep)[rows], ref["idx"]), "kept index sets differ"
    assert_close(out.cpu().numpy().reshape(-1, d)[rows], ref["out"], f"2-D bias {gh}x{gw}+{cls}")


@pytest.mark.parametrize("av", [synth.AV_Q8, synth.AV_Q4])
@pytest.mark.parametrize("gh,gw,cls", [(48, 48, 0), (16, 20, 1)])  # long-sequence, resident kernel
def test_topn_bias2d_quantized(av, gh, gw, cls):
    n, qb, kb, aq, ak, b2, v = _case(1, 2, gh, gw, cls, 64, synth.MEAN_SIGN, torch.bfloat16, seed=2)
    ws = ops.workspace(1, 2, n, 64)
    out, idx = ops.had_attention_topn(_dt(qb.view(np.int32)), _dt(kb.view(np.int32)), v.to(DEV), 256,
                                      alpha_q=_dt(aq), alpha_k=_dt(ak), bias2d=_dev2d(b2), av_mode=av,
                                      want_idx=True, ws=ws)
    torch.cuda.synchronize()
    rows = sample_rows(2 * n, 300, 7)
    ref = oracle.attention(qb, kb, f32(v), alpha_q=aq, alpha_k=ak, bias2d=b2, top_n=256, av_mode=av, rows=rows,
                           want_idx=True)
    assert np.array_equal(idx.cpu().numpy().reshape(-1, 256)[rows], ref["idx"])
    vq, sc = ws_vq(ws, 1, 2, n, 64, av)
    assert np.array_equal(vq.cpu().numpy(), ref["vq"]) and np.array_equal(sc.cpu().numpy(), ref["vscale"])
    diff = np.abs(out.cpu().numpy().reshape(-1, 64)[rows] - ref["out"])
    assert np.all(diff <= q8_tolerance(ref["vscale"], rows, n) + 1e-6)


@pytest.mark.parametrize("gh,gw,cls,d", [(14, 14, 1, 64), (5, 9, 0, 64), (7, 7, 1, 128)])
def test_dense_bias2d_matches_oracle(gh, gw, cls, d):
    n, qb, kb, aq, ak, b2, v = _case(2, 3, gh, gw, cls, d, synth.MEAN_SIGN, torch.bfloat16, seed=3)
    ws = ops.workspace(2, 3, n, d)
    out = ops.binattn_dense_q8(_dt(qb.view(np.int32)), _dt(kb.view(np.int32)), v.to(DEV), alpha_q=_dt(aq),
                               alpha_k=_dt(ak), bias2d=_dev2d(b2), ws=ws)
    torch.cuda.synchronize()
    ref = oracle.attention(qb, kb, f32(v), alpha_q=aq, alpha_k=ak, bias2d=b2, top_n=None, av_mode=oracle.AV_Q8)
    vq, sc = ops.workspace_view(ws, 2, 3, n, d)
    assert np.array_equal(vq.cpu().numpy(), ref["vq"])
    rows = np.arange(2 * 3 * n)
    diff = np.abs(out.cpu().numpy().reshape(-1, d) - ref["out"].reshape(-1, d))
    assert np.all(diff <= q8_tolerance(ref["vscale"], rows, n) + 1e-6)


def test_bias2d_single_row_equals_1d_table_on_device():
    # one grid row without a class token is the 1-D offset table R[0] + C: same bits on the GPU
    n, qb, kb, aq, ak, b2, v = _case(1, 2, 1, 300, 0, 64, synth.MEAN_SIGN, torch.bfloat16, seed=4)
    T = (b2["row"][:, :1] + b2["col"]).astype(np.float32)
    args = (_dt(qb.view(np.int32)), _dt(kb.view(np.int32)), v.to(DEV), 30)
    o2, i2 = ops.had_attention_topn(*args, alpha_q=_dt(aq), alpha_k=_dt(ak), bias2d=_dev2d(b2), want_idx=True)
    o1, i1 = ops.had_attention_topn(*args, alpha_q=_dt(aq), alpha_k=_dt(ak), bias=_dt(T), want_idx=True)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2) and torch.equal(o1, o2)


@pytest.mark.parametrize("name", ["c4b2d", "c5b2d"])
def test_bias2d_full_size_workloads(name):
    # c5b2d runs the long-sequence kernel with sixteen waves (n = 16384); c4b2d the dense kernel
    w = synth.workload(name)
    g = synth.generate(w)
    ws = ops.workspace(w.B, w.H, w.n, w.d)
    q, k, v = g["q"].to(DEV), g["k"].to(DEV), g["v"].to(DEV)
    qb, aq, _ = ops.had_pack(q, w.mode, ws=ws)
    kb, ak, _ = ops.had_pack(k, w.mode, ws=ws)
    b2 = {key: (x.to(DEV) if hasattr(x, "to") else x) for key, x in g["bias2d"].items()}
    if w.top_n is None:
        out = ops.binattn_dense_q8(qb, kb, v, alpha_q=aq, alpha_k=ak, bias2d=b2, ws=ws)
        idx = None
    else:
        out, idx = ops.had_attention_topn(qb, kb, v, w.top_n, alpha_q=aq, alpha_k=ak, bias2d=b2, av_mode=w.av_mode,
                                          want_idx=True, ws=ws)
    torch.cuda.synchronize()
    ob, oaq, _ = oracle.pack(f32(g["q"]), w.mode)
    okb, oak, _ = oracle.pack(f32(g["k"]), w.mode)
    # every row of c4b2d; 256 rows from every head of c5b2d (the oracle sorts 16384 keys per row)
    rows = np.arange(w.B * w.H * w.n, dtype=np.int64) if w.n <= 1024 else rows_per_head(w.B * w.H, w.n, 256, 8)
    ob2 = {key: (x.numpy() if hasattr(x, "numpy") else x) for key, x in g["bias2d"].items()}
    ref = oracle.attention(ob, okb, f32(g["v"]), alpha_q=oaq, alpha_k=oak, bias2d=ob2, top_n=w.top_n,
                           av_mode=w.av_mode, rows=rows, want_idx=idx is not None)
    if idx is not None:
        assert np.array_equal(idx.cpu().numpy().reshape(-1, w.top_n)[rows], ref["idx"])
    diff = np.abs(out.cpu().numpy().reshape(-1, w.d)[rows] - ref["out"])
    assert np.all(diff <= q8_tolerance(ref["vscale"], rows, w.n) + 1e-6)
