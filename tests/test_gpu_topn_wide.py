"""GPU parity of had_attention_topn for long sequences with large kept sets: the
streaming kernel with its larger candidate buffers (kept sets of 705 to 1472 keys)
and the threshold-first kernel beyond (up to every key, and two-dimensional tables
the streaming buffers leave no room for).

Bar: kept index sets bit-exact (ties to the lower key index); fp32 outputs within
1e-3 relative + 1e-4 absolute; the quantized paths within one int8 LSB of V per
element, with the integer V and its scales bit-exact.  Rows: a seeded sample from
every head plus the first and last rows.
"""
import numpy as np
import pytest
import torch

import oracle
from binarized_qk_sparse_amd import ops, synth
from parity_util import assert_close, f32, q8_tolerance, ws_vq

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    ops._lib.load()


def _case(B, H, n, d, mode, bias, vdtype, seed):
    g = np.random.default_rng([61, B, H, n, d, mode, int(bias), seed])
    xq = (g.standard_normal((B, H, n, d)) + 0.3 * g.standard_normal((1, H, 1, d))).astype(np.float32)
    xk = (g.standard_normal((B, H, n, d)) + 0.3 * g.standard_normal((1, H, 1, d))).astype(np.float32)
    v = torch.from_numpy(g.standard_normal((B, H, n, d)).astype(np.float32)).to(vdtype)
    T = (0.05 * g.standard_normal((H, 2 * n - 1))).astype(np.float32) if bias else None
    qb, aq, _ = oracle.pack(xq, mode)
    kb, ak, _ = oracle.pack(xk, mode)
    if mode == synth.SIGN:
        aq = ak = None
    return qb, kb, aq, ak, T, v


def _rows(BH, n, per_head, seed):
    g = np.random.default_rng([62, n, seed])
    rows = []
    for bh in range(BH):
        pick = set(g.choice(n, size=min(per_head, n), replace=False).tolist()) | {0, n - 1}
        rows.extend(bh * n + np.array(sorted(pick)))
    return np.array(rows, np.int64)


def _run_and_check(qb, kb, aq, ak, T, v, N, av, rows, what, bias2d=None):
    dt = lambda a: None if a is None else torch.from_numpy(a).to(DEV)
    B, H, n, d = v.shape
    ws = ops.workspace(B, H, n, d)
    b2 = None if bias2d is None else {k: (dt(x) if isinstance(x, np.ndarray) else x) for k, x in bias2d.items()}
    out, idx = ops.had_attention_topn(dt(qb.view(np.int32)), dt(kb.view(np.int32)), v.to(DEV), N, alpha_q=dt(aq),
                                      alpha_k=dt(ak), bias=dt(T), bias2d=b2, av_mode=av, want_idx=True, ws=ws)
    torch.cuda.synchronize()
    keep = min(N, n)
    ref = oracle.attention(qb, kb, f32(v), alpha_q=aq, alpha_k=ak, bias=T, bias2d=bias2d, top_n=N, av_mode=av,
                           rows=rows, want_idx=True)
    got_idx = idx.cpu().numpy().reshape(-1, keep)[rows]
    assert np.array_equal(got_idx, ref["idx"]), f"{what}: kept index sets differ"
    got = out.cpu().numpy().reshape(-1, d)[rows]
    if av == synth.AV_F32:
        assert_close(got, ref["out"], what)
    else:
        vq, sc = ws_vq(ws, B, H, n, d, av)
        assert np.array_equal(vq.cpu().numpy(), ref["vq"]), f"{what}: integer V differs"
        assert np.array_equal(sc.cpu().numpy(), ref["vscale"]), f"{what}: V scales differ"
        tol = q8_tolerance(ref["vscale"], rows, n)
        diff = np.abs(got - ref["out"])
        assert np.all(diff <= tol + 1e-6), f"{what}: {int((diff > tol + 1e-6).sum())} elements beyond one LSB"
    return idx


@pytest.mark.parametrize("av", [synth.AV_F32, synth.AV_Q8, synth.AV_Q4])
@pytest.mark.parametrize("keys", ["int", "alpha_bias"])
@pytest.mark.parametrize("N", [2048, 5000])
def test_wide_every_key_kept(N, keys, av):
    # n = 2048 with N >= n: the dense softmax over every key (no selection pass)
    n = 2048
    mode = synth.MEAN_SIGN if keys == "alpha_bias" else synth.SIGN
    qb, kb, aq, ak, T, v = _case(1, 2, n, 64, mode, keys != "int", torch.bfloat16, seed=1)
    idx = _run_and_check(qb, kb, aq, ak, T, v, N, av, _rows(2, n, 60, 1), f"N={N} n={n} {keys}")
    assert np.all(idx.cpu().numpy() == np.arange(n))


@pytest.mark.parametrize("av", [synth.AV_F32, synth.AV_Q8, synth.AV_Q4])
@pytest.mark.parametrize("keys", ["int", "bias", "alpha_bias"])
def test_wide_hads_linear_schedule_at_8192(keys, av):
    # N = 15 n / 128 = 960 at n = 8192 (the linear schedule carried to long contexts)
    n, N = 8192, 960
    mode = synth.MEAN_SIGN if keys == "alpha_bias" else synth.SIGN
    qb, kb, aq, ak, T, v = _case(1, 2, n, 64, mode, keys != "int", torch.bfloat16, seed=2)
    _run_and_check(qb, kb, aq, ak, T, v, N, av, _rows(2, n, 80, 2), f"N={N} n={n} {keys}")


@pytest.mark.parametrize("n,N", [(1025, 705), (2000, 705), (3000, 1999), (4100, 4099), (6000, 3000)])
def test_wide_past_the_streaming_buffer(n, N):
    # kept sets just past the streaming kernel's buffer, and up to one short of every key
    qb, kb, aq, ak, T, v = _case(1, 2, n, 64, synth.MEAN_SIGN, True, torch.bfloat16, seed=3)
    _run_and_check(qb, kb, aq, ak, T, v, N, synth.AV_F32, _rows(2, n, 60, 3), f"N={N} n={n}")


@pytest.mark.parametrize("n,N", [(3000, 1472), (3000, 1473), (9000, 1472), (9000, 1473)])
@pytest.mark.parametrize("av", [synth.AV_F32, synth.AV_Q4])
def test_wide_at_the_larger_buffer(n, N, av):
    # the largest kept set the streaming kernel's larger buffers take, and one more (the
    # threshold-first kernel), below and above the sixteen-wave length
    qb, kb, aq, ak, T, v = _case(1, 2, n, 64, synth.MEAN_SIGN, True, torch.bfloat16, seed=8)
    _run_and_check(qb, kb, aq, ak, T, v, N, av, _rows(2, n, 40, 8), f"N={N} n={n} av={av}")


def test_wide_bias2d_tables_past_the_streaming_limit():
    # a 60 x 60 grid with a class token (3601 keys): its staged tables (598 floats) exceed
    # what the streaming kernel keeps beside eight-wave chunks, so the threshold-first
    # kernel takes the row even with a kept set the streaming buffers would hold
    gh = gw = 60
    n, N, H = gh * gw + 1, 500, 2
    qb, kb, aq, ak, _, v = _case(1, H, n, 64, synth.MEAN_SIGN, False, torch.bfloat16, seed=9)
    g = np.random.default_rng(66)
    b2 = {"grid": (gh, gw), "row": (0.02 * g.standard_normal((H, 2 * gh - 1))).astype(np.float32),
          "col": (0.02 * g.standard_normal((H, 2 * gw - 1))).astype(np.float32),
          "cls": (0.02 * g.standard_normal((H, 3))).astype(np.float32)}
    _run_and_check(qb, kb, aq, ak, None, v, N, synth.AV_F32, _rows(H, n, 60, 9), "2-D bias 60x60", bias2d=b2)


@pytest.mark.parametrize("vdtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("keys", ["int", "alpha_bias"])
def test_wide_head_dim_128(keys, vdtype):
    n, N = 1500, 1000
    mode = synth.MEAN_SIGN if keys == "alpha_bias" else synth.SIGN
    qb, kb, aq, ak, T, v = _case(1, 2, n, 128, mode, keys != "int", vdtype, seed=4)
    _run_and_check(qb, kb, aq, ak, T, v, N, synth.AV_F32, _rows(2, n, 60, 4), f"d=128 N={N} {keys}")


@pytest.mark.parametrize("av", [synth.AV_Q8, synth.AV_Q4])
def test_wide_head_dim_128_q8(av):
    n, N = 1500, 1200
    qb, kb, aq, ak, T, v = _case(1, 2, n, 128, synth.MEAN_SIGN, True, torch.bfloat16, seed=5)
    _run_and_check(qb, kb, aq, ak, T, v, N, av, _rows(2, n, 60, 5), f"d=128 av={av}")


@pytest.mark.parametrize("N", [705, 1500, 2999])
def test_wide_all_keys_tied(N):
    # every key equal to every query: one logit value, so the kept set is the N lowest indices
    n = 3000
    g = np.random.default_rng(63)
    x = np.repeat(g.standard_normal((1, 1, 1, 64)).astype(np.float32), n, axis=2)
    qb, _, _ = oracle.pack(x, oracle.SIGN)
    v = torch.from_numpy(g.standard_normal((1, 1, n, 64)).astype(np.float32)).to(torch.bfloat16)
    idx = _run_and_check(qb, qb, None, None, None, v, N, synth.AV_F32, _rows(1, n, 50, 6), f"all ties N={N}")
    assert np.all(idx.cpu().numpy().reshape(-1, N) == np.arange(N))


@pytest.mark.parametrize("bias", [False, True])
def test_wide_heavy_ties(bias):
    # four distinct codes: long runs of equal logits, the threshold level split by index
    n, N = 2500, 1100
    g = np.random.default_rng(64)
    base = g.standard_normal((4, 64)).astype(np.float32)
    qb, _, _ = oracle.pack(base[g.integers(0, 4, (1, 2, n))], oracle.SIGN)
    kb, _, _ = oracle.pack(base[g.integers(0, 4, (1, 2, n))], oracle.SIGN)
    T = np.zeros((2, 2 * n - 1), np.float32) if bias else None  # float logits with exact ties
    v = torch.from_numpy(g.standard_normal((1, 2, n, 64)).astype(np.float32)).to(torch.bfloat16)
    _run_and_check(qb, kb, None, None, T, v, N, synth.AV_F32, np.arange(2 * n, dtype=np.int64), f"ties bias={bias}")


def test_wide_bias2d():
    # the two-dimensional bias with a class token on a 40 x 40 grid, 1000 of 1601 keys kept
    gh = gw = 40
    n, N, H = gh * gw + 1, 1000, 2
    qb, kb, aq, ak, _, v = _case(1, H, n, 64, synth.MEAN_SIGN, False, torch.bfloat16, seed=7)
    g = np.random.default_rng(65)
    b2 = {"grid": (gh, gw), "row": (0.02 * g.standard_normal((H, 2 * gh - 1))).astype(np.float32),
          "col": (0.02 * g.standard_normal((H, 2 * gw - 1))).astype(np.float32),
          "cls": (0.02 * g.standard_normal((H, 3))).astype(np.float32)}
    for av in (synth.AV_F32, synth.AV_Q8):
        _run_and_check(qb, kb, aq, ak, None, v, N, av, _rows(H, n, 60, 7), f"2-D bias av={av}", bias2d=b2)


@pytest.mark.parametrize("N,av", [(256, synth.AV_Q8), (256, synth.AV_F32), (1000, synth.AV_Q4), (3000, synth.AV_F32)])
def test_topn_maximum_length(N, av):
    # n = 65536, the largest the library takes: the streaming kernel (768- and 1536-entry
    # buffers) and the threshold-first kernel, one head, the first, middle and last rows
    n = 65536
    qb, kb, aq, ak, T, v = _case(1, 1, n, 64, synth.MEAN_SIGN, True, torch.bfloat16, seed=10)
    rows = np.array([0, 1, 4097, 32768, n - 65, n - 2, n - 1], np.int64)
    _run_and_check(qb, kb, aq, ak, T, v, N, av, rows, f"n=65536 N={N} av={av}")
