"""GPU parity of binattn_dense_q8 above 256 tokens (the long-sequence dense kernel: keys
streamed through LDS in tiles, two passes, int8 matrix cores).

Bar: int8 V and its scales bit-exact; every output element within one int8 LSB of V
(the channel's scale) of the oracle's dense softmax + uint8 A x int8 V.  Rows of
every case are compared in full up to n = 1024; above, a seeded sample of rows from
every head plus the last rows (the ragged final tile of queries and keys).
"""
import numpy as np
import pytest
import torch

import oracle
from binarized_qk_sparse_amd import ops, synth
from parity_util import f32, q8_tolerance

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    ops._lib.load()


def _case(B, H, n, d, mode, bias, seed):
    g = np.random.default_rng([51, B, H, n, d, mode, int(bias), seed])
    xq = (g.standard_normal((B, H, n, d)) + 0.5 * g.standard_normal((1, H, 1, d))).astype(np.float32)
    xk = (g.standard_normal((B, H, n, d)) - 0.5 * g.standard_normal((1, H, 1, d))).astype(np.float32)
    v = (g.standard_normal((B, H, n, d)) * g.uniform(0.3, 2.0, (1, H, 1, d))).astype(np.float32)
    v[0, 0, :, 3] = 0.0  # an all-zero channel: scale 0, codes 0
    T = (0.02 * g.standard_normal((H, 2 * n - 1))).astype(np.float32) if bias else None
    qb, aq, _ = oracle.pack(xq, mode)
    kb, ak, _ = oracle.pack(xk, mode)
    if mode == synth.SIGN:
        aq = ak = None
    return qb, kb, aq, ak, T, torch.from_numpy(v).to(torch.bfloat16)


def _rows(B, H, n, per_head, seed):
    if n <= 1024:
        return np.arange(B * H * n, dtype=np.int64)
    g = np.random.default_rng([52, n, seed])
    rows = []
    for bh in range(B * H):
        pick = set(g.choice(n, size=per_head, replace=False).tolist()) | {n - 1, n - 2, n - 65, 0}
        rows.extend(bh * n + np.array(sorted(pick)))
    return np.array(rows, np.int64)


def _run(qb, kb, aq, ak, T, v, bias2d=None):
    dt = lambda a: None if a is None else torch.from_numpy(a).to(DEV)
    B, H, n, d = v.shape
    ws = ops.workspace(B, H, n, d)
    b2 = None if bias2d is None else {k: (dt(x) if isinstance(x, np.ndarray) else x) for k, x in bias2d.items()}
    out = ops.binattn_dense_q8(dt(qb.view(np.int32)), dt(kb.view(np.int32)), v.to(DEV), alpha_q=dt(aq),
                               alpha_k=dt(ak), bias=dt(T), bias2d=b2, ws=ws)
    torch.cuda.synchronize()
    vq, sc = ops.workspace_view(ws, B, H, n, d)
    return out.cpu().numpy().reshape(-1, d), vq.cpu().numpy(), sc.cpu().numpy()


def _check(out, vq, sc, ref, rows, n, what):
    assert np.array_equal(vq, ref["vq"]), f"{what}: int8 V differs"
    assert np.array_equal(sc, ref["vscale"]), f"{what}: V scales differ"
    got = out[rows]
    tol = q8_tolerance(ref["vscale"], rows, n)
    diff = np.abs(got - ref["out"])
    assert np.all(diff <= tol + 1e-6), f"{what}: {int((diff > tol + 1e-6).sum())} elements beyond one int8 LSB"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n", [257, 577, 1024, 4096, 16384])
def test_dense_q8_long_scaled_codes_and_bias(n, d):
    B, H = (1, 2) if n > 4096 else (2, 2)
    qb, kb, aq, ak, T, v = _case(B, H, n, d, synth.MEAN_SIGN, True, seed=1)
    out, vq, sc = _run(qb, kb, aq, ak, T, v)
    rows = _rows(B, H, n, 96, 1)
    ref = oracle.attention(qb, kb, f32(v), alpha_q=aq, alpha_k=ak, bias=T, top_n=None, av_mode=oracle.AV_Q8,
                           rows=rows)
    _check(out, vq, sc, ref, rows, n, f"dense n={n} d={d}")


@pytest.mark.parametrize("n,d", [(300, 64), (1000, 128), (2049, 64)])
@pytest.mark.parametrize("bias", [False, True])
def test_dense_q8_long_plain_sign(n, d, bias):
    # alpha = 1 (the kernel's unscaled instance), with and without the 1-D table
    qb, kb, aq, ak, T, v = _case(2, 3, n, d, synth.SIGN, bias, seed=2)
    out, vq, sc = _run(qb, kb, aq, ak, T, v)
    rows = _rows(2, 3, n, 64, 2)
    ref = oracle.attention(qb, kb, f32(v), bias=T, top_n=None, av_mode=oracle.AV_Q8, rows=rows)
    _check(out, vq, sc, ref, rows, n, f"dense sign n={n} d={d} bias={bias}")


def test_dense_q8_long_heavy_ties():
    # a handful of distinct codes: long rows of equal logits, where A_q of the
    # tied keys must all round alike
    g = np.random.default_rng(53)
    B, H, n = 1, 2, 1500
    base = g.standard_normal((3, 64)).astype(np.float32)
    qb, _, _ = oracle.pack(base[g.integers(0, 3, (B, H, n))], synth.SIGN)
    kb, _, _ = oracle.pack(base[g.integers(0, 3, (B, H, n))], synth.SIGN)
    v = torch.from_numpy(g.standard_normal((B, H, n, 64)).astype(np.float32)).to(torch.bfloat16)
    out, vq, sc = _run(qb, kb, None, None, None, v)
    rows = np.arange(B * H * n, dtype=np.int64)
    ref = oracle.attention(qb, kb, f32(v), top_n=None, av_mode=oracle.AV_Q8, rows=rows)
    _check(out, vq, sc, ref, rows, n, "dense ties")


@pytest.mark.parametrize("grid,cls", [((24, 24), True), ((20, 30), False)])
def test_dense_q8_long_bias2d(grid, cls):
    # the two-dimensional decomposable bias above 256 tokens: DeiT at 384^2 (24 x 24 patches
    # plus the class token, 577 tokens) and a 20 x 30 grid without one
    gh, gw = grid
    n = gh * gw + (1 if cls else 0)
    B, H, d = 1, 3, 64
    qb, kb, aq, ak, _, v = _case(B, H, n, d, synth.MEAN_SIGN, False, seed=3)
    g = np.random.default_rng([54, gh, gw])
    b2 = {"grid": (gh, gw), "row": (0.02 * g.standard_normal((H, 2 * gh - 1))).astype(np.float32),
          "col": (0.02 * g.standard_normal((H, 2 * gw - 1))).astype(np.float32)}
    if cls:
        b2["cls"] = (0.02 * g.standard_normal((H, 3))).astype(np.float32)
    out, vq, sc = _run(qb, kb, aq, ak, None, v, bias2d=b2)
    rows = np.arange(B * H * n, dtype=np.int64)
    ref = oracle.attention(qb, kb, f32(v), alpha_q=aq, alpha_k=ak, bias2d=b2, top_n=None, av_mode=oracle.AV_Q8,
                           rows=rows)
    _check(out, vq, sc, ref, rows, n, f"dense 2-D bias {gh}x{gw}")


def test_dense_q8_long_maximum_length():
    # n = 65536 (the largest the library takes): one head, a few rows including the last
    B, H, n, d = 1, 1, 65536, 64
    qb, kb, aq, ak, T, v = _case(B, H, n, d, synth.MEAN_SIGN, True, seed=4)
    out, vq, sc = _run(qb, kb, aq, ak, T, v)
    rows = np.array([0, 1, 777, 32768, n - 65, n - 2, n - 1], np.int64)
    ref = oracle.attention(qb, kb, f32(v), alpha_q=aq, alpha_k=ak, bias=T, top_n=None, av_mode=oracle.AV_Q8,
                           rows=rows)
    _check(out, vq, sc, ref, rows, n, "dense n=65536")


def test_dense_q8_long_one_past_the_short_limit():
    # n = 256 is the register-resident kernel's limit; n = 257 is the streaming kernel's
    # smallest case: five key tiles, the last holding one key
    qb, kb, aq, ak, T, v = _case(1, 2, 257, 64, synth.MEAN_SIGN, True, seed=5)
    out, vq, sc = _run(qb, kb, aq, ak, T, v)
    rows = np.arange(2 * 257, dtype=np.int64)
    ref = oracle.attention(qb, kb, f32(v), alpha_q=aq, alpha_k=ak, bias=T, top_n=None, av_mode=oracle.AV_Q8)
    ref["out"] = ref["out"].reshape(-1, 64)
    _check(out, vq, sc, ref, rows, 257, "dense n=257")
