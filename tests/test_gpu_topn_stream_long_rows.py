"""GPU parity of the long-sequence top-N kernel on rows that stress its streaming threshold
(from 4096 keys on, where each row starts from a threshold taken from the logits of its
first chunk of keys and streams again from minus infinity if fewer than N keys pass it):
first chunks that tie at the top or sit at the bottom of the row, keys at one even
spread of positions that tie at the top or sit at the bottom, rows tied throughout, and
ordinary rows at several n and N.  The candidate buffer then fills with ties, or the
threshold rises late, and every compaction path of the stream runs.

Bar: kept index sets bit-exact (ties to the lower key index); fp32 outputs within 1e-3
relative + 1e-4 absolute of the oracle.  Rows: a seeded sample from every head plus the
first and last rows.
"""
import numpy as np
import pytest
import torch

import oracle
from binarized_qk_sparse_amd import ops, synth
from parity_util import assert_close, f32

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    ops._lib.load()


def _spread_positions(n):
    return (np.arange(1024, dtype=np.int64) * n) // 1024


def _rows(BH, n, per_head, seed):
    g = np.random.default_rng([93, n, seed])
    rows = []
    for bh in range(BH):
        pick = set(g.choice(n, size=min(per_head, n), replace=False).tolist()) | {0, n - 1}
        rows.extend(bh * n + np.array(sorted(pick)))
    return np.array(rows, np.int64)


def _check(qb, kb, aq, ak, T, v, N, rows, what):
    dt = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    out, idx = ops.had_attention_topn(dt(qb.view(np.int32)), dt(kb.view(np.int32)), v.to(DEV), N, alpha_q=dt(aq),
                                      alpha_k=dt(ak), bias=dt(T), want_idx=True)
    torch.cuda.synchronize()
    d = v.shape[-1]
    ref = oracle.attention(qb, kb, f32(v), alpha_q=aq, alpha_k=ak, bias=T, top_n=N, rows=rows, want_idx=True)
    keep = min(N, v.shape[2])
    got_idx = idx.cpu().numpy().reshape(-1, keep)[rows]
    assert np.array_equal(got_idx, ref["idx"]), f"{what}: kept index sets differ"
    assert_close(out.cpu().numpy().reshape(-1, d)[rows], ref["out"], what)
    return got_idx


def _inputs(H, n, d, mode, bias, seed):
    g = np.random.default_rng([94, H, n, d, mode, int(bias), seed])
    xq = (g.standard_normal((1, H, n, d)) + 0.3 * g.standard_normal((1, H, 1, d))).astype(np.float32)
    xk = (g.standard_normal((1, H, n, d)) + 0.3 * g.standard_normal((1, H, 1, d))).astype(np.float32)
    v = torch.from_numpy(g.standard_normal((1, H, n, d)).astype(np.float32)).to(torch.bfloat16)
    T = (0.05 * g.standard_normal((H, 2 * n - 1))).astype(np.float32) if bias else None
    return xq, xk, v, T, g


@pytest.mark.parametrize("n,N", [(4096, 1), (4096, 256), (5000, 40), (8192, 700), (12345, 128), (20000, 300)])
@pytest.mark.parametrize("keys", ["int", "alpha_bias"])
def test_ordinary_rows(n, N, keys):
    mode = synth.MEAN_SIGN if keys == "alpha_bias" else synth.SIGN
    xq, xk, v, T, _ = _inputs(2, n, 64, mode, keys != "int", 1)
    qb, aq, _ = oracle.pack(xq, mode)
    kb, ak, _ = oracle.pack(xk, mode)
    if mode == synth.SIGN:
        aq = ak = None
    _check(qb, kb, aq, ak, T, v, N, _rows(2, n, 40, 1), f"n={n} N={N} {keys}")


@pytest.mark.parametrize("N", [1, 256, 700])
def test_spread_keys_tie_at_the_top(N):
    # the keys at the spread positions equal every query (distance 0, the largest logit)
    # and no other key does: the kept set is the N lowest of them
    n = 8192
    g = np.random.default_rng(95)
    x = g.standard_normal((1, 1, n, 64)).astype(np.float32)
    base = g.standard_normal(64).astype(np.float32)
    xq = np.repeat(base[None, None, None, :], n, axis=2)
    pos = _spread_positions(n)
    x[0, 0, pos] = base
    qb, _, _ = oracle.pack(xq, synth.SIGN)
    kb, _, _ = oracle.pack(x, synth.SIGN)
    v = torch.from_numpy(g.standard_normal((1, 1, n, 64)).astype(np.float32)).to(torch.bfloat16)
    idx = _check(qb, kb, None, None, None, v, N, _rows(1, n, 60, 2), f"spread keys at the top N={N}")
    assert np.all(idx == pos[:N])


@pytest.mark.parametrize("N", [64, 600])
def test_spread_keys_at_the_bottom(N):
    # the keys at the spread positions are the farthest from query 0 (distance 64)
    n = 6000
    g = np.random.default_rng(96)
    xq = g.standard_normal((1, 1, n, 64)).astype(np.float32)
    xk = g.standard_normal((1, 1, n, 64)).astype(np.float32)
    pos = _spread_positions(n)
    xk[0, 0, pos] = -xq[0, 0, :1]  # opposite to query 0, unrelated to the others
    qb, _, _ = oracle.pack(xq, synth.SIGN)
    kb, _, _ = oracle.pack(xk, synth.SIGN)
    v = torch.from_numpy(g.standard_normal((1, 1, n, 64)).astype(np.float32)).to(torch.bfloat16)
    _check(qb, kb, None, None, None, v, N, _rows(1, n, 60, 3), f"spread keys at the bottom N={N}")


@pytest.mark.parametrize("bias", [False, True])
def test_row_tied_throughout(bias):
    # one logit for every key (a zero table keeps them equal): the kept set is the N
    # lowest indices
    n, N = 5000, 200
    g = np.random.default_rng(97)
    x = np.repeat(g.standard_normal((1, 1, 1, 64)).astype(np.float32), n, axis=2)
    qb, _, _ = oracle.pack(x, synth.SIGN)
    T = np.zeros((1, 2 * n - 1), np.float32) if bias else None
    v = torch.from_numpy(g.standard_normal((1, 1, n, 64)).astype(np.float32)).to(torch.bfloat16)
    idx = _check(qb, qb, None, None, T, v, N, _rows(1, n, 60, 4), f"tied bias={bias}")
    assert np.all(idx == np.arange(N))


def test_head_dim_128():
    n, N = 4500, 256
    xq, xk, v, T, _ = _inputs(2, n, 128, synth.MEAN_SIGN, True, 5)
    qb, aq, _ = oracle.pack(xq, synth.MEAN_SIGN)
    kb, ak, _ = oracle.pack(xk, synth.MEAN_SIGN)
    _check(qb, kb, aq, ak, T, v, N, _rows(2, n, 40, 5), "d=128")


@pytest.mark.parametrize("N", [1, 300, 700])
def test_first_chunk_ties_at_the_top(N):
    # the first 2048 keys equal every query (the largest logit): the starting threshold
    # is that logit, no key passes it, and the row streams again; the kept set is the N
    # lowest indices
    n = 9000
    g = np.random.default_rng(98)
    base = g.standard_normal(64).astype(np.float32)
    xq = np.repeat(base[None, None, None, :], n, axis=2)
    xk = g.standard_normal((1, 1, n, 64)).astype(np.float32)
    xk[0, 0, :2048] = base
    qb, _, _ = oracle.pack(xq, synth.SIGN)
    kb, _, _ = oracle.pack(xk, synth.SIGN)
    v = torch.from_numpy(g.standard_normal((1, 1, n, 64)).astype(np.float32)).to(torch.bfloat16)
    idx = _check(qb, kb, None, None, None, v, N, _rows(1, n, 60, 6), f"first chunk at the top N={N}")
    assert np.all(idx == np.arange(N))


@pytest.mark.parametrize("N", [64, 600])
def test_first_chunk_at_the_bottom(N):
    # the first 2048 keys oppose every query (the smallest logit): the starting threshold
    # is far below the row's kept logits and the stream compacts as it goes
    n = 7000
    g = np.random.default_rng(99)
    base = g.standard_normal(64).astype(np.float32)
    xq = np.repeat(base[None, None, None, :], n, axis=2)
    xk = g.standard_normal((1, 1, n, 64)).astype(np.float32)
    xk[0, 0, :2048] = -base
    qb, _, _ = oracle.pack(xq, synth.SIGN)
    kb, _, _ = oracle.pack(xk, synth.SIGN)
    T = (0.05 * g.standard_normal((1, 2 * n - 1))).astype(np.float32)
    v = torch.from_numpy(g.standard_normal((1, 1, n, 64)).astype(np.float32)).to(torch.bfloat16)
    _check(qb, kb, None, None, T, v, N, _rows(1, n, 60, 7), f"first chunk at the bottom N={N}")
