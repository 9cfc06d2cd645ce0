"""GPU parity of top-N attention with plain sign codes and a relative-position table on the
matrix-core path (head_dim 64, bf16 V, up to 256 tokens).  Heads whose table spans less than
one logit step keep the level order (float selection among the keys at the threshold level
only); the others select among every key of a row.

Bar: kept index sets bit-exact (ties to the lower key index); fp32 outputs within 1e-3
relative + 1e-4 absolute of the oracle and within the 16-bit weight bound
4e-5 sum_S p|V| + 1e-6 (weights split into bf16 high and low parts).
"""
import numpy as np
import pytest
import torch

import oracle
from binarized_qk_sparse_amd import ops, synth
from parity_util import assert_close, f32, packed_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    ops._lib.load()


def _run(qb, kb, T, v, N, want_idx=True):
    dt = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    res = ops.had_attention_topn(dt(qb.view(np.int32)), dt(kb.view(np.int32)), v.to(DEV), N, bias=dt(T),
                                 want_idx=want_idx)
    torch.cuda.synchronize()
    if want_idx:
        return res[0].cpu().numpy(), res[1].cpu().numpy()
    return res.cpu().numpy(), None


def _check(qb, kb, T, v, N, what, want_idx=True, weight_pin=True):
    out, idx = _run(qb, kb, T, v, N, want_idx)
    ref = oracle.attention(qb, kb, f32(v), bias=T, top_n=N, want_idx=True)
    if want_idx:
        assert np.array_equal(idx, ref["idx"]), f"{what}: kept index sets differ"
    assert_close(out, ref["out"], what)
    if weight_pin:
        mag = oracle.attention(qb, kb, np.abs(f32(v)), bias=T, top_n=N)["out"]
        err = np.abs(out.astype(np.float64) - ref["out"])
        bound = 4e-5 * mag + 1e-6
        assert np.all(err <= bound), f"{what}: worst {np.max(err / bound):.2f} of the 16-bit weight bound"


def _codes(B, H, n, seed):
    g = np.random.default_rng([71, B, H, n, seed])
    qb, _, _ = oracle.pack(g.standard_normal((B, H, n, 64)).astype(np.float32), oracle.SIGN)
    kb, _, _ = oracle.pack(g.standard_normal((B, H, n, 64)).astype(np.float32), oracle.SIGN)
    v = torch.from_numpy((2.0 * g.standard_normal((B, H, n, 64))).astype(np.float32)).to(torch.bfloat16)
    return qb, kb, v, g


@pytest.mark.parametrize("want_idx", [True, False])
def test_c2_every_row(want_idx):
    # the BERT-base workload: every query row, with and without the index output
    w = synth.workload("c2")
    p = packed_inputs(w)
    res = ops.had_attention_topn(p["dq"], p["dk"], p["dv"], w.top_n, bias=p["dbias"], want_idx=want_idx)
    torch.cuda.synchronize()
    out = res[0] if want_idx else res
    ref = oracle.attention(p["oq"], p["ok"], f32(p["v"]), bias=p["obias"], top_n=w.top_n, want_idx=True)
    if want_idx:
        assert np.array_equal(res[1].cpu().numpy(), ref["idx"])
    assert_close(out.cpu().numpy(), ref["out"], "c2")


@pytest.mark.parametrize("n", [1, 5, 64, 65, 100, 197, 256])
@pytest.mark.parametrize("N", [1, 7, 30, 120, 5000])
def test_sizes_and_kept_counts(n, N):
    qb, kb, v, g = _codes(2, 3, n, 1)
    T = (0.03 * g.standard_normal((3, 2 * n - 1))).astype(np.float32)
    _check(qb, kb, T, v, N, f"n={n} N={N}")


def test_mixed_heads_level_order_and_full_selection():
    # heads 0 and 2 keep their tables within a step (level order), heads 1 and 3 do not
    # (every key a candidate); every row of all four is compared
    n, H = 256, 4
    qb, kb, v, g = _codes(2, H, n, 2)
    T = (0.02 * g.standard_normal((H, 2 * n - 1))).astype(np.float32)
    T[1] *= 25.0
    T[3] = np.linspace(-0.2, 0.2, 2 * n - 1, dtype=np.float32)  # spans 0.4: no level order
    for N in (1, 30, 200):
        _check(qb, kb, T, v, N, f"mixed N={N}")


@pytest.mark.parametrize("span", [0.2399, 0.2401])
def test_table_at_the_level_test_edge(span):
    # a table spanning just below (level order) and just above (full selection) the
    # test's 0.24: both must give the oracle's index sets
    n, H = 256, 2
    qb, kb, v, g = _codes(1, H, n, 3)
    T = (0.5 * span * (2.0 * g.random((H, 2 * n - 1)) - 1.0)).astype(np.float32)
    T[:, 0], T[:, 1] = -0.5 * span, 0.5 * span
    _check(qb, kb, T, v, 30, f"span {span}")


@pytest.mark.parametrize("table", ["zero", "small", "wide"])
@pytest.mark.parametrize("N", [1, 10, 77, 255])
def test_heavy_ties_at_the_threshold_level(table, N):
    # few distinct codes: many keys share the threshold level (more than a lane caches);
    # a zero table makes their logits equal (the lower index wins), a small one splits them,
    # a wide one mixes the levels
    n, B, H = 256, 2, 3
    g = np.random.default_rng(72)
    base = g.standard_normal((4, 64)).astype(np.float32)
    qb, _, _ = oracle.pack(base[g.integers(0, 4, (B, H, n))], oracle.SIGN)
    kb, _, _ = oracle.pack(base[g.integers(0, 4, (B, H, n))], oracle.SIGN)
    v = torch.from_numpy(g.standard_normal((B, H, n, 64)).astype(np.float32)).to(torch.bfloat16)
    scale = {"zero": 0.0, "small": 0.01, "wide": 1.0}[table]  # "wide": every key a candidate
    T = (scale * g.standard_normal((H, 2 * n - 1))).astype(np.float32)
    _check(qb, kb, T, v, N, f"ties {table} N={N}")


def test_all_keys_at_one_level_with_a_table():
    # every key equal to every query: all keys at distance 0, ordered by the table alone
    n, N = 256, 40
    g = np.random.default_rng(73)
    x = np.repeat(g.standard_normal((1, 2, 1, 64)).astype(np.float32), n, axis=2)
    qb, _, _ = oracle.pack(x, oracle.SIGN)
    v = torch.from_numpy(g.standard_normal((1, 2, n, 64)).astype(np.float32)).to(torch.bfloat16)
    T = (0.05 * g.standard_normal((2, 2 * n - 1))).astype(np.float32)
    T[0, 100:140] = T[0, 99]  # runs of equal offsets: equal logits split by index
    _check(qb, qb, T, v, N, "one level")


def test_graph_replays_match_eager_with_a_table():
    # the float-key launch replayed from a captured graph
    w = synth.workload("c2")
    p = packed_inputs(w, B=2)
    eager = ops.had_attention_topn(p["dq"], p["dk"], p["dv"], w.top_n, bias=p["dbias"])
    out = torch.empty_like(eager)
    ops.had_attention_topn(p["dq"], p["dk"], p["dv"], w.top_n, bias=p["dbias"], out=out)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ops.had_attention_topn(p["dq"], p["dk"], p["dv"], w.top_n, bias=p["dbias"], out=out)
    for _ in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)


@pytest.mark.parametrize("scale", [1.0, 30.0])
def test_wide_tables(scale):
    # tables spanning many logit steps: every key a candidate, each weight its own
    # exp(l - max l); scale 30 makes the weights span far beyond fp32 exponents
    n, H = 197, 3
    qb, kb, v, g = _codes(2, H, n, 5)
    T = (scale * g.standard_normal((H, 2 * n - 1))).astype(np.float32)
    for N in (1, 30, 196, 5000):
        _check(qb, kb, T, v, N, f"wide x{scale} N={N}")


@pytest.mark.parametrize("layout,N", [("crowded", 6), ("crowded", 17), ("crowded", 18), ("crowded", 23),
                                      ("crowded", 24), ("crowded", 35), ("spread", 18), ("spread", 20),
                                      ("spread", 21), ("spread", 22)])
def test_ranks_at_the_merged_queue_limit(layout, N):
    # Every query is all +1; 5 keys at distance 0, 30 at distance 1, the rest at 5, so the
    # threshold level is 1 and a row keeps N - 5 of the 30 keys at it.  "crowded": 20 of
    # the 30 in the first key quarter (more than a lane's queue of twelve) and 10 in the
    # third; the rank from the nearer end is then 1, 12 (merged queues), 13, 13 (walk), 12
    # (from the low end, merged) and 1.  "spread": at most 8 in each quarter, so no queue
    # drops a candidate, with ranks 13, 15, 16 and 14 (from the low end), past what the
    # merged queues take.  Head 0 has distinct table values, head 1 a table rounded to a few
    # values, so that keys at the threshold tie on the logit and split by index.
    n, H = 256, 2
    g = np.random.default_rng(74)
    q = np.ones((1, H, n, 64), np.float32)
    k = np.ones((1, H, n, 64), np.float32)
    k[..., :5] = -1.0  # distance 5
    level0 = [3, 71, 141, 201, 250]
    if layout == "crowded":
        level1 = list(range(1, 61, 3)) + list(range(130, 190, 6))
    else:
        level1 = [4 + 8 * i for i in range(30)]
    assert len(level1) == 30 and not set(level1) & set(level0)
    k[0, :, level0] = 1.0
    k[0, :, level1] = 1.0
    k[0, :, level1, 0] = -1.0
    qb, _, _ = oracle.pack(q, oracle.SIGN)
    kb, _, _ = oracle.pack(k, oracle.SIGN)
    h = oracle.logits(qb, kb)[0][0, 0, 0]
    assert np.sum(h == 0) == 5 and np.sum(h == 1) == 30 and np.sum(h == 5) == n - 35
    T = (0.01 * g.standard_normal((H, 2 * n - 1))).astype(np.float32)
    T[1] = np.round(T[1] / 0.01).astype(np.float32) * np.float32(0.01)
    v = torch.from_numpy(g.standard_normal((1, H, n, 64)).astype(np.float32)).to(torch.bfloat16)
    _check(qb, kb, T, v, N, f"merge limit {layout} N={N}")
