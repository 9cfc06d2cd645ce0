"""GPU parity of the long-sequence top-N kernel on inputs far from the usual ones: scales
of either sign and zero, one key scale a million times the rest, a relative-position
table much wider than a logit step, and rows that reach a finite threshold only at their
first compaction (below 4096 keys no row starts from a sampled threshold).  Every
admission, compaction and selection path must keep the kept sets exact.

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


def _rows(BH, n, per_head, seed):
    g = np.random.default_rng([101, n, seed])
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


def _codes(H, n, d, seed):
    g = np.random.default_rng([102, H, n, d, seed])
    xq = g.standard_normal((1, H, n, d)).astype(np.float32)
    xk = g.standard_normal((1, H, n, d)).astype(np.float32)
    qb, aq, _ = oracle.pack(xq, synth.MEAN_SIGN)
    kb, ak, _ = oracle.pack(xk, synth.MEAN_SIGN)
    v = torch.from_numpy(g.standard_normal((1, H, n, d)).astype(np.float32)).to(torch.bfloat16)
    return qb, kb, aq, ak, v, g


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [50, 400])
def test_scales_of_either_sign(N, d):
    # alpha of both signs and exact zeros (a zero key scale leaves the logit equal to the
    # bias): the order of the logits no longer follows the Hamming levels
    n = 6000
    qb, kb, _, _, v, g = _codes(2, n, d, 1)
    aq = g.standard_normal((1, 2, n)).astype(np.float32)
    ak = g.standard_normal((1, 2, n)).astype(np.float32)
    ak[:, :, ::97] = 0.0
    aq[:, :, ::89] = 0.0
    T = (0.05 * g.standard_normal((2, 2 * n - 1))).astype(np.float32)
    _check(qb, kb, aq, ak, T, v, N, _rows(2, n, 40, 1), f"signed scales N={N} d={d}")


@pytest.mark.parametrize("N", [1, 200])
def test_one_key_scale_far_above_the_rest(N):
    # two keys whose scales are a million times the others': the one with the positive
    # scale is kept by every query whose code is closer to it than to its opposite, the
    # other by every query on the far side
    n = 8192
    qb, kb, aq, ak, v, g = _codes(1, n, 64, 2)
    ak = ak.copy()
    ak[0, 0, 3000] = 1e6
    ak[0, 0, 6000] = -1e6
    T = (0.05 * g.standard_normal((1, 2 * n - 1))).astype(np.float32)
    _check(qb, kb, aq, ak, T, v, N, _rows(1, n, 60, 2), f"one huge key scale N={N}")


@pytest.mark.parametrize("scale", [0.5, 3.0])
def test_wide_relative_position_table(scale):
    # a table whose spread reaches several logit steps: the bias reorders keys across
    # many Hamming levels
    n, N = 5000, 128
    qb, kb, aq, ak, v, g = _codes(2, n, 64, 3)
    T = (scale * g.standard_normal((2, 2 * n - 1))).astype(np.float32)
    _check(qb, kb, aq, ak, T, v, N, _rows(2, n, 40, 3), f"table spread {scale}")


@pytest.mark.parametrize("n,N", [(1500, 16), (3000, 300), (4095, 64)])
@pytest.mark.parametrize("keys", ["int", "alpha_bias"])
def test_filter_after_the_first_compaction(n, N, keys):
    # below 4096 keys no row starts from a sampled threshold: theta stays -inf until the
    # candidate buffer first fills
    qb, kb, aq, ak, v, g = _codes(2, n, 64, 4)
    T = None
    if keys == "alpha_bias":
        T = (0.05 * g.standard_normal((2, 2 * n - 1))).astype(np.float32)
    else:
        aq = ak = None
    _check(qb, kb, aq, ak, T, v, N, _rows(2, n, 40, 4), f"n={n} N={N} {keys}")
