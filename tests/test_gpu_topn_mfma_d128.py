"""GPU parity of the matrix-core top-N kernel at head_dim 128 (plain sign codes, no table,
bf16 V, fp32 A*V, up to 1024 tokens).

Its distance bytes cap the Hamming level at 127; a tile where a row's threshold reaches
level 127 recounts levels 127 and 128 from the codes and weighs every key on its own.
The cases below reach that path on purpose (keys opposite to a query, so that its
distances sit at 127 and 128, with and without padding keys), the capped bytes with a
threshold below the cap, every size class of the kernel (32, 64, ... 1024 padded keys,
full and ragged), kept counts from 1 to every key, and the full c3d128 workload.

Bar: kept index sets bit-exact (ties to the lower key index); fp32 outputs within 1e-3
relative + 1e-4 absolute of the oracle on every row, and the weights' 16 significant
bits pinned as at head_dim 64.
"""
import numpy as np
import pytest
import torch

import oracle
from binarized_qk_sparse_amd import ops, synth
from parity_util import assert_close, f32, packed_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda"
D = 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    ops._lib.load()


def _run(qb, kb, v, N, want_idx=True):
    dt = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).to(DEV)
    res = ops.had_attention_topn(dt(qb), dt(kb), v.to(DEV), N, want_idx=want_idx)
    torch.cuda.synchronize()
    if want_idx:
        return res[0].cpu().numpy(), res[1].cpu().numpy()
    return res.cpu().numpy(), None


def _check(xq, xk, v, N, what, want_idx=True):
    qb, _, _ = oracle.pack(xq, oracle.SIGN)
    kb, _, _ = oracle.pack(xk, oracle.SIGN)
    out, idx = _run(qb, kb, v, N, want_idx)
    ref = oracle.attention(qb, kb, f32(v), top_n=N, want_idx=True)
    n = xq.shape[2]
    if want_idx:
        assert np.array_equal(idx.reshape(ref["idx"].shape), ref["idx"]), f"{what}: kept index sets differ"
    assert_close(out.reshape(-1, D), ref["out"].reshape(-1, D), what)
    return idx


def _inputs(B, H, n, seed):
    g = np.random.default_rng([121, B, H, n, seed])
    xq = g.standard_normal((B, H, n, D)).astype(np.float32)
    xk = g.standard_normal((B, H, n, D)).astype(np.float32)
    v = torch.from_numpy(g.standard_normal((B, H, n, D)).astype(np.float32)).to(torch.bfloat16)
    return xq, xk, v, g


@pytest.mark.parametrize("n", [1, 5, 32, 33, 64, 65, 100, 128, 129, 255, 256, 257, 511, 512, 513, 700, 1023, 1024])
@pytest.mark.parametrize("N", [1, 30, 120, 5000])
def test_sizes_and_kept_counts(n, N):
    xq, xk, v, _ = _inputs(1, 2, n, 1)
    _check(xq, xk, v, N, f"n={n} N={N}")


@pytest.mark.parametrize("n", [200, 1024])
def test_without_index_output(n):
    # the instance the benchmark times writes no index list
    xq, xk, v, _ = _inputs(2, 2, n, 2)
    _check(xq, xk, v, 120, f"n={n} no idx", want_idx=False)


def _opposite_keys(n, n127, seed):
    # every key is the negation of query 0 (level 128 for it), the first n127 with one
    # channel flipped back (level 127); the other queries are random
    xq, _, v, g = _inputs(1, 1, n, seed)
    xk = np.repeat(-xq[:, :, :1], n, axis=2).copy()
    xk[0, 0, :n127, 5] = -xk[0, 0, :n127, 5]
    return xq, xk, v


@pytest.mark.parametrize("n", [1024, 700, 97])
@pytest.mark.parametrize("split", ["below", "inside", "all"])
def test_threshold_at_the_capped_levels(n, split):
    # query 0 sees n127 keys at level 127 and the rest at 128: with N at most n127 its
    # threshold is 127 (ties among the 127s), above it 128 (every 127 kept, ties among
    # the 128s); the other queries of its tile take the same exact path with their own
    # thresholds, all keys of a row tied at one level
    n127 = n // 3
    N = {"below": max(1, n127 // 2), "inside": n127 + (n - n127) // 2, "all": n}[split]
    xq, xk, v = _opposite_keys(n, n127, 3)
    idx = _check(xq, xk, v, N, f"capped levels n={n} N={N}")
    keep = min(N, n)
    got0 = idx.reshape(-1, keep)[0]
    expect = np.arange(min(N, n127)) if N <= n127 else np.concatenate([np.arange(n127), np.arange(n127, N)])
    assert np.array_equal(got0, expect)


@pytest.mark.parametrize("n", [1024, 333])
def test_capped_bytes_below_the_threshold(n):
    # most keys of query 0 sit at levels 127 and 128 but N of them are close to it:
    # the threshold stays below the cap and the capped keys must all be dropped
    xq, xk, v = _opposite_keys(n, n // 2, 4)
    near = np.arange(0, n, 37)
    xk[0, 0, near] = xq[0, 0, 0] * np.where(np.arange(D) < 100, 1.0, -1.0)  # level 28 from query 0
    _check(xq, xk, v, len(near), f"capped bytes n={n}")


def test_heavy_ties_at_one_level():
    # every key equal: one level per row, the kept set is the N lowest indices
    n, N = 1000, 77
    xq, xk, v, _ = _inputs(1, 2, n, 5)
    xk[:] = xk[:, :, :1]
    idx = _check(xq, xk, v, N, "all keys equal")
    assert np.array_equal(idx.reshape(-1, N), np.tile(np.arange(N, dtype=np.int32), (2 * n, 1)))


@pytest.mark.parametrize("n,N", [(64, 15), (1024, 120), (1000, 120)])
def test_weights_carry_sixteen_bits(n, N):
    """As at head_dim 64: weights split into bf16 high and low parts keep 16 significant
    bits, so |O - O_exact| <= 4e-5 sum_S p|V| + 1e-6, which high parts alone would miss."""
    g = np.random.default_rng([122, n, N])
    xq = g.standard_normal((2, 4, n, D)).astype(np.float32)
    xk = g.standard_normal((2, 4, n, D)).astype(np.float32)
    v = torch.from_numpy((3.0 * g.standard_normal((2, 4, n, D))).astype(np.float32)).to(torch.bfloat16)
    qb, _, _ = oracle.pack(xq, oracle.SIGN)
    kb, _, _ = oracle.pack(xk, oracle.SIGN)
    out, _ = _run(qb, kb, v, N)
    ref = oracle.attention(qb, kb, f32(v), top_n=N)["out"]
    mag = oracle.attention(qb, kb, np.abs(f32(v)), top_n=N)["out"]
    err = np.abs(out.astype(np.float64) - ref)
    bound = 4e-5 * mag + 1e-6
    assert np.all(err <= bound), f"worst {np.max(err / bound):.2f} of the bound"


@pytest.mark.parametrize("want_idx", [True, False])
def test_c3d128_every_row(want_idx):
    w = synth.workload("c3d128")
    p = packed_inputs(w)
    res = ops.had_attention_topn(p["dq"], p["dk"], p["dv"], w.top_n, want_idx=want_idx)
    out = res[0] if want_idx else res
    torch.cuda.synchronize()
    ref = oracle.attention(p["oq"], p["ok"], f32(p["v"]), top_n=w.top_n, want_idx=True)
    if want_idx:
        assert np.array_equal(res[1].cpu().numpy(), ref["idx"])
    assert_close(out.cpu().numpy(), ref["out"], w.name)
