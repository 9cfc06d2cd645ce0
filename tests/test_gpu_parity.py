"""GPU parity: every entry point of libhad.so against the CPU oracle on the same seeded inputs.

Bar: code bits, alpha, mu, Hamming-derived top-N index sets and int8 V are
bit-exact; fp32 outputs within 1e-3 relative + 1e-4 absolute; the quantized
path within one int8 LSB of V (the channel's scale) per output element.
"""
import numpy as np
import pytest
import torch

import oracle
from binarized_qk_sparse_amd import ops, synth
from parity_util import assert_close, f32, packed_inputs, q8_tolerance, rows_per_head, sample_rows, u32, ws_vq

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    ops._lib.load()


# ------------------------------------------------------------------ packing
@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_pack_full_size_configs(name):
    w = synth.workload(name)
    g = synth.generate(w)
    for t in ("q", "k"):
        x = g[t]
        bits, alpha, mu = ops.had_pack(x.to(DEV), w.mode)
        torch.cuda.synchronize()
        ob, oa, om = oracle.pack(f32(x), w.mode)
        assert np.array_equal(u32(bits), ob), f"{name} {t}: code bits differ"
        assert np.array_equal(alpha.cpu().numpy(), oa), f"{name} {t}: alpha differs"
        assert np.array_equal(mu.cpu().numpy(), om), f"{name} {t}: mu differs"


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("n", [1, 3, 255, 257, 700])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("mode", [synth.SIGN, synth.MEAN_SIGN])
def test_pack_ragged_and_special_values(d, n, dtype, mode):
    g = np.random.default_rng([3, d, n])
    x = (g.standard_normal((2, 3, n, d)) + g.standard_normal((1, 3, 1, d))).astype(np.float32)
    x[0, 0, 0, : d // 2] = 0.0
    x[0, 1, 0, : d // 2] = -0.0
    x[1, 2, :, 1] = 1.5  # a constant channel: x - mu is exactly 0 there
    xt = torch.from_numpy(x).to(dtype)
    bits, alpha, mu = ops.had_pack(xt.to(DEV), mode)
    torch.cuda.synchronize()
    ob, oa, om = oracle.pack(f32(xt), mode)
    assert np.array_equal(u32(bits), ob)
    assert np.array_equal(alpha.cpu().numpy(), oa)
    assert np.array_equal(mu.cpu().numpy(), om)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_pack_sign_nonfinite(dtype):
    # plain sign is the test x < 0: -inf gives the -1 code, +inf and NaN (either sign) +1
    x = np.random.default_rng(12).standard_normal((1, 2, 37, 64)).astype(np.float32)
    x[0, 0, 0, :6] = [-np.inf, np.inf, np.nan, -np.nan, -0.0, 0.0]
    x[0, 1, 36, -4:] = [-np.inf, -np.nan, np.inf, -1e-30]
    xt = torch.from_numpy(x).to(dtype)
    bits, alpha, mu = ops.had_pack(xt.to(DEV), synth.SIGN)
    torch.cuda.synchronize()
    ob, oa, om = oracle.pack(f32(xt), synth.SIGN)
    assert np.array_equal(u32(bits), ob)
    assert np.array_equal(alpha.cpu().numpy(), oa) and np.array_equal(mu.cpu().numpy(), om)


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("n", [1, 100, 197, 700])
@pytest.mark.parametrize("mode", [synth.SIGN, synth.MEAN_SIGN])
def test_pack_qk_matches_oracle_and_pack(d, n, mode):
    """had_pack_qk: both tensors exactly as the oracle (and had_pack) gives them, across the
    one-launch-per-pass path (n >= rows per workgroup, few chunks) and the separate-mu path."""
    g = np.random.default_rng([5, d, n, mode])
    xq = (g.standard_normal((2, 3, n, d)) + g.standard_normal((1, 3, 1, d))).astype(np.float32)
    xk = (0.5 * g.standard_normal((2, 3, n, d)) - g.standard_normal((1, 3, 1, d))).astype(np.float32)
    xq[1, 2, :, 3] = 0.25  # a constant channel: x - mu is exactly 0 there
    q, k = torch.from_numpy(xq).to(torch.bfloat16), torch.from_numpy(xk).to(torch.bfloat16)
    (qb, aq, mq), (kb, ak, mk) = ops.had_pack_qk(q.to(DEV), k.to(DEV), mode)
    pq = ops.had_pack(q.to(DEV), mode)
    torch.cuda.synchronize()
    for got, x, one in (((qb, aq, mq), q, pq), ((kb, ak, mk), k, None)):
        ob, oa, om = oracle.pack(f32(x), mode)
        assert np.array_equal(u32(got[0]), ob), "code bits differ"
        assert np.array_equal(got[1].cpu().numpy(), oa), "alpha differs"
        assert np.array_equal(got[2].cpu().numpy(), om), "mu differs"
        if one is not None:
            assert np.array_equal(u32(one[0]), u32(got[0]))


# ------------------------------------------------------------------ top-N, fp32 A*V
def _topn_case(B, H, n, N, vdtype, mode, bias, seed, av=synth.AV_F32, d=64):
    g = np.random.default_rng([11, B, H, n, N, seed] + ([d] if d != 64 else []))
    xq = (g.standard_normal((B, H, n, d)) + 0.3 * g.standard_normal((1, H, 1, d))).astype(np.float32)
    xk = (g.standard_normal((B, H, n, d)) + 0.3 * g.standard_normal((1, H, 1, d))).astype(np.float32)
    v = torch.from_numpy(g.standard_normal((B, H, n, d)).astype(np.float32)).to(vdtype)
    T = (0.05 * g.standard_normal((H, 2 * n - 1))).astype(np.float32) if bias else None
    qb, aq, _ = oracle.pack(xq, mode)
    kb, ak, _ = oracle.pack(xk, mode)
    if mode == synth.SIGN:
        aq = ak = None
    return qb, kb, aq, ak, T, v


def _run_topn(qb, kb, aq, ak, T, v, N, av=synth.AV_F32):
    dt = lambda a: None if a is None else torch.from_numpy(a).to(DEV)
    out, idx = ops.had_attention_topn(dt(qb.view(np.int32)), dt(kb.view(np.int32)), v.to(DEV), N,
                                      alpha_q=dt(aq), alpha_k=dt(ak), bias=dt(T), av_mode=av, want_idx=True)
    torch.cuda.synchronize()
    return out.cpu().numpy(), idx.cpu().numpy()


@pytest.mark.parametrize("n", [1, 5, 63, 64, 65, 197, 256, 300, 513, 1024])
@pytest.mark.parametrize("N", [1, 7, 30, 120, 5000])
@pytest.mark.parametrize("keys", ["int", "bias", "alpha_bias"])
def test_topn_fp32_matches_oracle(n, N, keys):
    vdtype = torch.float32 if (n <= 512 and N == 7) else torch.bfloat16
    mode = synth.MEAN_SIGN if keys == "alpha_bias" else synth.SIGN
    qb, kb, aq, ak, T, v = _topn_case(1, 2, n, N, vdtype, mode, keys != "int", seed=1)
    out, idx = _run_topn(qb, kb, aq, ak, T, v, N)
    ref = oracle.attention(qb, kb, f32(v), alpha_q=aq, alpha_k=ak, bias=T, top_n=N, want_idx=True)
    assert np.array_equal(idx, ref["idx"]), "kept index sets differ"
    assert_close(out, ref["out"], f"n={n} N={N} {keys}")


@pytest.mark.parametrize("vdtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("n", [300, 1024])
def test_topn_heavy_ties(vdtype, n):
    # only a handful of distinct codes: most logits tie and the lower index must win
    g = np.random.default_rng(5)
    B, H = 2, 3
    base = g.standard_normal((4, 64)).astype(np.float32)
    xq = base[g.integers(0, 4, (B, H, n))]
    xk = base[g.integers(0, 4, (B, H, n))]
    v = torch.from_numpy(g.standard_normal((B, H, n, 64)).astype(np.float32)).to(vdtype)
    qb, _, _ = oracle.pack(xq, oracle.SIGN)
    kb, _, _ = oracle.pack(xk, oracle.SIGN)
    T = np.zeros((H, 2 * n - 1), np.float32)  # float-key path with exact ties
    for bias in (None, T):
        for N in (1, 10, 77, min(n - 1, 600)):
            out, idx = _run_topn(qb, kb, None, None, bias, v, N)
            ref = oracle.attention(qb, kb, f32(v), bias=bias, top_n=N, want_idx=True)
            assert np.array_equal(idx, ref["idx"])
            assert_close(out, ref["out"], f"ties N={N}")


@pytest.mark.parametrize("name", ["c1", "c2"])
def test_topn_configs_full(name):
    w = synth.workload(name)
    p = packed_inputs(w)
    out, idx = ops.had_attention_topn(p["dq"], p["dk"], p["dv"], w.top_n, alpha_q=p["daq"], alpha_k=p["dak"],
                                      bias=p["dbias"], want_idx=True)
    torch.cuda.synchronize()
    ref = oracle.attention(p["oq"], p["ok"], f32(p["v"]), alpha_q=p["oaq"], alpha_k=p["oak"], bias=p["obias"],
                           top_n=w.top_n, want_idx=True)
    assert np.array_equal(idx.cpu().numpy(), ref["idx"])
    assert_close(out.cpu().numpy(), ref["out"], name)


@pytest.mark.parametrize("want_idx", [True, False])
@pytest.mark.parametrize("n", synth.C3_SWEEP)
def test_topn_c3_sweep_every_row(n, want_idx):
    # want_idx=False runs the kernel variant the benchmark times (no index output); every
    # query row of the full workload is compared
    w = synth.c3(n)
    p = packed_inputs(w)
    res = ops.had_attention_topn(p["dq"], p["dk"], p["dv"], w.top_n, want_idx=want_idx)
    out = res[0] if want_idx else res
    torch.cuda.synchronize()
    ref = oracle.attention(p["oq"], p["ok"], f32(p["v"]), top_n=w.top_n, want_idx=True)
    if want_idx:
        assert np.array_equal(res[1].cpu().numpy(), ref["idx"])
    assert_close(out.cpu().numpy(), ref["out"], w.name)


@pytest.mark.parametrize("n,N", [(64, 15), (197, 30), (1024, 120), (1000, 120)])
def test_topn_mfma_weights_carry_sixteen_bits(n, N):
    """The matrix-core kernel (integer logits, bf16 V) splits each softmax weight into bf16
    high and low parts, so a weight keeps 16 significant bits (relative error below 2^-16)
    and Z is summed from the same weights.  Then |O - O_exact| <= 2^-16 (sum_S p|V| + |O|)
    plus fp32 accumulation noise; the test allows 4e-5 sum_S p|V| + 1e-6.  High parts
    alone (2^-9 relative) would miss it by more than an order of magnitude.  n = 197 and
    1000 run the instance with padding keys, 64 and 1024 the one without."""
    g = np.random.default_rng([13, n, N])
    B, H = 2, 4
    xq = g.standard_normal((B, H, n, 64)).astype(np.float32)
    xk = g.standard_normal((B, H, n, 64)).astype(np.float32)
    v = torch.from_numpy((3.0 * g.standard_normal((B, H, n, 64))).astype(np.float32)).to(torch.bfloat16)
    qb, _, _ = oracle.pack(xq, oracle.SIGN)
    kb, _, _ = oracle.pack(xk, oracle.SIGN)
    out, _ = _run_topn(qb, kb, None, None, None, v, N)
    ref = oracle.attention(qb, kb, f32(v), top_n=N)["out"]
    mag = oracle.attention(qb, kb, np.abs(f32(v)), top_n=N)["out"]  # sum over S of p_j |V_j|
    err = np.abs(out.astype(np.float64) - ref)
    bound = 4e-5 * mag + 1e-6
    assert np.all(err <= bound), f"worst {np.max(err / bound):.2f} of the bound"


def test_topn_deterministic():
    w = synth.c3(512)
    p = packed_inputs(w)
    a = ops.had_attention_topn(p["dq"], p["dk"], p["dv"], w.top_n)
    b = ops.had_attention_topn(p["dq"], p["dk"], p["dv"], w.top_n)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# ------------------------------------------------------------------ quantized paths
def _check_q8(out, ws_vq, ws_sc, ref, rows, n, what):
    assert np.array_equal(ws_vq, ref["vq"]), f"{what}: int8 V differs"
    assert np.array_equal(ws_sc, ref["vscale"]), f"{what}: V scales differ"
    tol = q8_tolerance(ref["vscale"], rows, n)
    diff = np.abs(out - ref["out"])
    assert np.all(diff <= tol + 1e-6), f"{what}: {int((diff > tol).sum())} elements beyond one int8 LSB"


@pytest.mark.parametrize("n,N", [(5, 3), (197, 30), (256, 256), (700, 64), (1024, 120)])
@pytest.mark.parametrize("av", [synth.AV_Q8, synth.AV_Q4])
def test_topn_q8_matches_oracle(n, N, av):
    qb, kb, aq, ak, T, v = _topn_case(2, 2, n, N, torch.bfloat16, synth.MEAN_SIGN, True, seed=2)
    dt = lambda a: torch.from_numpy(a).to(DEV)
    ws = ops.workspace(2, 2, n, 64)
    out, idx = ops.had_attention_topn(dt(qb.view(np.int32)), dt(kb.view(np.int32)), v.to(DEV), N, alpha_q=dt(aq),
                                      alpha_k=dt(ak), bias=dt(T), av_mode=av, want_idx=True, ws=ws)
    torch.cuda.synchronize()
    vq, sc = ws_vq(ws, 2, 2, n, 64, av)
    ref = oracle.attention(qb, kb, f32(v), alpha_q=aq, alpha_k=ak, bias=T, top_n=N, av_mode=av, want_idx=True)
    if av == synth.AV_Q4:
        assert np.abs(vq.cpu().numpy()).max() == 7
    assert np.array_equal(idx.cpu().numpy(), ref["idx"])
    rows = np.arange(2 * 2 * n)
    _check_q8(out.cpu().numpy().reshape(-1, 64), vq.cpu().numpy(), sc.cpu().numpy(),
              {**ref, "out": ref["out"].reshape(-1, 64)}, rows, n, f"q8 n={n}")


@pytest.mark.parametrize("n", [1, 16, 33, 197, 256])
def test_dense_q8_small(n):
    qb, kb, aq, ak, T, v = _topn_case(2, 3, n, n, torch.bfloat16, synth.MEAN_SIGN, True, seed=3)
    dt = lambda a: torch.from_numpy(a).to(DEV)
    ws = ops.workspace(2, 3, n, 64)
    out = ops.binattn_dense_q8(dt(qb.view(np.int32)), dt(kb.view(np.int32)), v.to(DEV), alpha_q=dt(aq),
                               alpha_k=dt(ak), bias=dt(T), ws=ws)
    torch.cuda.synchronize()
    vq, sc = ops.workspace_view(ws, 2, 3, n, 64)
    ref = oracle.attention(qb, kb, f32(v), alpha_q=aq, alpha_k=ak, bias=T, top_n=None, av_mode=oracle.AV_Q8)
    _check_q8(out.cpu().numpy().reshape(-1, 64), vq.cpu().numpy(), sc.cpu().numpy(),
              {**ref, "out": ref["out"].reshape(-1, 64)}, np.arange(2 * 3 * n), n, f"dense n={n}")


def test_dense_q8_c4_every_row():
    w = synth.workload("c4")
    p = packed_inputs(w)
    ws = ops.workspace(w.B, w.H, w.n, w.d)
    out = ops.binattn_dense_q8(p["dq"], p["dk"], p["dv"], alpha_q=p["daq"], alpha_k=p["dak"], bias=p["dbias"],
                               ws=ws)
    torch.cuda.synchronize()
    vq, sc = ops.workspace_view(ws, w.B, w.H, w.n, w.d)
    rows = np.arange(w.B * w.H * w.n, dtype=np.int64)
    ref = oracle.attention(p["oq"], p["ok"], f32(p["v"]), alpha_q=p["oaq"], alpha_k=p["oak"], bias=p["obias"],
                           top_n=None, av_mode=oracle.AV_Q8, rows=rows)
    _check_q8(out.cpu().numpy().reshape(-1, 64), vq.cpu().numpy(), sc.cpu().numpy(), ref, rows, w.n, "c4")


def test_graph_replays_match_eager():
    # the benchmark replays a captured HIP graph: every replay must equal the eager result
    w = synth.c3(256)
    p = packed_inputs(w)
    eager = ops.had_attention_topn(p["dq"], p["dk"], p["dv"], w.top_n)
    out = torch.empty_like(eager)
    g = torch.cuda.CUDAGraph()
    ops.had_attention_topn(p["dq"], p["dk"], p["dv"], w.top_n, out=out)  # warm-up outside capture
    with torch.cuda.graph(g):
        ops.had_attention_topn(p["dq"], p["dk"], p["dv"], w.top_n, out=out)
    for _ in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)


# ------------------------------------------------------------------ long sequences (streaming kernel)
@pytest.mark.parametrize("n,N", [(1025, 1), (1500, 30), (2048, 256), (3000, 700), (4100, 120)])
@pytest.mark.parametrize("keys", ["int", "alpha_bias"])
@pytest.mark.parametrize("av", [synth.AV_F32, synth.AV_Q8, synth.AV_Q4])
def test_topn_long_sequence_matches_oracle(n, N, keys, av):
    mode = synth.MEAN_SIGN if keys == "alpha_bias" else synth.SIGN
    qb, kb, aq, ak, T, v = _topn_case(1, 2, n, N, torch.bfloat16, mode, keys != "int", seed=4)
    dt = lambda a: None if a is None else torch.from_numpy(a).to(DEV)
    ws = ops.workspace(1, 2, n, 64)
    out, idx = ops.had_attention_topn(dt(qb.view(np.int32)), dt(kb.view(np.int32)), v.to(DEV), N, alpha_q=dt(aq),
                                      alpha_k=dt(ak), bias=dt(T), av_mode=av, want_idx=True, ws=ws)
    torch.cuda.synchronize()
    rows = sample_rows(2 * n, 700, n)
    ref = oracle.attention(qb, kb, f32(v), alpha_q=aq, alpha_k=ak, bias=T, top_n=N, av_mode=av, rows=rows,
                           want_idx=True)
    keep = min(N, n)
    assert np.array_equal(idx.cpu().numpy().reshape(-1, keep)[rows], ref["idx"])
    got = out.cpu().numpy().reshape(-1, 64)[rows]
    if av == synth.AV_F32:
        assert_close(got, ref["out"], f"long n={n} N={N}")
    else:
        vq, sc = ws_vq(ws, 1, 2, n, 64, av)
        _check_q8(got, vq.cpu().numpy(), sc.cpu().numpy(), ref, rows, n, f"long q8 n={n}")


@pytest.mark.parametrize("N", [100, 600])
def test_topn_long_sequence_all_ties(N):
    # every key equal to the query: one logit value for all 3000 keys, so no
    # threshold can split the candidate buffer and each compaction falls back to
    # the exact selection, which keeps the lowest key indices
    n = 3000
    g = np.random.default_rng(8)
    x = np.repeat(g.standard_normal((1, 1, 1, 64)).astype(np.float32), n, axis=2)
    qb, _, _ = oracle.pack(x, oracle.SIGN)
    v = torch.from_numpy(g.standard_normal((1, 1, n, 64)).astype(np.float32)).to(torch.bfloat16)
    rows = sample_rows(n, 200, 9)
    out, idx = _run_topn(qb, qb, None, None, None, v, N)
    ref = oracle.attention(qb, qb, f32(v), top_n=N, rows=rows, want_idx=True)
    assert np.array_equal(idx.reshape(-1, N)[rows], ref["idx"])
    assert np.all(idx.reshape(-1, N) == np.arange(N))
    assert_close(out.reshape(-1, 64)[rows], ref["out"], f"all ties N={N}")


@pytest.mark.parametrize("name", ["c5", "c5q4"])
def test_topn_c5_full_size_sampled(name):
    w = synth.workload(name)
    g = synth.generate(w)
    ws = ops.workspace(w.B, w.H, w.n, w.d)
    q, k, v = g["q"].to(DEV), g["k"].to(DEV), g["v"].to(DEV)
    qb, aq, _ = ops.had_pack(q, w.mode, ws=ws)
    kb, ak, _ = ops.had_pack(k, w.mode, ws=ws)
    bias = g["bias"].to(DEV)
    out, idx = ops.had_attention_topn(qb, kb, v, w.top_n, alpha_q=aq, alpha_k=ak, bias=bias, av_mode=w.av_mode,
                                      want_idx=True, ws=ws)
    torch.cuda.synchronize()
    # the oracle packs the same inputs itself (end-to-end check of the whole path)
    oq, oaq, _ = oracle.pack(f32(g["q"]), w.mode)
    okb, oak, _ = oracle.pack(f32(g["k"]), w.mode)
    assert np.array_equal(qb.cpu().numpy().view(np.uint32), oq)
    assert np.array_equal(kb.cpu().numpy().view(np.uint32), okb)
    assert np.array_equal(aq.cpu().numpy(), oaq)
    assert np.array_equal(ak.cpu().numpy(), oak)
    rows = rows_per_head(w.B * w.H, w.n, 256, 5)  # 4096 rows, 256 from every head
    ref = oracle.attention(oq, okb, f32(g["v"]), alpha_q=oaq, alpha_k=oak, bias=g["bias"].numpy(), top_n=w.top_n,
                           av_mode=w.av_mode, rows=rows, want_idx=True)
    assert np.array_equal(idx.cpu().numpy().reshape(-1, w.top_n)[rows], ref["idx"])
    vq, sc = ws_vq(ws, w.B, w.H, w.n, w.d, w.av_mode)
    _check_q8(out.cpu().numpy().reshape(-1, 64)[rows], vq.cpu().numpy(), sc.cpu().numpy(), ref, rows, w.n, name)


def test_topn_zero_distance_ties():
    # identical codes give Hamming distance 0 for many keys: the threshold level is
    # the lowest one and the tie budget runs out part-way through the keys
    g = np.random.default_rng(6)
    B, H, n = 1, 2, 256
    x = g.standard_normal((B, H, n, 64)).astype(np.float32)
    x[:, :, ::3] = x[:, :, :1]  # every third key equals key 0
    qb, _, _ = oracle.pack(x, oracle.SIGN)
    v = torch.from_numpy(g.standard_normal((B, H, n, 64)).astype(np.float32)).to(torch.bfloat16)
    for N in (1, 5, 40, 85, 86, 200):
        out, idx = _run_topn(qb, qb, None, None, None, v, N)
        ref = oracle.attention(qb, qb, f32(v), top_n=N, want_idx=True)
        assert np.array_equal(idx, ref["idx"]), N
        assert_close(out, ref["out"], f"zero-distance ties N={N}")


# ------------------------------------------------------------------ head_dim 128
# The same entry points at d = 128 (codes of four words): the matrix-core kernel for
# plain sign codes with bf16 V and no table up to n = 1024, else the resident kernel up
# to n = 512 (256 with fp32 V) and the long-sequence kernel beyond; and the dense q8 kernel.
@pytest.mark.parametrize("n,N,vdtype", [(1, 1, torch.float32), (65, 7, torch.float32), (197, 30, torch.bfloat16),
                                        (256, 120, torch.float32), (300, 30, torch.float32),
                                        (512, 120, torch.bfloat16), (700, 64, torch.bfloat16),
                                        (1500, 256, torch.bfloat16)])
@pytest.mark.parametrize("keys", ["int", "bias", "alpha_bias"])
def test_topn_d128_matches_oracle(n, N, vdtype, keys):
    mode = synth.MEAN_SIGN if keys == "alpha_bias" else synth.SIGN
    qb, kb, aq, ak, T, v = _topn_case(1, 2, n, N, vdtype, mode, keys != "int", seed=5, d=128)
    out, idx = _run_topn(qb, kb, aq, ak, T, v, N)
    rows = sample_rows(2 * n, 600, n)
    ref = oracle.attention(qb, kb, f32(v), alpha_q=aq, alpha_k=ak, bias=T, top_n=N, rows=rows, want_idx=True)
    keep = min(N, n)
    assert np.array_equal(idx.reshape(-1, keep)[rows], ref["idx"]), "kept index sets differ"
    assert_close(out.reshape(-1, 128)[rows], ref["out"], f"d=128 n={n} N={N} {keys}")


@pytest.mark.parametrize("n,N", [(197, 30), (512, 64), (1300, 120)])
@pytest.mark.parametrize("av", [synth.AV_Q8, synth.AV_Q4])
def test_topn_q8_d128_matches_oracle(n, N, av):
    qb, kb, aq, ak, T, v = _topn_case(1, 2, n, N, torch.bfloat16, synth.MEAN_SIGN, True, seed=6, d=128)
    dt = lambda a: torch.from_numpy(a).to(DEV)
    ws = ops.workspace(1, 2, n, 128)
    out, idx = ops.had_attention_topn(dt(qb.view(np.int32)), dt(kb.view(np.int32)), v.to(DEV), N, alpha_q=dt(aq),
                                      alpha_k=dt(ak), bias=dt(T), av_mode=av, want_idx=True, ws=ws)
    torch.cuda.synchronize()
    vq, sc = ws_vq(ws, 1, 2, n, 128, av)
    rows = sample_rows(2 * n, 600, n)
    ref = oracle.attention(qb, kb, f32(v), alpha_q=aq, alpha_k=ak, bias=T, top_n=N, av_mode=av,
                           rows=rows, want_idx=True)
    keep = min(N, n)
    assert np.array_equal(idx.cpu().numpy().reshape(-1, keep)[rows], ref["idx"])
    _check_q8(out.cpu().numpy().reshape(-1, 128)[rows], vq.cpu().numpy(), sc.cpu().numpy(), ref, rows, n,
              f"av={av} d=128 n={n}")


@pytest.mark.parametrize("n", [1, 33, 197, 256])
def test_dense_q8_d128(n):
    qb, kb, aq, ak, T, v = _topn_case(2, 2, n, n, torch.bfloat16, synth.MEAN_SIGN, True, seed=7, d=128)
    dt = lambda a: torch.from_numpy(a).to(DEV)
    ws = ops.workspace(2, 2, n, 128)
    out = ops.binattn_dense_q8(dt(qb.view(np.int32)), dt(kb.view(np.int32)), v.to(DEV), alpha_q=dt(aq),
                               alpha_k=dt(ak), bias=dt(T), ws=ws)
    torch.cuda.synchronize()
    vq, sc = ops.workspace_view(ws, 2, 2, n, 128)
    ref = oracle.attention(qb, kb, f32(v), alpha_q=aq, alpha_k=ak, bias=T, top_n=None, av_mode=oracle.AV_Q8)
    _check_q8(out.cpu().numpy().reshape(-1, 128), vq.cpu().numpy(), sc.cpu().numpy(),
              {**ref, "out": ref["out"].reshape(-1, 128)}, np.arange(2 * 2 * n), n, f"dense d=128 n={n}")
