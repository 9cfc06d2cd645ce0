"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test fixes one step of the method with something independent: a brute
force over unpacked +-1 floats, a closed form, a textbook routine
(torch scaled_dot_product_attention in float64), an invariant, or a value
stated on the pages (Theorem 1 of BinaryAttention, section 2.1).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _signs(x):
    """+-1 codes with sign(0)=+1, as float64 (independent of the bit packing)."""
    return np.where(np.asarray(x) < 0, -1.0, 1.0)


def _unpack(bits, d):
    w = np.asarray(bits, dtype=np.uint64)
    c = np.arange(d)
    b = (w[..., c // 32] >> (c % 32).astype(np.uint64)) & np.uint64(1)
    return np.where(b == 1, -1.0, 1.0)


# ------------------------------------------------------------------ binarize
def test_sign_bits_brute_force_and_layout():
    g = np.random.default_rng(1)
    x = g.standard_normal((2, 3, 37, 64)).astype(np.float32)
    x[0, 0, 0, :8] = 0.0
    x[0, 0, 1, :8] = -0.0
    bits, alpha, mu = oracle.pack(x, oracle.SIGN)
    assert np.array_equal(_unpack(bits, 64), _signs(x))
    assert np.all(alpha == 1.0) and np.all(mu == 0.0)
    # one negative channel c sets bit c%32 of word c//32 and nothing else
    for c in (0, 5, 31, 32, 63):
        y = np.ones((1, 1, 1, 64), np.float32)
        y[..., c] = -1.0
        b, _, _ = oracle.pack(y, oracle.SIGN)
        want = np.zeros(2, np.uint32)
        want[c // 32] = np.uint32(1 << (c % 32))
        assert np.array_equal(b[0, 0, 0], want)


def test_sign_invariant_under_positive_channel_scaling():
    # configs with per-channel std: plain sign must not depend on a positive scale
    g = np.random.default_rng(2)
    x = g.standard_normal((1, 2, 50, 64)).astype(np.float32)
    s = g.uniform(0.5, 2.0, (1, 2, 1, 64)).astype(np.float32)
    assert np.array_equal(oracle.pack(x, oracle.SIGN)[0], oracle.pack(x * s, oracle.SIGN)[0])


def _mean_sign_case(n=64, d=64, seed=3):
    """x[i,c] = m[c] + e[i]*s[i,c] with tokens i and i+n/2 carrying opposite
    signs and equal e, so the token mean is exactly m and |x-m| is exactly e.
    All values are multiples of 1/8 so every sum is exact."""
    g = np.random.default_rng(seed)
    half = n // 2
    s_half = np.where(g.integers(0, 2, (half, d)) == 1, 1.0, -1.0)
    s = np.concatenate([s_half, -s_half])
    e_half = g.integers(1, 16, half) / 8.0
    e = np.concatenate([e_half, e_half])
    m = g.integers(-40, 40, d) / 8.0
    x = (m[None, :] + e[:, None] * s).astype(np.float32)
    return x[None, None], s, e, m


def test_mean_sign_closed_form():
    x, s, e, m = _mean_sign_case()
    bits, alpha, mu = oracle.pack(x, oracle.MEAN_SIGN)
    assert np.array_equal(mu[0, 0], m.astype(np.float32))
    assert np.array_equal(alpha[0, 0], e.astype(np.float32))
    assert np.array_equal(_unpack(bits, 64)[0, 0], s)


def test_mean_sign_exact_zero_is_plus_one():
    # a token equal to the mean in some channel gets code +1 there
    x = np.zeros((1, 1, 4, 32), np.float32)
    x[0, 0, 0, 0], x[0, 0, 1, 0] = 1.0, -1.0  # channel 0: mean 0, tokens 2,3 exactly 0
    bits, alpha, mu = oracle.pack(x, oracle.MEAN_SIGN)
    assert mu[0, 0, 0] == 0.0
    assert [int(b[0]) & 1 for b in bits[0, 0]] == [0, 1, 0, 0]
    assert np.allclose(alpha[0, 0], [1 / 32, 1 / 32, 0, 0])


def test_mean_sign_matches_float64_definition_on_random_data():
    g = np.random.default_rng(4)
    x = (g.standard_normal((2, 2, 97, 64)) + g.standard_normal((1, 2, 1, 64))).astype(np.float32)
    bits, alpha, mu = oracle.pack(x, oracle.MEAN_SIGN)
    mu64 = x.astype(np.float64).mean(axis=2)
    assert np.all(np.abs(mu - mu64) <= np.spacing(np.abs(mu64).astype(np.float32)))
    y = x - mu[:, :, None, :]  # float32 subtraction as defined
    assert np.array_equal(_unpack(bits, 64), _signs(y))
    a64 = np.abs(y.astype(np.float64)).mean(axis=3)
    assert np.all(np.abs(alpha - a64) <= np.spacing(a64.astype(np.float32)))


def test_theorem1_expected_code_product():
    # BinaryAttention 2.1, Theorem 1: for zero-mean jointly Gaussian q,k with
    # correlation rho, E[sign(q) sign(k)] = (2/pi) arcsin(rho).
    g = np.random.default_rng(5)
    for rho in (0.5, -0.3, 0.9):
        z1 = g.standard_normal((1, 64, 128, 64))
        z2 = g.standard_normal((1, 64, 128, 64))
        q = z1.astype(np.float32)
        k = (rho * z1 + math.sqrt(1 - rho * rho) * z2).astype(np.float32)
        qb, _, _ = oracle.pack(q, oracle.SIGN)
        kb, _, _ = oracle.pack(k, oracle.SIGN)
        ham, _ = oracle.logits(qb, kb)
        diag = np.diagonal(ham, axis1=2, axis2=3)  # same token: correlated pair
        est = np.mean(64 - 2 * diag) / 64.0
        assert abs(est - 2.0 / math.pi * math.asin(rho)) < 5e-3
        off = (64 - 2 * ham[..., 0, 1:]) / 64.0  # independent tokens
        assert abs(off.mean()) < 5e-3


# ------------------------------------------------------------------ hamming / logits
@pytest.mark.parametrize("d", [32, 64, 128])
def test_hamming_identity_against_pm1_float_dot(d):
    g = np.random.default_rng(6 + d)
    xq = g.standard_normal((2, 2, 41, d)).astype(np.float32)
    xk = g.standard_normal((2, 2, 41, d)).astype(np.float32)
    qb, _, _ = oracle.pack(xq, oracle.SIGN)
    kb, _, _ = oracle.pack(xk, oracle.SIGN)
    ham, lg = oracle.logits(qb, kb)
    dot = np.einsum("bhic,bhjc->bhij", _signs(xq), _signs(xk))
    assert np.array_equal(dot, d - 2 * ham)
    # no scales, no bias: l = dot * float(1/sqrt(d)) (exact dot/8 for d=64)
    s = np.float32(1.0 / math.sqrt(d))
    assert np.array_equal(lg, (dot.astype(np.float32) * s).astype(np.float32))
    if d == 64:
        assert np.array_equal(lg, dot / 8.0)


def test_logits_with_scales_and_bias_against_float64():
    # BinaryAttention 2.2-2.3: l = alpha_q*alpha_k*dot/sqrt(d) + T[j-i+n-1]
    g = np.random.default_rng(7)
    B, H, n, d = 1, 2, 23, 64
    xq = g.standard_normal((B, H, n, d)).astype(np.float32)
    xk = g.standard_normal((B, H, n, d)).astype(np.float32)
    qb, aq, _ = oracle.pack(xq, oracle.MEAN_SIGN)
    kb, ak, _ = oracle.pack(xk, oracle.MEAN_SIGN)
    T = g.standard_normal((H, 2 * n - 1)).astype(np.float32)  # asymmetric on purpose
    ham, lg = oracle.logits(qb, kb, aq, ak, T)
    dot = (d - 2 * ham).astype(np.float64)
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    bias = T[:, j - i + n - 1]  # [H, n, n]
    prod = aq[..., :, None].astype(np.float64) * ak[..., None, :] * dot / 8.0
    want = prod + bias[None]
    # three float32 roundings on the product side, one on the sum
    mag = np.maximum(np.abs(prod), np.abs(want)).astype(np.float32)
    assert np.all(np.abs(lg - want) <= 4 * np.spacing(mag))
    # a transposed offset (i-j) or a dropped scale is far outside that bound
    wrong = prod + T[:, i - j + n - 1][None]
    assert np.max(np.abs(lg - wrong)) > 1e-3


# ------------------------------------------------------------------ top-N
def _brute_topn(l, N):
    n = len(l)
    order = sorted(range(n), key=lambda j: (-float(l[j]), j))
    return sorted(order[: min(N, n)])


@pytest.mark.parametrize("N,d", [(1, 32), (5, 32), (30, 32), (64, 32), (200, 32), (5, 128), (30, 128)])
def test_topn_matches_brute_force_full_sort(N, d):
    g = np.random.default_rng(8 + N + d)
    # d=32: only 33 logit levels, so ties are everywhere; d=128: four code words per row and an
    # irrational 1/sqrt(d), which keeps distinct integer products distinct and equal ones tied
    B, H, n = 1, 2, 64
    xq = g.standard_normal((B, H, n, d)).astype(np.float32)
    xk = g.standard_normal((B, H, n, d)).astype(np.float32)
    v = g.standard_normal((B, H, n, d)).astype(np.float32)
    qb, _, _ = oracle.pack(xq, oracle.SIGN)
    kb, _, _ = oracle.pack(xk, oracle.SIGN)
    res = oracle.attention(qb, kb, v, top_n=N, want_idx=True)
    dot = np.einsum("bhic,bhjc->bhij", _signs(xq), _signs(xk))
    for h in range(H):
        for i in range(n):
            assert list(res["idx"][0, h, i]) == _brute_topn(dot[0, h, i], N)


def test_topn_ties_go_to_lower_key_index():
    n, d = 40, 64
    x = np.ones((1, 1, n, d), np.float32)  # every key identical -> all logits tie
    bits, _, _ = oracle.pack(x, oracle.SIGN)
    v = np.random.default_rng(9).standard_normal((1, 1, n, d)).astype(np.float32)
    res = oracle.attention(bits, bits, v, top_n=7, want_idx=True)
    assert np.all(res["idx"][0, 0] == np.arange(7))
    assert np.allclose(res["out"][0, 0], v[0, 0, :7].mean(axis=0), atol=1e-6)


# ------------------------------------------------------------------ softmax + A*V
def _sdpa64(xq, xk, v, aq, ak, T, keep_mask=None):
    """Textbook attention in float64 on the scaled codes (torch SDPA)."""
    q = torch.from_numpy(_signs(xq) * (1.0 if aq is None else aq[..., None].astype(np.float64)))
    k = torch.from_numpy(_signs(xk) * (1.0 if ak is None else ak[..., None].astype(np.float64)))
    n = xq.shape[2]
    mask = torch.zeros((xq.shape[1], n, n), dtype=torch.float64)
    if T is not None:
        i = np.arange(n)[:, None]
        j = np.arange(n)[None, :]
        mask = torch.from_numpy(T[:, j - i + n - 1].astype(np.float64))
    mask = mask[None].expand(xq.shape[0], -1, -1, -1).clone()
    if keep_mask is not None:
        mask[~torch.from_numpy(keep_mask)] = float("-inf")
    return torch.nn.functional.scaled_dot_product_attention(
        q, k, torch.from_numpy(v.astype(np.float64)), attn_mask=mask).numpy()


def _case(seed, B=2, H=2, n=48, d=64, mode=oracle.MEAN_SIGN, bias=True):
    g = np.random.default_rng(seed)
    xq = (g.standard_normal((B, H, n, d)) + 0.5 * g.standard_normal((1, H, 1, d))).astype(np.float32)
    xk = (g.standard_normal((B, H, n, d)) + 0.5 * g.standard_normal((1, H, 1, d))).astype(np.float32)
    v = g.standard_normal((B, H, n, d)).astype(np.float32)
    T = (0.3 * g.standard_normal((H, 2 * n - 1))).astype(np.float32) if bias else None
    qb, aq, _ = oracle.pack(xq, mode)
    kb, ak, _ = oracle.pack(xk, mode)
    if mode == oracle.SIGN:
        aq = ak = None
    return xq, xk, v, T, qb, kb, aq, ak


@pytest.mark.parametrize("mode,d", [(oracle.SIGN, 64), (oracle.MEAN_SIGN, 64), (oracle.MEAN_SIGN, 128)])
def test_dense_equals_textbook_attention(mode, d):
    xq, xk, v, T, qb, kb, aq, ak = _case(10, mode=mode, d=d)
    if mode == oracle.MEAN_SIGN:
        # the codes are sign(x - mu); hand SDPA the centred inputs' signs
        _, _, mq = oracle.pack(xq, mode)
        _, _, mk = oracle.pack(xk, mode)
        xq, xk = xq - mq[:, :, None, :], xk - mk[:, :, None, :]
    got = oracle.attention(qb, kb, v, alpha_q=aq, alpha_k=ak, bias=T, top_n=None)["out"]
    want = _sdpa64(xq, xk, v, aq, ak, T)
    assert np.allclose(got, want, rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("d", [64, 128])
def test_topn_equals_masked_textbook_attention(d):
    xq, xk, v, T, qb, kb, aq, ak = _case(11, d=d)
    _, _, mq = oracle.pack(xq, oracle.MEAN_SIGN)
    _, _, mk = oracle.pack(xk, oracle.MEAN_SIGN)
    yq, yk = xq - mq[:, :, None, :], xk - mk[:, :, None, :]
    N = 9
    res = oracle.attention(qb, kb, v, alpha_q=aq, alpha_k=ak, bias=T, top_n=N, want_idx=True)
    # kept set from a brute-force sort of float64 logits built independently
    B, H, n, d = xq.shape
    dot = np.einsum("bhic,bhjc->bhij", _signs(yq), _signs(yk))
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    l = (aq[..., :, None] * ak[..., None, :]).astype(np.float64) * dot / np.sqrt(d) + T[:, j - i + n - 1][None]
    keep = np.zeros((B, H, n, n), bool)
    for b in range(B):
        for h in range(H):
            for q in range(n):
                sel = _brute_topn(l[b, h, q], N)
                assert list(res["idx"][b, h, q]) == sel
                keep[b, h, q, sel] = True
    want = _sdpa64(yq, yk, v, aq, ak, T, keep_mask=keep)
    assert np.allclose(res["out"], want, rtol=1e-5, atol=1e-6)


def test_rows_sum_to_one_and_hard_attention():
    xq, xk, v, T, qb, kb, aq, ak = _case(12)
    ones = np.ones_like(v)
    for N in (1, 7, None):
        out = oracle.attention(qb, kb, ones, alpha_q=aq, alpha_k=ak, bias=T, top_n=N)["out"]
        assert np.all(np.abs(out.astype(np.float64) - 1.0) < 1e-6)
    res = oracle.attention(qb, kb, v, alpha_q=aq, alpha_k=ak, bias=T, top_n=1, want_idx=True)
    B, H, n, d = v.shape
    j = res["idx"][..., 0]
    assert np.array_equal(res["out"], np.take_along_axis(v, j[..., None, None].repeat(d, -1).reshape(B, H, n, d), 2))


def test_single_token():
    x = np.random.default_rng(13).standard_normal((1, 1, 1, 64)).astype(np.float32)
    bits, a, _ = oracle.pack(x, oracle.MEAN_SIGN)
    assert a[0, 0, 0] == 0.0 and np.all(bits == 0)  # x - mu == 0 everywhere
    v = np.random.default_rng(14).standard_normal((1, 1, 1, 64)).astype(np.float32)
    assert np.array_equal(oracle.attention(bits, bits, v, top_n=5)["out"][0, 0], v[0, 0])
    r = oracle.attention(bits, bits, v, top_n=5, av_mode=oracle.AV_Q8, want_aq8=True)
    assert r["aq8"][0, 0, 0, 0] == 255
    assert np.allclose(r["out"][0, 0], v[0, 0], atol=np.abs(v).max() / 127)


# ------------------------------------------------------------------ two-dimensional decomposable bias
def _bias2d_case(seed, H, gh, gw, cls):
    g = np.random.default_rng(seed)
    b2 = {"grid": (gh, gw), "row": (0.3 * g.standard_normal((H, 2 * gh - 1))).astype(np.float32),
          "col": (0.3 * g.standard_normal((H, 2 * gw - 1))).astype(np.float32)}
    if cls:
        b2["cls"] = (0.3 * g.standard_normal((H, 3))).astype(np.float32)
    return b2


def _bias2d_dense(b2, H):
    """The bias matrix [H, n, n] written out token pair by token pair."""
    gh, gw = b2["grid"]
    cls = 1 if "cls" in b2 else 0
    n = cls + gh * gw
    out = np.zeros((H, n, n), np.float32)
    for h in range(H):
        for i in range(n):
            for j in range(n):
                if i < cls and j < cls:
                    out[h, i, j] = b2["cls"][h, 2]
                elif i < cls:
                    out[h, i, j] = b2["cls"][h, 0]
                elif j < cls:
                    out[h, i, j] = b2["cls"][h, 1]
                else:
                    ri, ci = divmod(i - cls, gw)
                    rj, cj = divmod(j - cls, gw)
                    out[h, i, j] = np.float32(b2["row"][h, rj - ri + gh - 1]) + np.float32(b2["col"][h, cj - ci + gw - 1])
    return out


@pytest.mark.parametrize("gh,gw,cls", [(3, 5, 1), (4, 4, 0), (2, 7, 1)])
def test_bias2d_logits_add_the_written_out_bias(gh, gw, cls):
    H = 2
    n = cls + gh * gw
    g = np.random.default_rng(40 + gh)
    x = g.standard_normal((1, H, n, 64)).astype(np.float32)
    y = g.standard_normal((1, H, n, 64)).astype(np.float32)
    qb, aq, _ = oracle.pack(x, oracle.MEAN_SIGN)
    kb, ak, _ = oracle.pack(y, oracle.MEAN_SIGN)
    b2 = _bias2d_case(gh * 10 + gw, H, gh, gw, cls)
    _, plain = oracle.logits(qb, kb, aq, ak)
    _, lg = oracle.logits(qb, kb, aq, ak, bias2d=b2)
    dense = _bias2d_dense(b2, H)
    assert np.array_equal(lg, (plain + dense[None]).astype(np.float32))
    # a transposed offset (r_i - r_j) or the row and column tables swapped give other values
    wrong = dict(b2, row=b2["row"][:, ::-1].copy())
    assert not np.array_equal(_bias2d_dense(wrong, H), dense)


def test_bias2d_single_row_is_the_1d_offset_table():
    # one grid row and no class token: B[i][j] = R[0] + C[j - i + n - 1], the 1-D table R[0] + C
    H, gw = 2, 9
    b2 = _bias2d_case(3, H, 1, gw, 0)
    g = np.random.default_rng(41)
    qb, _, _ = oracle.pack(g.standard_normal((1, H, gw, 64)).astype(np.float32), oracle.SIGN)
    kb, _, _ = oracle.pack(g.standard_normal((1, H, gw, 64)).astype(np.float32), oracle.SIGN)
    T = (b2["row"][:, :1] + b2["col"]).astype(np.float32)
    assert np.array_equal(oracle.logits(qb, kb, bias2d=b2)[1], oracle.logits(qb, kb, bias=T)[1])


def test_topn_bias2d_equals_masked_textbook_attention():
    H, gh, gw, cls = 2, 4, 6, 1
    n = cls + gh * gw
    xq, xk, v, _, qb, kb, aq, ak = _case(42, H=H, n=n, bias=False)
    _, _, mq = oracle.pack(xq, oracle.MEAN_SIGN)
    _, _, mk = oracle.pack(xk, oracle.MEAN_SIGN)
    yq, yk = xq - mq[:, :, None, :], xk - mk[:, :, None, :]
    b2 = _bias2d_case(5, H, gh, gw, cls)
    dense = _bias2d_dense(b2, H)
    N = 7
    res = oracle.attention(qb, kb, v, alpha_q=aq, alpha_k=ak, bias2d=b2, top_n=N, want_idx=True)
    B = xq.shape[0]
    dot = np.einsum("bhic,bhjc->bhij", _signs(yq), _signs(yk))
    l = (aq[..., :, None] * ak[..., None, :]).astype(np.float64) * dot / 8.0 + dense[None]
    keep = np.zeros((B, H, n, n), bool)
    for b in range(B):
        for h in range(H):
            for q in range(n):
                sel = _brute_topn(l[b, h, q], N)
                assert list(res["idx"][b, h, q]) == sel
                keep[b, h, q, sel] = True
    q = torch.from_numpy(_signs(yq) * aq[..., None].astype(np.float64))
    k = torch.from_numpy(_signs(yk) * ak[..., None].astype(np.float64))
    mask = torch.from_numpy(dense.astype(np.float64))[None].expand(B, -1, -1, -1).clone()
    mask[~torch.from_numpy(keep)] = float("-inf")
    want = torch.nn.functional.scaled_dot_product_attention(q, k, torch.from_numpy(v.astype(np.float64)),
                                                            attn_mask=mask).numpy()
    assert np.allclose(res["out"], want, rtol=1e-5, atol=1e-6)


# ------------------------------------------------------------------ quantized path
def test_vquant_closed_form_and_rounding():
    # per-channel scale s (a power of two) with max |V| = 127 s: scale is s exactly
    # and integer multiples come back unchanged; half-way values round to even.
    g = np.random.default_rng(15)
    d, n = 64, 50
    s = 2.0 ** g.integers(-6, 3, d)
    k = g.integers(-126, 127, (n, d)).astype(np.float64)
    k[0] = 127.0
    k[1] = -127.0
    v = (k * s).astype(np.float32)[None, None]
    vq, sc = oracle.vquant(v)
    assert np.array_equal(sc[0, 0], s.astype(np.float32))
    assert np.array_equal(vq[0, 0], k.astype(np.int8))
    col = np.array([2.5, -3.5, 0.5, 127.0], np.float32)
    vh = np.repeat(col[:, None], 32, axis=1)[None, None]
    vq2, sc2 = oracle.vquant(vh)
    assert sc2[0, 0, 0] == 1.0 and list(vq2[0, 0, :, 0]) == [2, -4, 0, 127]
    z = np.zeros((1, 1, 3, 32), np.float32)
    vq3, sc3 = oracle.vquant(z)
    assert np.all(vq3 == 0) and np.all(sc3 == 0)


def test_q8_uniform_attention_closed_form():
    # all logits equal -> p = 1/n, A_q = rint(255/n): O[c] = A_q * sum_j Vq[j,c] * s_c / 255
    n, d = 10, 64
    bits = np.zeros((1, 1, n, 2), np.uint32)
    v = np.random.default_rng(16).standard_normal((1, 1, n, d)).astype(np.float32)
    r = oracle.attention(bits, bits, v, top_n=None, av_mode=oracle.AV_Q8, want_aq8=True)
    a = int(np.rint(255 / n))
    assert np.all(r["aq8"] == a)
    acc = a * r["vq"][0, 0].astype(np.int64).sum(axis=0)
    want = ((acc.astype(np.float32) * r["vscale"][0, 0]).astype(np.float32) / np.float32(255)).astype(np.float32)
    assert np.array_equal(r["out"][0, 0], np.broadcast_to(want, (n, d)))


@pytest.mark.parametrize("N,d", [(5, 64), (None, 64), (5, 128)])
def test_q8_integer_product_and_error_bound(N, d):
    xq, xk, v, T, qb, kb, aq, ak = _case(17, n=40, d=d)
    fp = oracle.attention(qb, kb, v, alpha_q=aq, alpha_k=ak, bias=T, top_n=N, want_idx=True)
    q8 = oracle.attention(qb, kb, v, alpha_q=aq, alpha_k=ak, bias=T, top_n=N, av_mode=oracle.AV_Q8,
                          want_idx=True, want_aq8=True)
    assert np.array_equal(fp["idx"], q8["idx"])
    B, H, n, d = v.shape
    keep = q8["idx"].shape[-1]
    # integer accumulation = int64 matmul of A_q with the gathered Vq rows
    vq = torch.from_numpy(q8["vq"].astype(np.int64))
    idx = torch.from_numpy(q8["idx"].astype(np.int64))
    rows = torch.gather(vq[:, :, None].expand(B, H, n, n, d), 3,
                        idx[..., None].expand(B, H, n, keep, d))
    acc = torch.einsum("bhik,bhikc->bhic", torch.from_numpy(q8["aq8"].astype(np.int64)), rows).numpy()
    sc = q8["vscale"][:, :, None, :]
    want = ((acc.astype(np.float32) * sc).astype(np.float32) / np.float32(255)).astype(np.float32)
    assert np.array_equal(q8["out"], want)
    # sum of A_q within |S|/2 of 255; analytic bound against the fp path
    s = q8["aq8"].sum(-1)
    assert np.all(np.abs(s - 255) <= keep / 2)
    bound = (keep / 510.0) * 127 * sc + sc / 2 + 1e-6
    assert np.all(np.abs(q8["out"] - fp["out"]) <= bound)


def test_vquant_q4_closed_form_and_rounding():
    # 4-bit V (7 levels each side): per-channel scale s with max |V| = 7 s gives scale s
    # exactly and integer multiples back; half-way values round to even; |code| <= 7
    g = np.random.default_rng(18)
    d, n = 64, 50
    s = 2.0 ** g.integers(-6, 3, d)
    k = g.integers(-6, 7, (n, d)).astype(np.float64)
    k[0] = 7.0
    k[1] = -7.0
    v = (k * s).astype(np.float32)[None, None]
    vq, sc = oracle.vquant(v, 7)
    assert np.array_equal(sc[0, 0], s.astype(np.float32))
    assert np.array_equal(vq[0, 0], k.astype(np.int8))
    col = np.array([2.5, -3.5, 0.5, 7.0], np.float32)
    vh = np.repeat(col[:, None], 32, axis=1)[None, None]
    vq2, sc2 = oracle.vquant(vh, 7)
    assert sc2[0, 0, 0] == 1.0 and list(vq2[0, 0, :, 0]) == [2, -4, 0, 7]
    x = g.standard_normal((1, 2, 40, 64)).astype(np.float32)
    vq3, sc3 = oracle.vquant(x, 7)
    assert np.abs(vq3).max() == 7
    # the int8 quantizer of the same tensor is a different, finer grid
    vq4, sc4 = oracle.vquant(x, 127)
    assert np.allclose(sc4 * 127, sc3 * 7, rtol=1e-6)


@pytest.mark.parametrize("N", [5, None])
def test_q4_integer_product_and_error_bound(N):
    xq, xk, v, T, qb, kb, aq, ak = _case(19, n=40)
    fp = oracle.attention(qb, kb, v, alpha_q=aq, alpha_k=ak, bias=T, top_n=N, want_idx=True)
    q4 = oracle.attention(qb, kb, v, alpha_q=aq, alpha_k=ak, bias=T, top_n=N, av_mode=oracle.AV_Q4,
                          want_idx=True, want_aq8=True)
    assert np.array_equal(fp["idx"], q4["idx"])
    vq, sc = oracle.vquant(v, 7)
    assert np.array_equal(q4["vq"], vq) and np.array_equal(q4["vscale"], sc)
    B, H, n, d = v.shape
    keep = q4["idx"].shape[-1]
    vqt = torch.from_numpy(vq.astype(np.int64))
    idx = torch.from_numpy(q4["idx"].astype(np.int64))
    rows = torch.gather(vqt[:, :, None].expand(B, H, n, n, d), 3, idx[..., None].expand(B, H, n, keep, d))
    acc = torch.einsum("bhik,bhikc->bhic", torch.from_numpy(q4["aq8"].astype(np.int64)), rows).numpy()
    scb = sc[:, :, None, :]
    want = ((acc.astype(np.float32) * scb).astype(np.float32) / np.float32(255)).astype(np.float32)
    assert np.array_equal(q4["out"], want)
    # A_q rounding moves each weight by at most 1/510, V by at most s_c / 2
    bound = (keep / 510.0) * 7 * scb + scb / 2 + 1e-6
    assert np.all(np.abs(q4["out"] - fp["out"]) <= bound)


# ------------------------------------------------------------------ pages' constants
def test_golden_constants_from_the_pages():
    with open(os.path.join(GOLDEN, "page_constants.json")) as f:
        g = json.load(f)
    from binarized_qk_sparse_amd import synth
    for n, N in g["had_quality_topn"]["points"]:
        assert synth.c3(n).top_n == N
    assert synth.WORKLOADS["c2"].top_n == g["had_bert_topn"]["N"]
    assert synth.WORKLOADS["c2"].n == g["had_bert_topn"]["n"]
    assert synth.WORKLOADS["c1"].top_n == g["had_deit_topn"]["N"]
    assert synth.WORKLOADS["c1"].n == g["had_deit_topn"]["n"]
    # uint8 attention scale: A in [0,1] maps onto [0,255]
    assert g["binaryattention_a_scale"]["value"] == "1/255"
    n = 4
    bits = np.zeros((1, 1, n, 2), np.uint32)
    v = np.ones((1, 1, n, 64), np.float32)
    r = oracle.attention(bits, bits, v, top_n=1, av_mode=oracle.AV_Q8, want_aq8=True)
    assert np.all(r["aq8"] == 255)
