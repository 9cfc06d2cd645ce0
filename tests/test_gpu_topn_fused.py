"""GPU parity of had_attention_topn_fused: binarization of Q and K on chip and the
top-N attention (fp32 A*V) in one launch.

Bar: the kept index sets equal those of had_pack_qk followed by had_attention_topn on
the same inputs, and the oracle's (bit-exact, ties to the lower key index); the outputs
are the same bits as that pair where it runs the resident kernel (fp32 V, mean-centred
codes, or a table at head_dim 128 or past 256 tokens), and within 1e-3 relative + 1e-4
absolute of the oracle everywhere.
"""
import numpy as np
import pytest
import torch

import oracle
from binarized_qk_sparse_amd import ops, synth
from parity_util import assert_close, f32

pytestmark = pytest.mark.gpu

DEV = "cuda"
SIGN, MEAN = synth.SIGN, synth.MEAN_SIGN


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    ops._lib.load()


def _inputs(B, H, n, d, qkdt, vdt, bias, seed):
    g = np.random.default_rng([91, B, H, n, d, seed])
    off = 0.6 * g.standard_normal((1, H, 1, d))  # per-channel offsets: the means matter
    q = torch.from_numpy((g.standard_normal((B, H, n, d)) + off).astype(np.float32)).to(qkdt)
    k = torch.from_numpy((g.standard_normal((B, H, n, d)) + off).astype(np.float32)).to(qkdt)
    v = torch.from_numpy(g.standard_normal((B, H, n, d)).astype(np.float32)).to(vdt)
    T = torch.from_numpy((0.05 * g.standard_normal((H, 2 * n - 1))).astype(np.float32)) if bias else None
    return q, k, v, T


def _pair_runs_resident(mode, vdt, bias, n, d):
    # had_attention_topn sends plain sign codes with bf16 V to the matrix-core kernel: at
    # head_dim 64 with a table only up to 256 tokens, at head_dim 128 without one
    return vdt == torch.float32 or mode == MEAN or (bias and (d == 128 or n > 256))


def _check(q, k, v, T, N, mode, what):
    dq, dk, dv = q.to(DEV), k.to(DEV), v.to(DEV)
    dT = None if T is None else T.to(DEV)
    out, idx = ops.had_attention_topn_fused(dq, dk, dv, N, mode, bias=dT, want_idx=True)
    (qb, aq, _), (kb, ak, _) = ops.had_pack_qk(dq, dk, mode)
    al = dict(alpha_q=aq, alpha_k=ak) if mode == MEAN else {}
    pout, pidx = ops.had_attention_topn(qb, kb, dv, N, bias=dT, want_idx=True, **al)
    torch.cuda.synchronize()
    out, idx, pout, pidx = out.cpu(), idx.cpu(), pout.cpu(), pidx.cpu()
    assert torch.equal(idx, pidx), f"{what}: kept index sets differ from pack + top-N"
    B, H, n, d = v.shape
    if _pair_runs_resident(mode, v.dtype, T is not None, n, d):
        assert torch.equal(out, pout), f"{what}: outputs differ from pack + top-N"
    oqb, oaq, _ = oracle.pack(f32(q), mode)
    okb, oak, _ = oracle.pack(f32(k), mode)
    if mode == SIGN:
        oaq = oak = None
    ref = oracle.attention(oqb, okb, f32(v), alpha_q=oaq, alpha_k=oak, bias=None if T is None else T.numpy(),
                           top_n=N, want_idx=True)
    assert np.array_equal(idx.numpy(), ref["idx"]), f"{what}: kept index sets differ from the oracle"
    assert_close(out.numpy(), ref["out"], what)


def test_single_image_workload():
    # three heads of one 197-token image, plain sign codes, fp32 Q, K and V, 30 keys kept
    w = synth.workload("c1")
    g = synth.generate(w)
    _check(g["q"], g["k"], g["v"], g["bias"], w.top_n, w.mode, "single image")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("bias", [False, True])
@pytest.mark.parametrize("vdt", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("qkdt", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("mode", [SIGN, MEAN])
def test_modes_dtypes_tables(mode, qkdt, vdt, bias, d):
    q, k, v, T = _inputs(2, 3, 197, d, qkdt, vdt, bias, 1)
    _check(q, k, v, T, 30, mode, f"mode={mode} qk={qkdt} v={vdt} bias={bias} d={d}")


@pytest.mark.parametrize("n", [1, 5, 64, 65, 100, 256])
@pytest.mark.parametrize("N", [1, 30, 5000])
@pytest.mark.parametrize("kind", ["sign_f32v", "mean_bias_bf16v"])
def test_sizes_and_kept_counts(kind, n, N):
    if kind == "sign_f32v":
        q, k, v, T = _inputs(2, 2, n, 64, torch.float32, torch.float32, False, 2)
        _check(q, k, v, T, N, SIGN, f"{kind} n={n} N={N}")
    else:
        q, k, v, T = _inputs(2, 2, n, 64, torch.bfloat16, torch.bfloat16, True, 2)
        _check(q, k, v, T, N, MEAN, f"{kind} n={n} N={N}")


@pytest.mark.parametrize("n,d,vdt", [(512, 64, torch.float32), (1024, 64, torch.bfloat16),
                                     (256, 128, torch.float32), (512, 128, torch.bfloat16), (777, 64, torch.bfloat16)])
@pytest.mark.parametrize("bias", [False, True])
def test_longest_resident_sequences(n, d, vdt, bias):
    # plain sign codes up to what one workgroup holds; many workgroups share each head
    q, k, v, T = _inputs(1, 2, n, d, torch.bfloat16, vdt, bias, 3)
    _check(q, k, v, T, max(1, (15 * n) // 128), SIGN, f"n={n} d={d} v={vdt} bias={bias}")


@pytest.mark.parametrize("mode", [SIGN, MEAN])
def test_zeros_and_constant_channels(mode):
    # channels equal to their mean (x - mu = 0 codes +1), negative zeros, and keys equal
    # to each other: the codes and the ties must match had_pack's
    n, d = 150, 64
    q, k, v, T = _inputs(1, 2, n, d, torch.float32, torch.float32, True, 4)
    q[..., :8] = 0.75
    k[..., 8:16] = -0.0
    k[:, :, 40:80] = k[:, :, 40:41]
    q[:, :, ::7, 16:24] = -0.0
    for N in (1, 45, 149):
        _check(q, k, v, T, N, mode, f"constant channels mode={mode} N={N}")


def test_every_key_equal():
    # one key code and one scale for the whole head: the kept set is the N lowest indices
    n, d, N = 200, 64, 50
    q, k, v, _ = _inputs(1, 1, n, d, torch.float32, torch.bfloat16, False, 5)
    k[:] = k[:, :, :1]
    _check(q, k, v, None, N, MEAN, "every key equal")
    out, idx = ops.had_attention_topn_fused(q.to(DEV), k.to(DEV), v.to(DEV), N, MEAN, want_idx=True)
    assert torch.equal(idx.cpu().reshape(-1, N), torch.arange(N, dtype=torch.int32).expand(n, N))


def test_graph_replays_match_eager():
    q, k, v, T = _inputs(2, 3, 197, 64, torch.bfloat16, torch.float32, True, 6)
    dq, dk, dv, dT = q.to(DEV), k.to(DEV), v.to(DEV), T.to(DEV)
    eager = ops.had_attention_topn_fused(dq, dk, dv, 30, MEAN, bias=dT)
    out = torch.empty_like(eager)
    ops.had_attention_topn_fused(dq, dk, dv, 30, MEAN, bias=dT, out=out)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ops.had_attention_topn_fused(dq, dk, dv, 30, MEAN, bias=dT, out=out)
    for _ in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
