"""binattn_dense_q8_noalloc through the C ABI: the same results as binattn_dense_q8 with a
caller workspace, on two calls in a row (the second smaller, so the static scratch
still holds the first call's larger contents), and the oracle's dense q8 attention
within one int8 LSB of V per element."""
import numpy as np
import pytest
import torch

import oracle
from binarized_qk_sparse_amd import ops, synth
from parity_util import f32, q8_tolerance

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _case(B, H, n, d, seed):
    g = np.random.default_rng([41, B, H, n, d, seed])
    xq = (g.standard_normal((B, H, n, d)) + 0.5 * g.standard_normal((1, H, 1, d))).astype(np.float32)
    xk = (g.standard_normal((B, H, n, d)) - 0.5 * g.standard_normal((1, H, 1, d))).astype(np.float32)
    v = torch.from_numpy((g.standard_normal((B, H, n, d)) * g.uniform(0.3, 2.0, (1, H, 1, d))).astype(np.float32))
    v = v.to(torch.bfloat16)
    T = (0.02 * g.standard_normal((H, 2 * n - 1))).astype(np.float32)
    qb, aq, _ = oracle.pack(xq, synth.MEAN_SIGN)
    kb, ak, _ = oracle.pack(xk, synth.MEAN_SIGN)
    return qb, kb, aq, ak, T, v


def test_noalloc_matches_workspace_entry_point_twice():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    for (B, H, n, d), seed in (((4, 3, 256, 64), 1), ((1, 2, 77, 128), 2)):
        print(f"noalloc case B={B} H={H} n={n} d={d}", flush=True)
        qb, kb, aq, ak, T, v = _case(B, H, n, d, seed)
        dt = lambda a: torch.from_numpy(a).to(DEV)
        args = (dt(qb.view(np.int32)), dt(kb.view(np.int32)), v.to(DEV))
        kw = dict(alpha_q=dt(aq), alpha_k=dt(ak), bias=dt(T))
        got = ops.binattn_dense_q8_noalloc(*args, **kw)
        torch.cuda.synchronize()
        want = ops.binattn_dense_q8(*args, **kw, ws=ops.workspace(B, H, n, d))
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"B={B} H={H} n={n} d={d}: differs from binattn_dense_q8"
        ref = oracle.attention(qb, kb, f32(v), alpha_q=aq, alpha_k=ak, bias=T, top_n=None, av_mode=oracle.AV_Q8)
        rows = np.arange(B * H * n)
        diff = np.abs(got.cpu().numpy().reshape(-1, d) - ref["out"].reshape(-1, d))
        assert np.all(diff <= q8_tolerance(ref["vscale"], rows, n) + 1e-6)


def test_noalloc_rejects_sizes_beyond_the_scratch():
    x = torch.zeros((256, 16, 256, 2), dtype=torch.int32, device=DEV)
    v = torch.zeros((256, 16, 256, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ops.HadError) as e:
        ops.binattn_dense_q8_noalloc(x, x, v)
    assert e.value.status == ops._lib.HAD_ERR_UNSUPPORTED
