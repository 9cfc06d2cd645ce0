"""The bench's A_q flip count (host logic): differences planted in a copy of the oracle's
output, on the CPU, are found and counted."""
import numpy as np

import bench
import oracle
from binarized_qk_sparse_amd import synth


def _out_from(aq8, idx, vq, s):
    acc = (aq8.astype(np.int64)[:, None] * vq[idx].astype(np.int64)).sum(axis=0)
    return (acc.astype(np.float32) * s) / np.float32(255.0)


def test_planted_flips_are_counted():
    w = synth.Workload("t", 0, 1, 2, 96, 64, 20, "f32", synth.MEAN_SIGN, False, synth.AV_Q8, "iid")
    g = np.random.default_rng(5)
    q = g.standard_normal((1, 2, 96, 64)).astype(np.float32)
    k = g.standard_normal((1, 2, 96, 64)).astype(np.float32)
    v = g.standard_normal((1, 2, 96, 64)).astype(np.float32)
    qb, aq, _ = oracle.pack(q, w.mode)
    kb, ak, _ = oracle.pack(k, w.mode)
    rows = np.array([0, 5, 100, 150, 191], np.int64)
    ref = oracle.attention(qb, kb, v, alpha_q=aq, alpha_k=ak, top_n=20, av_mode=synth.AV_Q8, rows=rows,
                           want_idx=True, want_aq8=True)
    ref["rows"] = rows
    vq = ref["vq"].reshape(2, 96, 64)
    sc = ref["vscale"].reshape(2, 64).astype(np.float32)
    gpu = ref["out"].copy()
    flips, dif, unres = bench.aq_flips(w, gpu, ref)
    assert (flips, dif, unres) == (0, 0, 0)
    # one flip in row 1 (+1 on its third kept key), two in row 3
    for r, plant in ((1, {2: 1}), (3, {0: -1, 7: 1})):
        a = ref["aq8"][r].copy()
        for kk, dlt in plant.items():
            a[kk] += dlt
        bh = int(rows[r]) // 96
        gpu[r] = _out_from(a, ref["idx"][r], vq[bh], sc[bh])
    flips, dif, unres = bench.aq_flips(w, gpu, ref)
    assert (flips, dif, unres) == (3, 2, 0)
