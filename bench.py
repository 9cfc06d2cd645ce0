"""Benchmark of the binarized-QK attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c3@1024]

A step is one pass of the whole path over one batch already resident in HBM:
pack Q and K (one had_pack_qk call), then attention (which also quantizes V on
the q8 paths).  The K timed
steps are captured into one HIP graph, replayed once untimed and then once
inside the timed region, so that region holds GPU work only, with no host
launch gap between steps.  The line printed on stdout is the only output on
stdout:

  value         query-key pairs per second of the whole step (B*H*n^2 / time)
  roofline      the dominant kernel (attention) against the VALU issue roof:
                algorithmic VALU lane-slots per launch / the kernel's duration
                (HIP events on the stream it runs on: around 100 back-to-back
                launches while the host enqueues faster than the GPU runs them,
                else around each launch), against 256 CU * 64 lanes * 2.4 GHz;
                beside it the per-launch-pair mean and median, the median with L2
                and the last-level cache flushed before each launch (cold), and the
                fraction of the
                measured integer-VALU ceiling (libhad_ubench.so: XOR + popcount
                chains; also v_exp_f32 and a device copy)
  cpu_baseline  the CPU oracle timed on a bounded sample of the same workload
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "binarized-attention QK pairs/sec at n=1024,12 heads; % of roofline"
VALU_PEAK = 256 * 64 * 2.4e9  # lane-slots per second: 256 CUs x 64 lanes x 2.4 GHz
HBM_PEAK = 8.0e12
STREAM_MAX_KEEP = 1472  # most keys the streaming top-N kernel buffers per query (1536 entries less one tile)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_slots(w) -> float:
    """VALU lane-slots the method needs per attention launch.

    Per query row: n * (2W + 1 + F) for the logits (XOR and popcount per
    32-bit word, one compare for the selection, F = 4 conversion/scale/bias
    ops when alpha or a bias is present) plus, over the kept keys,
    6 (exp at quarter rate + subtract + sum) + d/2 (fp32 FMA, two per slot on
    packed hardware) for the fp32 A*V, or + d/4 (four 8-bit products per slot)
    for the int8 A*V; the dense int8 path adds 9 per key (max, exp, sum,
    quantize) and its contraction runs on the matrix cores.
    """
    W = w.d // 32
    F = 4 if (w.bias or w.mode == 1) else 0
    keep = w.kept
    if w.top_n is None:
        per_row = w.n * (2 * W + F + 9)
    else:
        per_row = w.n * (2 * W + 1 + F) + keep * (6 + (w.d / 2 if w.av_mode == 0 else w.d / 4))
    return per_row * w.B * w.H * w.n


def algorithmic_bytes(w) -> float:
    """HBM bytes the attention launch must move: codes, scales, bias table, V (or int8 V), O."""
    bh = w.B * w.H
    b = 2 * w.n * w.d / 8
    if w.mode == 1:
        b += 2 * 4 * w.n
    if w.bias:
        b += 4 * (2 * w.n - 1) / w.B
    vbytes = 2 if w.dtype == "bf16" else 4
    b += w.n * w.d * (1 if w.av_mode != 0 else vbytes) + (4 * w.d if w.av_mode != 0 else 0)
    b += 4 * w.n * w.d
    return b * bh


def attention_kernel(w, fused=False):
    """(kernel name, source file) of the attention launch, by the library's dispatch rule:
    dense softmax -> dense_q8 up to 256 tokens, dense_long beyond; n above the resident limit (512 keys for fp32 V, 1024
    otherwise, half that at head_dim 128) -> the streaming kernel, past its buffer -> the
    threshold-first kernel; head_dim 64 with bf16 V, plain sign codes, fp32 A*V and no
    table (up to 1024 tokens) or a 1-D table (up to 256) -> the matrix-core kernel, head_dim
    128 with no table (up to 1024 tokens, ahead of the resident limit) -> its head_dim 128
    instance; anything else, and the fused top-N launch -> the resident kernel."""
    if fused and w.top_n is not None:
        return "topn_resident_kernel", "topn.hip"
    if w.top_n is None:
        return ("dense_q8_kernel", "dense_q8.hip") if w.n <= 256 else ("dense_long_kernel", "dense_long.hip")
    if w.d == 128 and w.dtype == "bf16" and w.mode == 0 and not w.bias and w.av_mode == 0 and w.n <= 1024:
        return "topn_mfma_d128_kernel", "topn_mfma.hip"
    resident_max = 512 if (w.dtype == "f32" and w.av_mode == 0) else 1024
    if w.d == 128:
        resident_max //= 2  # rows twice as long in LDS
    if w.n > resident_max:
        if w.top_n > STREAM_MAX_KEEP:
            return "topn_wide_kernel", "topn_wide.hip"
        return "topn_stream_kernel", "topn_stream.hip"
    table_ok = not w.bias or (w.grid is None and w.n <= 256)
    if w.d == 64 and w.dtype == "bf16" and w.mode == 0 and table_ok and w.av_mode == 0:
        return "topn_mfma_kernel", "topn_mfma.hip"
    return "topn_resident_kernel", "topn.hip"


def path_dtype(w, kname: str) -> str:
    """The arithmetic types of the attention path: 1-bit codes for the logits, then the A*V
    operands.  The matrix-core top-N kernel multiplies bf16 V by softmax weights split into
    bf16 high and low parts (16 significant bits) and accumulates in fp32."""
    if w.av_mode == 1:
        return "b1+u8/i8"
    if w.av_mode == 2:
        return "b1+u8/i4"
    if kname in ("topn_mfma_kernel", "topn_mfma_d128_kernel"):
        return "b1+bf16x2 weights*bf16 V, f32 acc"
    return "b1+f32"


def traffic_from_profile(config: str, kernel: str, kernel_src: str):
    """HBM bytes per launch from the committed rocprof counter summary, if it was
    taken on this workload with the current kernel source; otherwise None."""
    path = os.path.join(ROOT, "profiles", f"{config.replace('@', '_n')}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    with open(kernel_src, "rb") as f:
        h = hashlib.sha256(f.read()).hexdigest()
    if rec.get("kernel_sha256") != h or not rec.get("kernel", "").startswith(kernel):
        return None
    return rec.get("bytes_per_launch")


def cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo (empty when unreadable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def aq_flips(w, gpu_rows, ref):
    """Count the u8 probabilities A_q where the GPU and the oracle differ, on the rows of one
    oracle call (q8/q4 A*V).  The V codes and scales are exact on both sides, so each output
    element O = fl(fl(acc) s_c) / 255 gives back the GPU's integer accumulator acc, and
    acc_gpu - acc_oracle = sum_j dA_j V_q[j, c] over the kept keys; a row's difference is
    matched against one key's V_q row (one flip) or two keys' (two flips), each of sign +-1.
    Returns (flips, rows with a difference, rows not resolved by one or two flips)."""
    import numpy as np

    vq = ref["vq"].reshape(-1, w.n, w.d).astype(np.int64)  # [B*H, n, d]
    sc = ref["vscale"].reshape(-1, w.d).astype(np.float32)  # [B*H, d]
    flips = differ = unresolved = 0
    for r, row in enumerate(ref["rows"]):
        bh = int(row) // w.n
        s = sc[bh]
        o = gpu_rows[r].astype(np.float32)
        a0 = np.rint(o.astype(np.float64) * 255.0 / np.where(s > 0, s, 1.0)).astype(np.int64)
        acc = np.full(w.d, np.iinfo(np.int64).min, np.int64)
        for dlt in (0, -1, 1, -2, 2):
            cand = a0 + dlt
            back = (cand.astype(np.float32) * s) / np.float32(255.0)
            hit = (back == o) & (acc == np.iinfo(np.int64).min)
            acc[hit] = cand[hit]
        keys = ref["idx"][r].astype(np.int64)
        want = (ref["aq8"][r].astype(np.int64)[:, None] * vq[bh, keys]).sum(axis=0)
        if np.any(acc == np.iinfo(np.int64).min):
            differ += 1
            unresolved += 1
            continue
        delta = acc - want
        if not delta.any():
            continue
        differ += 1
        rowsv = vq[bh, keys]  # [keep, d]
        one = np.nonzero(np.all(rowsv == delta, axis=1) | np.all(rowsv == -delta, axis=1))[0]
        if one.size:
            flips += 1
            continue
        found = False
        for sgn in ((1, -1) if len(keys) <= 1024 else ()):  # the pair search holds keep^2 d booleans
            rest = delta[None, :] - sgn * rowsv  # remove one key, look for a second
            hit = np.all(rest[:, None, :] == rowsv[None, :, :], axis=2) | np.all(rest[:, None, :] == -rowsv[None, :, :],
                                                                                     axis=2)
            if hit.any():
                found = True
                break
        if found:
            flips += 2
        else:
            unresolved += 1
    return flips, differ, unresolved


def cpu_baseline(w, g, budget_s: float, gpu_out=None):
    """The oracle, as it stands, on a bounded sample of rows of the same workload; on the
    quantized A*V path also the count of A_q flips between the GPU's output and the oracle's
    on the first sample of rows."""
    import numpy as np

    import oracle

    q = g["q"].float().numpy()
    k = g["k"].float().numpy()
    v = g["v"].float().numpy()
    t0 = time.perf_counter()
    qb, aq, _ = oracle.pack(q, w.mode)
    kb, ak, _ = oracle.pack(k, w.mode)
    t_pack = time.perf_counter() - t0
    if w.mode == 0:
        aq = ak = None
    bias = None if g["bias"] is None else g["bias"].numpy()
    b2 = None if g.get("bias2d") is None else {k: (x.numpy() if hasattr(x, "numpy") else x)
                                                for k, x in g["bias2d"].items()}
    total = w.B * w.H * w.n
    rows_done, t_att, count = 0, 0.0, 256
    rng = np.random.default_rng(12345)
    # doubling seeded samples of query rows until the budget is spent or the
    # sample covers as many rows as the workload holds
    flip_ref = None
    while t_att < budget_s and rows_done < total:
        size = min(count, total - rows_done)
        rows = np.sort(rng.choice(total, size=size, replace=False)).astype(np.int64)
        want = flip_ref is None and gpu_out is not None and w.av_mode != 0
        t1 = time.perf_counter()
        ref = oracle.attention(qb, kb, v, alpha_q=aq, alpha_k=ak, bias=bias, bias2d=b2, top_n=w.top_n,
                               av_mode=w.av_mode, rows=rows, want_idx=want, want_aq8=want)
        t_att += time.perf_counter() - t1
        if want:
            flip_ref = dict(ref, rows=rows)
        rows_done += len(rows)
        count *= 2
    per_row = t_att / rows_done + t_pack / total
    value = w.n / per_row  # pairs per second
    res = {
        "value": value,
        "unit": "pairs/s",
        "cores": oracle.threads(),
        "affinity_cpus": len(os.sched_getaffinity(0)),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"{rows_done} query rows of {w.name} (random, seeded) in {t_att:.1f} s plus the full Q/K pack "
                  f"({t_pack:.2f} s) scaled per row",
    }
    if flip_ref is not None:
        gpu_rows = gpu_out.reshape(-1, w.d)[flip_ref["rows"]]
        f, dif, unres = aq_flips(w, gpu_rows, flip_ref)
        res["aq_flips"] = {"flips": f, "rows_checked": int(len(flip_ref["rows"])), "rows_differing": dif,
                           "rows_unresolved": unres,
                           "note": "u8 probabilities that differ between the GPU and the oracle (fp32 vs fp64 exp)"}
    if w.n <= 1024:
        # the same oracle on one thread, on a sample of at most 1024 rows (attention only)
        threads = oracle.threads()
        oracle.set_threads(1)
        try:
            rows = np.sort(rng.choice(total, size=min(1024, total), replace=False)).astype(np.int64)
            t1 = time.perf_counter()
            oracle.attention(qb, kb, v, alpha_q=aq, alpha_k=ak, bias=bias, bias2d=b2, top_n=w.top_n,
                             av_mode=w.av_mode, rows=rows)
            res["value_1thread"] = w.n * len(rows) / (time.perf_counter() - t1)
        finally:
            oracle.set_threads(threads)
    return res


def measured_ceilings(torch, dev) -> dict:
    """Measured ceilings beside the datasheet peaks: integer VALU (independent XOR + popcount
    chains, 2 lane-ops per step, libhad_ubench.so), v_exp_f32, a 256 MiB device copy, and the
    VALU issue cycles one 16x16x32 bf16 matrix-core product takes from its SIMD (the same VALU
    chains with and without ten products per loop, three waves per SIMD)."""
    import ctypes

    lib = ctypes.CDLL(os.path.join(ROOT, "binarized_qk_sparse_amd", "libhad_ubench.so"))
    for f in (lib.hub_xor_bcnt, lib.hub_exp):
        f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        f.restype = ctypes.c_int
    lib.hub_coissue.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.hub_coissue.restype = ctypes.c_int
    blocks, iters = 256 * 16, 1024
    out = torch.empty(blocks * 256, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def timed(fn, reps=5):
        for _ in range(2):
            assert fn() == 0
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            assert fn() == 0
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / reps

    s = stream.cuda_stream
    t_x = timed(lambda: lib.hub_xor_bcnt(out.data_ptr(), blocks, iters, s))
    t_e = timed(lambda: lib.hub_exp(out.data_ptr(), blocks, iters, s))
    # three workgroups of four waves per CU: three waves per SIMD, as in the top-N kernel
    cblocks, citers = 256 * 3, 512
    t_v = timed(lambda: lib.hub_coissue(out.data_ptr(), cblocks, citers, 0, s))
    t_vm = timed(lambda: lib.hub_coissue(out.data_ptr(), cblocks, citers, 1, s))
    simd_valu = cblocks * 4 * citers * 120 / 1024  # VALU instructions per SIMD
    clock = simd_valu * 4 / t_v  # the VALU-only loop keeps the issue port busy
    simd_mfma = cblocks * 4 * citers * 10 / 1024
    nbytes = 256 << 20
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    t_c = timed(lambda: (dst.copy_(src), 0)[1])
    del src, dst, out
    valu = blocks * 256 * iters * 8 * 2 / t_x
    return {
        "valu_int_tlane_ops": valu / 1e12,
        "clock_ghz_at_full_valu": valu / (256 * 64) / 1e9,
        "exp_t_per_s": blocks * 256 * iters * 8 / t_e / 1e12,
        "copy_gb_per_s": 2 * nbytes / t_c / 1e9,
        "mfma_valu_issue_cycles": (t_vm - t_v) * clock / simd_mfma,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="c3@1024")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--fused", action="store_true",
                    help="a step is one launch that binarizes Q and K on chip: binattn_dense_q8_fused for dense "
                         "workloads with n <= 256 (in place of had_pack_qk + binattn_dense_q8), "
                         "had_attention_topn_fused for top-N workloads with fp32 A*V that one workgroup holds "
                         "(in place of had_pack_qk + had_attention_topn)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB five times (the reference kernel that scales "
                         "the HBM byte counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path shards by "
              f"(batch, head) with no communication, so the N-GPU figure is N times the one-GPU figure.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration > 0:
        nbytes = args.copy_calibration << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: 5 copies of {nbytes} bytes (reads {nbytes}, writes {nbytes} per copy)")
        return

    from binarized_qk_sparse_amd import ops, synth

    w = synth.workload(args.config)
    if args.fused and w.top_n is None and w.n > 256:
        print("--fused takes dense workloads with n <= 256 (c4)", file=sys.stderr)
        sys.exit(2)
    fused_cap = (512 if w.dtype == "f32" else 1024) // (w.d // 64)
    if args.fused and w.top_n is not None and (w.av_mode != 0 or w.n > fused_cap or (w.mode == 1 and w.n > 256)):
        print("--fused takes top-N workloads with fp32 A*V and n up to what one workgroup holds (c1, c2)",
              file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    g = synth.generate(w)
    q, k, v = (g[t].to(dev) for t in ("q", "k", "v"))
    bias = None if g["bias"] is None else g["bias"].to(dev)
    ws = ops.workspace(w.B, w.H, w.n, w.d, dev)
    out = torch.empty((w.B, w.H, w.n, w.d), dtype=torch.float32, device=dev)
    lib = ops._lib.load()
    dt = ops._dtype_code(q)
    W = w.d // 32
    qb = torch.empty((w.B, w.H, w.n, W), dtype=torch.int32, device=dev)
    kb = torch.empty_like(qb)
    aq = torch.empty((w.B, w.H, w.n), dtype=torch.float32, device=dev)
    ak = torch.empty_like(aq)
    mq = torch.empty((w.B, w.H, w.d), dtype=torch.float32, device=dev)
    mk = torch.empty_like(mq)
    pa = aq.data_ptr() if w.mode == 1 else None
    pk = ak.data_ptr() if w.mode == 1 else None
    pb = None if bias is None else bias.data_ptr()
    b2 = None
    if g.get("bias2d") is not None:  # two-dimensional decomposable bias: the *_2d entry points
        b2d = {k: (x.to(dev) if hasattr(x, "to") else x) for k, x in g["bias2d"].items()}
        b2 = (b2d["row"].data_ptr(), b2d["col"].data_ptr(), b2d["cls"].data_ptr() if "cls" in b2d else None,
              b2d["grid"][0], b2d["grid"][1])
        if args.fused:
            print("--fused takes the 1-D bias table only", file=sys.stderr)
            sys.exit(2)
    # plain sign codes: no scales or means to write (the attention call takes alpha = 1)
    pmq = mq.data_ptr() if w.mode == 1 else None
    pmk = mk.data_ptr() if w.mode == 1 else None

    def pack():
        s = torch.cuda.current_stream().cuda_stream  # the capture stream while a graph records
        ops._lib.check("had_pack_qk", lib.had_pack_qk(q.data_ptr(), k.data_ptr(), dt, w.B, w.H, w.n, w.d, w.mode,
                                                      qb.data_ptr(), kb.data_ptr(), pa, pk, pmq, pmk, ws.data_ptr(),
                                                      ws.numel(), s))

    def attend():
        s = torch.cuda.current_stream().cuda_stream
        if args.fused and w.top_n is not None:
            st = lib.had_attention_topn_fused(q.data_ptr(), k.data_ptr(), dt, w.mode, pb, v.data_ptr(),
                                              ops._dtype_code(v), w.B, w.H, w.n, w.d, w.top_n, out.data_ptr(), None,
                                              s)
        elif args.fused:
            st = lib.binattn_dense_q8_fused(q.data_ptr(), k.data_ptr(), dt, w.mode, pb, v.data_ptr(),
                                            ops._dtype_code(v), w.B, w.H, w.n, w.d, out.data_ptr(), s)
        elif w.top_n is None and b2 is not None:
            st = lib.binattn_dense_q8_2d(qb.data_ptr(), kb.data_ptr(), pa, pk, *b2, v.data_ptr(), dt, w.B, w.H, w.n,
                                         w.d, out.data_ptr(), ws.data_ptr(), ws.numel(), s)
        elif w.top_n is None:
            st = lib.binattn_dense_q8(qb.data_ptr(), kb.data_ptr(), pa, pk, pb, v.data_ptr(), dt, w.B, w.H, w.n,
                                      w.d, out.data_ptr(), ws.data_ptr(), ws.numel(), s)
        elif b2 is not None:
            st = lib.had_attention_topn_2d(qb.data_ptr(), kb.data_ptr(), pa, pk, *b2, v.data_ptr(), dt, w.B, w.H, w.n,
                                           w.d, w.top_n, w.av_mode, out.data_ptr(), None, ws.data_ptr(), ws.numel(),
                                           s)
        else:
            st = lib.had_attention_topn(qb.data_ptr(), kb.data_ptr(), pa, pk, pb, v.data_ptr(), dt, w.B, w.H, w.n,
                                        w.d, w.top_n, w.av_mode, out.data_ptr(), None, ws.data_ptr(), ws.numel(), s)
        ops._lib.check("attention", st)

    def step():
        if not args.fused:  # the fused launch binarizes Q and K itself
            pack()
        attend()

    # eager warm-up (also initialises the kernels' one-time launch attributes)
    for _ in range(3):
        step()
    torch.cuda.synchronize()
    # warm-up: W replays of a one-step graph; the timed region is ONE replay of a graph that holds
    # exactly K steps (so no host launch gap sits between steps), after one untimed replay of it
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(args.warmup):
        graph.replay()
    graph_k = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph_k):
        for _ in range(args.steps):
            step()
    graph_k.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    graph_k.replay()
    torch.cuda.synchronize()
    dt_s = (time.perf_counter() - t0) / args.steps
    log(f"{w.name}: step {dt_s * 1e6:.1f} us ({args.steps} steps in one graph replay)")
    del graph_k

    # the dominant kernel alone, on the stream it runs on.  Two HIP-event measurements:
    #  batch: one pair of events around R back-to-back eager launches.  While the host enqueues
    #         faster than the GPU runs them, the queue never drains and this is the kernel's
    #         steady-state duration, as rocprofv3 reports it;
    #  pairs: a pair of events around each launch, which adds the events' own overhead (a few
    #         microseconds), and so bounds the duration from above.
    # kernel_us is the batch figure when the host kept ahead of the GPU, else the pairs mean.
    R = 100
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    attend()
    torch.cuda.synchronize()
    h0 = time.perf_counter()
    e0.record(stream)
    for _ in range(R):
        attend()
    e1.record(stream)
    t_host = (time.perf_counter() - h0) / R
    torch.cuda.synchronize()
    t_batch = e0.elapsed_time(e1) / 1e3 / R
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(R)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(R)]
    for i in range(R):
        starts[i].record(stream)
        attend()
        ends[i].record(stream)
    torch.cuda.synchronize()
    durs = sorted(starts[i].elapsed_time(ends[i]) / 1e3 for i in range(R))
    t_pairs = sum(durs) / R
    t_med = durs[R // 2]
    host_ahead = t_host < 0.8 * t_batch
    t_att = t_batch if host_ahead else t_pairs
    log(f"{w.name}: attention {t_batch * 1e6:.2f} us per launch over {R} back-to-back launches "
        f"(host enqueue {t_host * 1e6:.1f} us/launch); {t_pairs * 1e6:.2f} us mean, {t_med * 1e6:.2f} us median "
        f"with events around each launch; using {'the batch' if host_ahead else 'the pairs'} figure")
    # cold: L2 and the last-level cache flushed by a 512 MiB read-modify-write before each launch
    flush = torch.zeros(128 << 20, dtype=torch.float32, device=dev)
    RC = 20
    cs = [torch.cuda.Event(enable_timing=True) for _ in range(RC)]
    ce = [torch.cuda.Event(enable_timing=True) for _ in range(RC)]
    for i in range(RC):
        flush.add_(1.0)
        cs[i].record(stream)
        attend()
        ce[i].record(stream)
    torch.cuda.synchronize()
    t_cold = sorted(cs[i].elapsed_time(ce[i]) / 1e3 for i in range(RC))[RC // 2]
    del flush
    log(f"{w.name}: attention {t_cold * 1e6:.2f} us median per launch, cold ({RC} launches)")
    ceil = measured_ceilings(torch, dev)
    log(f"measured ceilings: XOR+popcount {ceil['valu_int_tlane_ops']:.1f} T lane-ops/s "
        f"(clock ~{ceil['clock_ghz_at_full_valu']:.2f} GHz), v_exp_f32 {ceil['exp_t_per_s']:.2f} T/s, "
        f"device copy {ceil['copy_gb_per_s']:.0f} GB/s")

    slots = algorithmic_slots(w)
    achieved = slots / t_att
    kname, ksrc = attention_kernel(w, args.fused)
    src = os.path.join(ROOT, "binarized_qk_sparse_amd", "csrc", ksrc)
    traffic = traffic_from_profile(args.config, kname, src)
    roof = {
        "bound": "alu",
        "achieved": achieved / 1e12,
        "peak": VALU_PEAK / 1e12,
        "unit": "Tlane-slot/s",
        "frac": achieved / VALU_PEAK,
        "traffic": traffic,
        "kernel": kname,
        "kernel_us": t_att * 1e6,
        "kernel_us_batch": t_batch * 1e6,
        "kernel_us_event_pairs": t_pairs * 1e6,
        "kernel_us_event_pairs_median": t_med * 1e6,
        "kernel_us_cold_median": t_cold * 1e6,
        "frac_of_measured_valu_ceiling": achieved / (ceil["valu_int_tlane_ops"] * 1e12),
        "measured_ceilings": ceil,
        "slots_per_launch": slots,
        "hbm_bytes_per_launch_alg": algorithmic_bytes(w),
        "hbm_frac": algorithmic_bytes(w) / t_att / HBM_PEAK,
    }
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, g, args.cpu_budget, gpu_out=out.cpu().numpy())
        log(f"cpu baseline: {cpu['value']:.3e} pairs/s on {cpu['cores']} threads ({cpu['sample']})")
    kept = "dense" if w.top_n is None else f"N={w.top_n}"
    line = {
        "metric": METRIC,
        "value": w.pairs / dt_s,
        "unit": "pairs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": dt_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": path_dtype(w, kname),
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: B={w.B} H={w.H} n={w.n} d={w.d} {kept} {w.dtype} "
                        f"{'plain sign' if w.mode == 0 else 'mean-centred scaled sign'}"
                        f"{'' if not w.bias else (' + rel-pos bias' if w.grid is None else f' + 2-D rel-pos bias over a {w.grid[0]}x{w.grid[1]} grid')}"
                        f", {['fp32', 'uint8 x int8', 'uint8 x int4'][w.av_mode]} A*V",
            "global_batch": w.B,
            "heads": w.H,
            "seq_len": w.n,
            "head_dim": w.d,
            "top_n": w.top_n,
            "parallelism": "single GPU",
            "entry_points": ("binattn_dense_q8_fused" if w.top_n is None else "had_attention_topn_fused")
                            if args.fused else
                            ("had_pack_qk + " + ("binattn_dense_q8" if w.top_n is None else "had_attention_topn")),
        },
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
