#!/usr/bin/env python3
"""Benchmark of the sink-attention hot path on one MI355X.

Default run (one JSON line on stdout):
  * headline: paged split-KV decode, 64 requests with KV lengths uniform in
    [1, 4096], 64 query / 8 KV heads, head_dim 64, page size 16, pages
    permuted in a shared pool, sinks N(0, 2).  One step = one whole pass of
    the decode path: per-(request, KV head, chunk) split decode (chunk bounds
    computed on the device, paged gather, scores, mask, streaming softmax
    with the sink in chunk 0, P.V, partials) followed by the LSE merge.
    ``value`` = algorithmic HBM bytes / step time (GB/s), inputs resident in
    HBM, three replicas of the KV pool rotated so no step finds its KV in the
    256 MB Infinity Cache.  The K timed steps are captured in one HIP graph
    and replayed, as a serving loop issues its decode steps; the time of the
    same steps issued one by one is reported beside it.
  * ``roofline``: the decode kernel alone, timed with HIP events on the
    stream it runs on, against 8 TB/s.
  * ``prefill``: causal prefill, 4 x 8192 tokens, 64/8 heads: TFLOP/s of
    4 * head_dim flops per visible (query, key, head) against 2.5 PFLOP/s.
  * ``cpu_baseline``: the fp64 oracle on the host, timed on the whole decode
    workload, plus the parity of the timed GPU output against it.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor spec
MFMA_PEAK_TFLOPS = 2500.0      # MI355X dense bf16/fp16 MFMA, vendor spec
METRIC = "decode HBM GB/s (% peak) + prefill TFLOP/s (% MFMA peak), oracle-matched"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--splits", type=int, default=0, help="decode split count (0: library's pick)")
    p.add_argument("--replicas", type=int, default=3)
    p.add_argument("--prefill-steps", type=int, default=20)
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--workload", default="paged_decode",
                   choices=["paged_decode", "long_split_decode", "causal_prefill", "mixed_batch", "tiny_prefill",
                            "verify_decode", "verify_tree", "append_rope", "moe_topk",
                            "copy_calibration"],
                   help="for profiling runs: time only this workload (copy_calibration: a plain "
                        "256 MiB device copy, the reference for HBM byte counters)")
    return p.parse_args()


# ---------------------------------------------------------------------------
# algorithmic work
# ---------------------------------------------------------------------------

def decode_bytes(w):
    """K + V of every live key once per KV head, + Q + out of every query row
    + metadata."""
    kv = int(np.sum(w.kv_len, dtype=np.int64)) * w.num_kv_heads * w.head_dim * 2 * 2
    qo = 2 * int(w.qo_indptr[-1]) * w.num_qo_heads * w.head_dim * 2
    meta = 4 * (len(w.page_indices) + 2 * w.batch + 1)
    return kv + qo + meta


def prefill_flops(w, window=0):
    """4 * head_dim per visible (query, key, head)."""
    vis = 0
    for b in range(w.batch):
        n_q, n_k = int(w.qo_len[b]), int(w.kv_len[b])
        p = n_k - n_q + np.arange(n_q, dtype=np.int64)
        lo = np.maximum(0, p - window + 1) if window > 0 else np.zeros_like(p)
        vis += int(np.sum(p - lo + 1))
    return 4 * w.head_dim * vis * w.num_qo_heads


# ---------------------------------------------------------------------------
# GPU runs
# ---------------------------------------------------------------------------

class Dev:
    def __init__(self, w, torch, dev):
        def bits(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

        def i32(a):
            return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
        self.q = bits(w.q)
        self.qo_indptr = i32(w.qo_indptr)
        self.k = bits(w.k)
        self.v = bits(w.v)
        self.kv_indptr = i32(w.kv_indptr)
        self.kv_len = i32(w.kv_len)
        self.page_indices = i32(w.page_indices) if w.paged else None
        self.sinks = torch.from_numpy(w.sinks).to(dev)

    def replica(self):
        r = Dev.__new__(Dev)
        r.__dict__ = {k: (v.clone() if v is not None else None) for k, v in self.__dict__.items()}
        return r


def time_decode(w, args, torch, dev):
    """Decode + merge steps through the C ABI with prebuilt arguments (the
    Python binding's checks would otherwise cost more than a step).  The
    step time is that of the K steps captured in one HIP graph and replayed
    (as a serving loop issues its decode steps); the same steps issued one by
    one from Python are timed beside it.  The output checked against the
    oracle is the graph replay's."""
    import ctypes
    import gqa_attention_sinks_amd as sa
    from gqa_attention_sinks_amd import binding
    lib = sa.load_library()
    base = Dev(w, torch, dev)
    reps = [base] + [base.replica() for _ in range(max(0, args.replicas - 1))]
    s = args.splits if args.splits > 0 else (w.num_splits or sa.pick_num_splits(w.kv_len, w.num_kv_heads))
    B, H, HKV = w.batch, w.num_qo_heads, w.num_kv_heads
    outs = [torch.empty_like(r.q) for r in reps]
    o_part = torch.empty((B, H, s, 64), dtype=torch.float32, device=dev)
    lse_part = torch.empty((B, H, s), dtype=torch.float32, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = ctypes.c_void_p
    kvs = [binding.kv_descriptor(r.k, r.v, r.kv_indptr, r.page_indices, r.kv_len) for r in reps]
    qp = [P(r.q.data_ptr()) for r in reps]
    sk = [P(r.sinks.data_ptr()) for r in reps]
    op = [P(o.data_ptr()) for o in outs]
    opart, lpart, lsep = P(o_part.data_ptr()), P(lse_part.data_ptr()), P(lse.data_ptr())
    scale = ctypes.c_float(w.scale)

    def step(i, sp=sp):
        r = i % len(reps)
        if s > 1:
            st = lib.sinkattn_decode_paged(qp[r], ctypes.byref(kvs[r]), sk[r], s, None, opart, lpart, None,
                                           B, H, HKV, 64, scale, 0, sp)
            st |= lib.sinkattn_merge(opart, lpart, B, H, s, 64, op[r], lsep, sp)
        else:
            st = lib.sinkattn_decode_paged(qp[r], ctypes.byref(kvs[r]), sk[r], 1, op[r], None, None, lsep,
                                           B, H, HKV, 64, scale, 0, sp)
        if st != 0:
            raise RuntimeError(lib.sinkattn_last_error().decode())

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall_eager = (time.perf_counter() - t0) / args.steps
    # the same K steps captured in one graph (on a side stream), replayed once
    # untimed and once timed
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    side_p = ctypes.c_void_p(side.cuda_stream)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for i in range(args.steps):
                step(i, side_p)
    torch.cuda.synchronize()
    for o in outs:
        o.zero_()
    graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    graph.replay()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    last = (args.steps - 1) % len(reps)
    out_host = outs[last].float().cpu().numpy().astype(np.float64)
    # the decode kernel alone: K back-to-back launches between two events on
    # the stream they run on (rotating the replicas), then the merge alone
    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    e0.record(stream)
    for i in range(args.steps):
        r = i % len(reps)
        if s > 1:
            st = lib.sinkattn_decode_paged(qp[r], ctypes.byref(kvs[r]), sk[r], s, None, opart, lpart, None,
                                           B, H, HKV, 64, scale, 0, sp)
        else:
            st = lib.sinkattn_decode_paged(qp[r], ctypes.byref(kvs[r]), sk[r], 1, op[r], None, None, lsep,
                                           B, H, HKV, 64, scale, 0, sp)
        if st != 0:
            raise RuntimeError(lib.sinkattn_last_error().decode())
    e1.record(stream)
    if s > 1:
        for i in range(args.steps):
            lib.sinkattn_merge(opart, lpart, B, H, s, 64, op[i % len(reps)], lsep, sp)
    e2.record(stream)
    torch.cuda.synchronize()
    dec_ms = e0.elapsed_time(e1) / args.steps
    mer_ms = e1.elapsed_time(e2) / args.steps if s > 1 else 0.0
    return dict(step_ms=wall * 1e3, step_ms_eager=wall_eager * 1e3, decode_ms=dec_ms, merge_ms=mer_ms, splits=s,
                out=out_host)


def time_verify(w, args, torch, dev):
    """Several query rows per request (sinkattn_decode_paged_multi): the
    decode kernel alone between two events on its stream, replicas rotated,
    and the whole step (decode + merge) by wall clock."""
    import ctypes
    import gqa_attention_sinks_amd as sa
    from gqa_attention_sinks_amd import binding
    lib = sa.load_library()
    base = Dev(w, torch, dev)
    reps = [base] + [base.replica() for _ in range(max(0, args.replicas - 1))]
    R = int(w.meta["max_rows"])
    s = args.splits if args.splits > 0 else sa.pick_num_splits_multi(w.kv_len, w.num_qo_heads, w.num_kv_heads, R,
                                                                     with_mask="masks" in w.meta)
    B, H, HKV = w.batch, w.num_qo_heads, w.num_kv_heads
    TQ = int(w.qo_indptr[-1])
    outs = [torch.empty_like(r.q) for r in reps]
    o_part = torch.empty((TQ, H, s, 64), dtype=torch.float32, device=dev)
    lse_part = torch.empty((TQ, H, s), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = ctypes.c_void_p
    kvs = [binding.kv_descriptor(r.k, r.v, r.kv_indptr, r.page_indices, r.kv_len) for r in reps]
    scale = ctypes.c_float(w.scale)
    opart, lpart = P(o_part.data_ptr()), P(lse_part.data_ptr())
    mask = mask_ptr = None
    if "masks" in w.meta:            # a draft tree per request (custom mask)
        from gqa_attention_sinks_amd import workloads as wl
        bits, indptr = wl.pack_masks(w.meta["masks"])
        mask_t = torch.from_numpy(bits).to(dev)
        mask_indptr_t = torch.from_numpy(indptr).to(dev)
        mask, mask_ptr = P(mask_t.data_ptr()), P(mask_indptr_t.data_ptr())

    def call(i, merge):
        r = reps[i % len(reps)]
        out = P(outs[i % len(reps)].data_ptr()) if (merge or s == 1) else None
        st = lib.sinkattn_decode_paged_multi(P(r.q.data_ptr()), P(r.qo_indptr.data_ptr()), mask, mask_ptr,
                                             ctypes.byref(kvs[i % len(reps)]), P(r.sinks.data_ptr()), s, out,
                                             opart if s > 1 else None, lpart if s > 1 else None, None,
                                             B, TQ, R, H, HKV, 64, scale, 0, sp)
        if st != 0:
            raise RuntimeError(lib.sinkattn_last_error().decode())

    for i in range(args.warmup):
        call(i, True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        call(i, True)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        call(i, False)
    e1.record(stream)
    torch.cuda.synchronize()
    return dict(step_ms=wall * 1e3, decode_ms=e0.elapsed_time(e1) / args.steps, splits=s)


def per_call_ms(call, args, torch):
    """Time per call of a short kernel.  ``ms``: ``args.steps`` calls captured
    in one HIP graph and replayed, so the host's launch rate does not enter
    (these kernels run for a few microseconds, about what a launch from Python
    costs); ``ms_eager``: the same calls issued one by one from Python."""
    for _ in range(args.warmup):
        call()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_eager = e0.elapsed_time(e1) / args.steps
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(args.steps):
            call()
    g.replay()
    torch.cuda.synchronize()
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / args.steps, ms_eager


def time_append(args, torch, dev):
    """Paged KV append with rotary embedding of queries and keys
    (sinkattn_append_paged_kv_rope): 16 prefill chunks of 512 tokens on
    prefixes uniform in [0, 16384], 64 query / 8 KV heads, random pages."""
    import gqa_attention_sinks_amd as sa
    from gqa_attention_sinks_amd import workloads as wl
    rng = np.random.default_rng(0)
    kv_len = (rng.integers(0, 16385, size=16) + 512).astype(np.int32)
    n_new = np.full(16, 512, dtype=np.int32)
    hq, hkv = 64, 8
    append_indptr = np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32)
    n_pages = (kv_len + 15) // 16
    page_indptr = np.concatenate([[0], np.cumsum(n_pages)]).astype(np.int32)
    pool = int(page_indptr[-1])
    page_indices = rng.permutation(pool).astype(np.int32)
    t = int(append_indptr[-1])
    bits = lambda shape: torch.from_numpy(wl._normal_bf16(rng, shape).view(np.int16)).to(dev).view(torch.bfloat16)
    i32 = lambda a: torch.from_numpy(a).to(dev)
    q, k, v = bits((t, hq, 64)), bits((t, hkv, 64)), bits((t, hkv, 64))
    kp, vp = bits((pool, hkv, 16, 64)), bits((pool, hkv, 16, 64))
    f = np.arange(32)
    ang = np.arange(int(kv_len.max()) + 1)[:, None] * 10000.0 ** (-2.0 * f / 64)[None, :]
    table = torch.from_numpy(np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)).to(dev)
    q_out = torch.empty_like(q)
    args_ = (k, v, i32(append_indptr), kp, vp, i32(page_indptr), i32(page_indices), i32(kv_len), table)
    ms, ms_eager = per_call_ms(lambda: sa.append_paged_kv_rope(*args_, q=q, q_out=q_out), args, torch)
    nbytes = t * (2 * hq * 128 + 4 * hkv * 128 + 256) + 4 * (len(page_indices) + 3 * 17)
    return dict(tokens=t, ms=ms, ms_eager=ms_eager, bytes=nbytes, GBs=nbytes / (ms * 1e-3) / 1e9)


def time_moe(args, torch, dev):
    """MoE routing weights (sinkattn_moe_topk_softmax): 65536 tokens of bf16
    router logits N(0, 1), 128 experts, top 4."""
    import gqa_attention_sinks_amd as sa
    from gqa_attention_sinks_amd import workloads as wl
    t, e, k = 65536, 128, 4
    logits = torch.from_numpy(wl._normal_bf16(np.random.default_rng(0), (t, e)).view(np.int16)).to(dev)
    logits = logits.view(torch.bfloat16)
    idx = torch.empty((t, k), dtype=torch.int32, device=dev)
    w = torch.empty((t, k), dtype=torch.bfloat16, device=dev)
    ms, ms_eager = per_call_ms(lambda: sa.moe_topk_softmax(logits, k, idx, w), args, torch)
    nbytes = t * (e * 2 + k * 6)
    return dict(tokens=t, experts=e, top_k=k, ms=ms, ms_eager=ms_eager, bytes=nbytes,
                GBs=nbytes / (ms * 1e-3) / 1e9)


def time_prefill(w, steps, warmup, torch, dev, window=0):
    from gqa_attention_sinks_amd import binding
    d = Dev(w, torch, dev)
    out = torch.empty_like(d.q)
    stream = torch.cuda.current_stream()

    host = np.ascontiguousarray(w.qo_indptr, dtype=np.int32)

    def call():
        binding.prefill(d.q, d.qo_indptr, d.k, d.v, d.kv_indptr, d.sinks, w.scale, window=window,
                        page_indices=d.page_indices, kv_len=d.kv_len if w.paged else None, out=out,
                        qo_indptr_host=host)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    return dict(step_ms=wall * 1e3, kernel_ms=e0.elapsed_time(e1) / steps, out=out)


def measured_traffic(kernel, workload, splits):
    """HBM bytes per launch from the committed FETCH_SIZE/WRITE_SIZE runs, or
    None when the kernel's sources changed since they were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(kernel)
    csrc = os.path.join(ROOT, "gqa_attention_sinks_amd", "csrc")
    files = [os.path.join(csrc, f) for f in ("decode.hip", "device_common.hpp", "kernel_args.hpp")]
    digest = hashlib.sha256(b"".join(open(f, "rb").read() for f in files)).hexdigest()
    if not rec or rec.get("source_sha256") != digest or rec.get("workload") != workload \
            or rec.get("num_splits") != splits:
        return None
    return int(round(rec["bytes"]))


def parity(g, r):
    err = np.abs(g - r)
    return dict(max_abs=float(err.max()), within_tol=bool(np.all(err <= 2e-3 + 1e-2 * np.abs(r))))


def cpu_baseline(w, gpu_out, min_seconds=10.0):
    """The fp64 oracle (as it stands) on the whole decode workload, one
    thread, repeated until about ten seconds of CPU work have been timed (a
    pass takes a fraction of a second); the rate is the mean over the
    passes."""
    import oracle
    from threadpoolctl import threadpool_limits
    kv = oracle.KVCache(k=w.k, v=w.v, kv_indptr=w.kv_indptr, paged=True, page_indices=w.page_indices,
                        kv_len=w.kv_len)
    passes, dt = 0, 0.0
    with threadpool_limits(limits=1):
        while dt < min_seconds and passes < 1000:
            t0 = time.perf_counter()
            ro, _ = oracle.sink_attention_ref(w.q, w.qo_indptr, kv, w.sinks, w.scale, 0, workers=1)
            dt += time.perf_counter() - t0
            passes += 1
    return dict(value=passes * decode_bytes(w) / dt / 1e9, unit="GB/s", cores=1, kind="oracle",
                sample=f"whole workload ({w.batch} requests, {int(w.kv_len.sum())} keys), fp64 numpy, "
                       f"{passes} passes in {dt:.1f} s", seconds=dt), parity(gpu_out, ro)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); sharding the path over several "
              "GPUs is not built", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import gqa_attention_sinks_amd as sa
    from gqa_attention_sinks_amd import workloads as wl
    if not os.path.exists(sa.library_path()):
        import __graft_entry__
        __graft_entry__.build()
    sa.load_library()
    dev = torch.device("cuda:0")

    if args.workload not in ("paged_decode",):
        return profile_only(args, torch, dev, wl)

    log("generating paged_decode workload")
    w = wl.paged_decode()
    res = time_decode(w, args, torch, dev)
    nbytes = decode_bytes(w)
    value = nbytes / (res["step_ms"] * 1e-3) / 1e9
    achieved = nbytes / (res["decode_ms"] * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["step_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "paged decode: batch 64, one query token each, KV lengths uniform in [1, 4096], "
                        "64 query / 8 KV heads, head_dim 64, page size 16, pages permuted in a shared pool, "
                        "sinks N(0, 2), seed 0",
            "num_splits": res["splits"],
            "kv_replicas_rotated": args.replicas,
            "algorithmic_bytes": nbytes,
            "compute": "bf16 Q.K^T and fp16 P.V on MFMA, fp32 accumulation",
            "step": "K steps (decode + merge launches) captured in one HIP graph, replayed",
            "ms_per_step_eager": round(res["step_ms_eager"], 5),
            "decode_kernel_ms": round(res["decode_ms"], 5),
            "merge_kernel_ms": round(res["merge_ms"], 5),
            "pct_hbm_peak_step": round(100 * value / HBM_PEAK_GBS, 2),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic("decode_paged_kernel", "paged_decode", res["splits"]),
            "kernel": "decode_paged_kernel",
        },
    }
    if not args.no_prefill:
        log("generating causal_prefill workload")
        wp = wl.causal_prefill()
        pr = time_prefill(wp, args.prefill_steps, 3, torch, dev)
        flops = prefill_flops(wp)
        tflops = flops / (pr["kernel_ms"] * 1e-3) / 1e12
        line["prefill"] = {
            "workload": "causal prefill: batch 4 x 8192 tokens, 64 query / 8 KV heads, head_dim 64, contiguous KV, "
                        "sinks N(0, 2)",
            "value": round(tflops, 1),
            "unit": "TFLOP/s",
            "ms_per_call": round(pr["kernel_ms"], 4),
            "algorithmic_flops": flops,
            "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / MFMA_PEAK_TFLOPS, 4), "traffic": None,
                         "kernel": "prefill_kernel"},
        }
        del pr
    if not args.no_cpu:
        log("timing the oracle on the host")
        cb, par = cpu_baseline(w, res["out"])
        line["cpu_baseline"] = {k: v for k, v in cb.items() if k != "seconds"}
        line["parity"] = par
    print(json.dumps(line), flush=True)


def profile_only(args, torch, dev, wl):
    """Time one named workload only (for rocprofv3 runs)."""
    if args.workload == "copy_calibration":
        n = 256 << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / args.steps
        print(json.dumps({"workload": "copy_calibration", "bytes_read": n, "bytes_written": n,
                          "ms": dt * 1e3, "GBs_rw": 2 * n / dt / 1e9}))
        return
    if args.workload == "moe_topk":
        r = time_moe(args, torch, dev)
        print(json.dumps({"workload": "moe_topk", **r, "frac": r["GBs"] / HBM_PEAK_GBS}))
        return
    if args.workload == "append_rope":
        r = time_append(args, torch, dev)
        print(json.dumps({"workload": "append_rope", **r, "frac": r["GBs"] / HBM_PEAK_GBS}))
        return
    w = getattr(wl, args.workload)()
    log(f"timing {args.workload}")
    if args.workload in ("verify_decode", "verify_tree"):
        res = time_verify(w, args, torch, dev)
        gbs = decode_bytes(w) / (res["decode_ms"] * 1e-3) / 1e9
        print(json.dumps({"workload": args.workload, "rows": int(w.qo_indptr[-1]), "splits": res["splits"],
                          "step_ms": res["step_ms"], "decode_ms": res["decode_ms"], "decode_GBs": gbs,
                          "frac": gbs / HBM_PEAK_GBS}))
        return
    if args.workload == "long_split_decode":
        res = time_decode(w, args, torch, dev)
        gbs = decode_bytes(w) / (res["decode_ms"] * 1e-3) / 1e9
        print(json.dumps({"workload": args.workload, "step_ms": res["step_ms"],
                          "step_ms_eager": res["step_ms_eager"], "decode_ms": res["decode_ms"],
                          "merge_ms": res["merge_ms"], "decode_GBs": gbs, "frac": gbs / HBM_PEAK_GBS}))
        return
    for window in w.windows:
        pr = time_prefill(w, args.steps, args.warmup, torch, dev, window=window)
        flops = prefill_flops(w, window)
        print(json.dumps({"workload": args.workload, "window": window, "ms": pr["kernel_ms"],
                          "TFLOPs": flops / (pr["kernel_ms"] * 1e-3) / 1e12}))


if __name__ == "__main__":
    main()
