#!/usr/bin/env python3
"""Benchmark of the sink-attention hot path on one MI355X.

Default run (one JSON line on stdout), every workload at full size, inputs
resident in HBM before any timed region:

  * headline (``value``): paged split-KV decode, 64 requests with KV lengths
    uniform in [1, 4096], 64 query / 8 KV heads, head_dim 64, page size 16,
    pages permuted in a shared pool, sinks N(0, 2).  One step = one whole pass
    of the decode path: per-(request, KV head, chunk) split decode (chunk
    bounds computed on the device, paged gather, scores, mask, streaming
    softmax with the sink in chunk 0, P.V, partials) and the LSE merge.
    ``value`` = algorithmic HBM bytes / step time (GB/s); three replicas of
    the KV pool are rotated so that no step finds its KV in the 256 MB
    Infinity Cache.  The K timed steps are captured in one HIP graph and
    replayed, as a serving loop issues its decode steps; the same steps
    issued one by one are timed beside it.
  * ``roofline``: the decode kernel alone, each launch timed with HIP events
    on the stream it runs on, against 8 TB/s.
  * ``configs``: every workload -- tiny prefill, paged decode, causal
    prefill 4 x 8192, long split decode (8 x 131072 keys, 16 chunks + merge),
    and the mixed chunked-prefill + decode batch under a 128-key window and
    under full causal attention (its prefill and decode kernels timed apart,
    plus the whole call against the sum of their roofline times).  Each
    kernel carries mean / median / p10 / p90 launch times, its algorithmic
    work and its fraction of the roofline; each workload carries a parity
    summary of the timed output against the fp64 oracle.
  * ``cpu_baseline``: the fp64 oracle, as it stands, timed on the host's
    cores in this same run (a process pool over request sub-batches, one
    BLAS thread per process), before the GPU is touched; per workload a
    stated sample.  Its outputs are the parity reference above.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
       python bench.py --workload NAME     (one workload only, for profiling)
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
ATOL, RTOL = 2e-3, 1e-2        # per element |gpu - ref| <= ATOL + RTOL * |ref|

WORKLOADS = ["paged_decode", "tiny_prefill", "causal_prefill", "long_split_decode", "mixed_batch", "skewed_decode",
             "verify_decode", "verify_tree", "append_rope", "moe_topk", "copy_calibration"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--splits", type=int, default=0, help="split decode: split count (0: library's pick)")
    p.add_argument("--segments", type=int, default=0, help="balanced decode: segment count (0: library's pick)")
    p.add_argument("--decode", default="split", choices=["balanced", "split"],
                   help="the decode path of the headline (the other is timed beside it)")
    p.add_argument("--replicas", type=int, default=3)
    p.add_argument("--no-host-order", action="store_true",
                   help="paged decode calls without the host copy of kv_len (the kernels rank the batch)")
    p.add_argument("--no-cpu", action="store_true", help="skip the oracle (no cpu_baseline, no parity)")
    p.add_argument("--workload", default=None, choices=WORKLOADS,
                   help="for profiling runs: time only this workload (copy_calibration: a plain 256 MiB "
                        "device copy, the reference for HBM byte counters)")
    return p.parse_args()


# ---------------------------------------------------------------------------
# algorithmic work
# ---------------------------------------------------------------------------

def visible_keys(w, window=0):
    """Per request, the keys some query row sees: row t of a request with
    n_q rows over n_k keys sits at n_k - n_q + t, so the union of the rows'
    ranges holds min(n_k, n_q + W - 1) keys under a window W, n_k without."""
    n_k = np.asarray(w.kv_len, dtype=np.int64)
    if window <= 0:
        return n_k
    return np.minimum(n_k, np.diff(np.asarray(w.qo_indptr, dtype=np.int64)) + window - 1)


def decode_bytes(w, window=0):
    """K + V of every visible key once per KV head, + Q + out of every query
    row + metadata."""
    kv = int(np.sum(visible_keys(w, window))) * w.num_kv_heads * w.head_dim * 2 * 2
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


def sub_batch(w, reqs):
    """The same attention call restricted to the requests ``reqs`` (the
    paged pool is shared, contiguous K/V rows are copied)."""
    from gqa_attention_sinks_amd import workloads as wl
    reqs = np.asarray(reqs, dtype=np.int64)
    qo = np.asarray(w.qo_indptr, dtype=np.int64)
    rows = np.concatenate([np.arange(qo[b], qo[b + 1]) for b in reqs]) if len(reqs) else np.zeros(0, np.int64)
    qo_len = qo[reqs + 1] - qo[reqs]
    new = wl.Workload(**{**w.__dict__})
    if "masks" in w.meta:
        new.meta = {**w.meta, "masks": [w.meta["masks"][b] for b in reqs]}
    new.q = w.q[rows]
    new.qo_indptr = np.concatenate([[0], np.cumsum(qo_len)]).astype(np.int32)
    new.kv_len = np.asarray(w.kv_len)[reqs].astype(np.int32)
    kvp = np.asarray(w.kv_indptr, dtype=np.int64)
    if w.paged:
        new.page_indices = np.concatenate([w.page_indices[kvp[b]:kvp[b + 1]] for b in reqs]).astype(np.int32)
        n_pages = kvp[reqs + 1] - kvp[reqs]
        new.kv_indptr = np.concatenate([[0], np.cumsum(n_pages)]).astype(np.int32)
    else:
        krows = np.concatenate([np.arange(kvp[b], kvp[b + 1]) for b in reqs])
        new.k, new.v = w.k[krows], w.v[krows]
        new.kv_indptr = np.concatenate([[0], np.cumsum(kvp[reqs + 1] - kvp[reqs])]).astype(np.int32)
    return new


def kv_head_group(w, g):
    """A contiguous workload restricted to KV head g and its query heads (a
    GQA group of one KV head)."""
    from gqa_attention_sinks_amd import workloads as wl
    G = w.num_qo_heads // w.num_kv_heads
    new = wl.Workload(**{**w.__dict__})
    new.q = np.ascontiguousarray(w.q[:, g * G:(g + 1) * G])
    new.k = np.ascontiguousarray(w.k[:, g:g + 1])
    new.v = np.ascontiguousarray(w.v[:, g:g + 1])
    new.sinks = w.sinks[g * G:(g + 1) * G].copy()
    new.num_qo_heads, new.num_kv_heads = G, 1
    return new


def balanced_groups(weights, n):
    """Split request indices into n groups of about equal total weight."""
    order = np.argsort(-np.asarray(weights, dtype=np.float64), kind="stable")
    load = np.zeros(n)
    groups = [[] for _ in range(n)]
    for b in order:
        i = int(np.argmin(load))
        groups[i].append(int(b))
        load[i] += weights[b]
    return [sorted(g) for g in groups if g]


def stats_ms(samples):
    a = np.asarray(samples, dtype=np.float64)
    return {"mean": round(float(a.mean()), 5), "median": round(float(np.median(a)), 5),
            "p10": round(float(np.percentile(a, 10)), 5), "p90": round(float(np.percentile(a, 90)), 5),
            "n": int(a.size)}


def roofline_entry(kernel, bound, work, ms, traffic=None):
    """Achieved rate of one kernel from its mean launch time."""
    if bound == "hbm":
        achieved, peak, unit = work / (ms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s"
    else:
        achieved, peak, unit = work / (ms * 1e-3) / 1e12, MFMA_PEAK_TFLOPS, "TFLOP/s"
    return {"bound": bound, "achieved": round(achieved, 1), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic, "kernel": kernel}


# ---------------------------------------------------------------------------
# the oracle on the host (cpu_baseline): a fork-based process pool, started
# before anything touches the GPU, each process running the unchanged oracle
# on a sub-batch with one BLAS thread
# ---------------------------------------------------------------------------

_JOBS = {}          # job id -> (workload, window, kind); inherited by the forked workers


def _limit_blas():
    from threadpoolctl import threadpool_limits
    threadpool_limits(limits=1)


def _oracle_job(key):
    import oracle
    w, window, kind = _JOBS[key]
    kv = (oracle.KVCache(k=w.k, v=w.v, kv_indptr=w.kv_indptr, paged=True, page_indices=w.page_indices,
                         kv_len=w.kv_len, page_size=w.page_size) if w.paged
          else oracle.KVCache(k=w.k, v=w.v, kv_indptr=w.kv_indptr))
    t0 = time.perf_counter()
    if kind == "split":
        o_part, lse_part = oracle.split_partials_ref(w.q, kv, w.sinks, w.scale, w.num_splits, window, workers=1)
        out, lse = oracle.merge_ref(o_part, lse_part)
    else:
        out, lse = oracle.sink_attention_ref(w.q, w.qo_indptr, kv, w.sinks, w.scale, window, workers=1,
                                             custom_mask=w.meta.get("masks"))
    return key, out.astype(np.float32), lse.astype(np.float32), time.perf_counter() - t0


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class OracleRuns:
    """Runs every workload's oracle sample on the host cores and keeps the
    outputs (fp32 copies of the fp64 results) for the parity summaries."""

    def __init__(self, cores):
        import multiprocessing as mp
        self.cores = cores
        self.ctx = mp.get_context("fork")
        self.results = {}
        self.baselines = {}

    def run(self, name, jobs, work, unit, sample, min_seconds=0.0):
        """jobs: list of (workload, window, kind, rows_or_None); the jobs run
        together on the pool (repeated until min_seconds have passed, the
        outputs kept from the first pass)."""
        _JOBS.clear()
        for i, (w, window, kind, _) in enumerate(jobs):
            _JOBS[i] = (w, window, kind)
        procs = min(self.cores, len(jobs))
        passes, wall = 0, 0.0
        with self.ctx.Pool(procs, initializer=_limit_blas) as pool:
            while passes == 0 or wall < min_seconds:
                t0 = time.perf_counter()
                res = pool.map(_oracle_job, range(len(jobs)), chunksize=1)
                wall += time.perf_counter() - t0
                if passes == 0:
                    self.results[name] = [(jobs[k][3], out, lse) for k, out, lse, _ in sorted(res, key=lambda r: r[0])]
                passes += 1
        rate = passes * work / wall / (1e12 if unit == "TFLOP/s" else 1e9)
        self.baselines[name] = {"value": float(f"{rate:.4g}"), "unit": unit, "cores": procs, "kind": "oracle",
                                "sample": f"{sample}; {passes} pass(es) in {wall:.1f} s on {procs} processes "
                                          f"(fp64 numpy, one BLAS thread each)",
                                "seconds": round(wall, 2)}
        log(f"oracle {name}: {self.baselines[name]['value']} {unit}, {wall:.1f} s")


def run_oracles(ws, cores):
    """The oracle samples of every workload (and the parity references)."""
    oc = OracleRuns(cores)
    # tiny prefill: the whole call (one (request, KV head) unit)
    w = ws["tiny_prefill"]
    oc.run("tiny_prefill", [(w, 0, "attn", np.asarray([0]))], prefill_flops(w), "GFLOP/s",
           "whole call (1 request x 1 KV head)", min_seconds=1.0)
    # paged decode: the whole batch in balanced sub-batches of requests
    w = ws["paged_decode"]
    groups = balanced_groups(w.kv_len, cores)
    jobs = [(sub_batch(w, g), 0, "attn", np.asarray(g)) for g in groups]
    oc.run("paged_decode", jobs, decode_bytes(w), "GB/s",
           f"whole workload ({w.batch} requests, {int(w.kv_len.sum())} keys) in {len(groups)} sub-batches",
           min_seconds=5.0)
    # causal prefill: every (request, KV head) unit
    w = ws["causal_prefill"]
    units = [(u // w.num_kv_heads, u % w.num_kv_heads) for u in range(w.batch * w.num_kv_heads)]
    jobs = []
    for b, g in units:
        jobs.append((kv_head_group(sub_batch(w, [b]), g), 0, "attn", (b, g)))
    flops = sum(prefill_flops(j[0]) for j in jobs)
    oc.run("causal_prefill", jobs, flops, "TFLOP/s",
           f"whole workload as its {len(units)} (request, KV head) units")
    # long split decode: each request's 16 chunk partials and their merge
    w = ws["long_split_decode"]
    jobs = [(sub_batch(w, [b]), 0, "split", np.asarray([b])) for b in range(w.batch)]
    oc.run("long_split_decode", jobs, decode_bytes(w), "GB/s",
           f"whole workload ({w.batch} requests x {int(w.kv_len[0])} keys, {w.num_splits} chunk partials "
           f"+ merge), one request per process")
    # skewed decode: the long request alone, the rest in balanced sub-batches
    w = ws["skewed_decode"]
    groups = [[0]] + [[b + 1 for b in g] for g in balanced_groups(w.kv_len[1:], max(1, cores - 1))]
    jobs = [(sub_batch(w, g), 0, "attn", np.asarray(g)) for g in groups]
    oc.run("skewed_decode", jobs, decode_bytes(w), "GB/s",
           f"whole workload ({w.batch} requests, {int(w.kv_len.sum())} keys) in {len(groups)} sub-batches")
    # verify (several rows per request), with and without draft-tree masks:
    # the whole batch in balanced sub-batches
    for name in ("verify_decode", "verify_tree"):
        if name not in ws:
            continue
        w = ws[name]
        groups = balanced_groups(np.asarray(w.kv_len) * np.diff(w.qo_indptr), cores)
        jobs = [(sub_batch(w, g), 0, "attn", np.asarray(g)) for g in groups]
        oc.run(name, jobs, decode_bytes(w), "GB/s",
               f"whole workload ({w.batch} requests, {int(w.qo_indptr[-1])} rows) in {len(groups)} sub-batches")
    # mixed batch, 128-key window: the whole call
    w = ws["mixed_batch"]
    n_pre = int(w.meta["n_prefill"])
    work = np.asarray(w.qo_len, dtype=np.float64) * np.minimum(np.asarray(w.kv_len), 128 + w.qo_len)
    groups = balanced_groups(work, cores)
    jobs = [(sub_batch(w, g), 128, "attn", np.asarray(g)) for g in groups]
    oc.run("mixed_batch_w128", jobs, prefill_flops(w, 128), "TFLOP/s",
           f"whole call ({w.batch} requests) in {len(groups)} sub-batches")
    # mixed batch, full causal: every prefill chunk on its own, the decode rows
    # in balanced sub-batches
    pre = list(range(n_pre))
    dec = list(range(n_pre, w.batch))
    dec_groups = balanced_groups(np.asarray(w.kv_len)[dec], max(1, cores - len(pre)))
    jobs = [(sub_batch(w, [b]), 0, "attn", np.asarray([b])) for b in pre]
    jobs += [(sub_batch(w, [dec[i] for i in g]), 0, "attn", np.asarray([dec[i] for i in g])) for g in dec_groups]
    sample_w = sub_batch(w, pre + dec)
    oc.run("mixed_batch_full", jobs, prefill_flops(sample_w), "TFLOP/s",
           f"whole call: the {len(pre)} prefill chunks one per job, the {len(dec)} decode rows in "
           f"{len(dec_groups)} sub-batches")
    return oc


def parity_summary(g, r, lse_g=None, lse_r=None, rows=None):
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    err = np.abs(g - r)
    big = np.abs(r) >= 1e-2
    res = {"rows": int(g.shape[0]), "elements": int(g.size), "max_abs": float(err.max()),
           "max_rel": float((err[big] / np.abs(r[big])).max()) if big.any() else 0.0,
           "within_tol": bool(np.all(err <= ATOL + RTOL * np.abs(r)) and np.isfinite(g).all())}
    if lse_g is not None:
        lg, lr = np.asarray(lse_g, np.float64), np.asarray(lse_r, np.float64)
        fin = np.isfinite(lr)
        res["lse_max_abs"] = float(np.abs(lg[fin] - lr[fin]).max()) if fin.any() else 0.0
        res["lse_inf_match"] = bool(np.array_equal(lg[~fin], lr[~fin]))
    return res


def parity_from_oracle(oc, name, w, out_host, lse_host):
    """Compare the GPU output rows that the oracle sample covers."""
    if oc is None or name not in oc.results:
        return None
    gs, rs, lgs, lrs = [], [], [], []
    qo = np.asarray(w.qo_indptr, dtype=np.int64)
    G = w.num_qo_heads // w.num_kv_heads
    for key, out, lse in oc.results[name]:
        if isinstance(key, tuple):                       # (request, KV head) unit
            b, g = key
            rows = np.arange(qo[b], qo[b + 1])
            heads = slice(g * G, (g + 1) * G)
            gs.append(out_host[rows][:, heads])
            lgs.append(lse_host[rows][:, heads] if lse_host is not None else None)
        else:                                            # whole requests
            rows = np.concatenate([np.arange(qo[b], qo[b + 1]) for b in key])
            gs.append(out_host[rows])
            lgs.append(lse_host[rows] if lse_host is not None else None)
        rs.append(out)
        lrs.append(lse)
    flat = lambda xs: np.concatenate([x.reshape(-1, x.shape[-1]) for x in xs])
    g, r = flat(gs), flat(rs)
    lse_ok = all(x is not None for x in lgs)
    lg = np.concatenate([x.reshape(-1) for x in lgs]) if lse_ok else None
    lr = np.concatenate([x.reshape(-1) for x in lrs]) if lse_ok else None
    return parity_summary(g, r, lg, lr)


# ---------------------------------------------------------------------------
# GPU runs
# ---------------------------------------------------------------------------

class Dev:
    """A workload's inputs in device memory."""

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


def launch_times(fn, n, stream, torch, group=10):
    """Per-launch times of n calls of fn issued back to back on ``stream``:
    the calls run in groups of ``group`` between two HIP events, and each
    group gives one sample (its time / group).  Events between single
    launches would add their own few microseconds to every sample; within a
    group the launches follow each other as in a serving loop, so the mean
    matches the kernel durations a profiler records (plus the short gaps
    between launches)."""
    groups = max(1, n // group)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * groups)]
    i = 0
    for gi in range(groups):
        ev[2 * gi].record(stream)
        for _ in range(group):
            fn(i)
            i += 1
        ev[2 * gi + 1].record(stream)
    torch.cuda.synchronize()
    return [ev[2 * gi].elapsed_time(ev[2 * gi + 1]) / group for gi in range(groups)]


def to_host(t):
    return t.float().cpu().numpy()


def time_decode(w, args, torch, dev, window=0, mode="balanced"):
    """Decode steps through the C ABI with prebuilt arguments (the Python
    binding's checks would otherwise cost more than a step).  ``mode``:
    "balanced" (sinkattn_decode_paged_balanced: the batch's live pages in
    equal segments, then the merge of the requests that cross segments) or
    "split" (sinkattn_decode_paged with the library's split count, then
    sinkattn_merge).  The step time is that of the K steps captured in one
    HIP graph and replayed (as a serving loop issues its decode steps); the
    same steps issued one by one from Python are timed beside it; then each
    of the two kernels is timed per launch.  The output returned is the
    graph replay's."""
    import ctypes
    import gqa_attention_sinks_amd as sa
    from gqa_attention_sinks_amd import binding
    lib = sa.load_library()
    base = Dev(w, torch, dev)
    reps = [base] + [base.replica() for _ in range(max(0, args.replicas - 1))]
    B, H, HKV = w.batch, w.num_qo_heads, w.num_kv_heads
    outs = [torch.empty_like(r.q) for r in reps]
    lses = [torch.empty((B, H), dtype=torch.float32, device=dev) for _ in reps]
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = ctypes.c_void_p
    host_len = None if args.no_host_order else w.kv_len
    kvs = [binding.kv_descriptor(r.k, r.v, r.kv_indptr, r.page_indices, r.kv_len, host_len) for r in reps]
    qp = [P(r.q.data_ptr()) for r in reps]
    sk = [P(r.sinks.data_ptr()) for r in reps]
    op = [P(o.data_ptr()) for o in outs]
    lp = [P(x.data_ptr()) for x in lses]
    scale = ctypes.c_float(w.scale)

    def check(st):
        if st != 0:
            raise RuntimeError(lib.sinkattn_last_error().decode())

    if mode == "balanced":
        s = args.segments if args.segments > 0 else sa.pick_num_segments(HKV)
        nbytes = sa.decode_balanced_workspace_bytes(B, H, s)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        wsp = P(ws.data_ptr())

        def decode_only(i, sp=sp):
            r = i % len(reps)
            check(lib.sinkattn_decode_paged_balanced_pieces(qp[r], ctypes.byref(kvs[r]), sk[r], s, wsp, nbytes, op[r],
                                                            lp[r], B, H, HKV, 64, scale, window, sp))

        def merge_only(i, sp=sp):
            r = i % len(reps)
            check(lib.sinkattn_merge_balanced(sk[r], s, wsp, nbytes, op[r], lp[r], B, H, 64, sp))

        def step(i, sp=sp):
            r = i % len(reps)
            check(lib.sinkattn_decode_paged_balanced(qp[r], ctypes.byref(kvs[r]), sk[r], s, wsp, nbytes, op[r], lp[r],
                                                     B, H, HKV, 64, scale, window, sp))
    else:
        s = args.splits if args.splits > 0 else (w.num_splits or sa.pick_num_splits(w.kv_len, w.num_kv_heads))
        o_part = torch.empty((B, H, s, 64), dtype=torch.float32, device=dev)
        lse_part = torch.empty((B, H, s), dtype=torch.float32, device=dev)
        opart, lpart = P(o_part.data_ptr()), P(lse_part.data_ptr())

        def decode_only(i, sp=sp):
            r = i % len(reps)
            if s > 1:
                check(lib.sinkattn_decode_paged(qp[r], ctypes.byref(kvs[r]), sk[r], s, None, opart, lpart, None,
                                                B, H, HKV, 64, scale, window, sp))
            else:
                check(lib.sinkattn_decode_paged(qp[r], ctypes.byref(kvs[r]), sk[r], 1, op[r], None, None, lp[r],
                                                B, H, HKV, 64, scale, window, sp))

        def merge_only(i, sp=sp):
            r = i % len(reps)
            check(lib.sinkattn_merge(opart, lpart, B, H, s, 64, op[r], lp[r], sp))

        def step(i, sp=sp):
            decode_only(i, sp)
            if s > 1:
                merge_only(i, sp)

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
    out_host, lse_host = to_host(outs[last]), to_host(lses[last])
    del graph
    n = max(args.steps, 200)
    dec = launch_times(decode_only, n, stream, torch)
    mer = launch_times(merge_only, n, stream, torch) if (mode == "balanced" or s > 1) else [0.0]
    torch.cuda.synchronize()
    return dict(step_ms=wall * 1e3, step_ms_eager=wall_eager * 1e3, decode=dec, merge=mer, splits=s, mode=mode,
                out=out_host, lse=lse_host)


def time_prefill(w, n, warmup, torch, dev, window=0, d=None, group=10, host_order=True):
    """sinkattn_prefill on a workload, each call between events; returns the
    per-call times and the output."""
    from gqa_attention_sinks_amd import binding
    d = d or Dev(w, torch, dev)
    out = torch.empty_like(d.q)
    lse = torch.empty((w.total_q, w.num_qo_heads), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    host = np.ascontiguousarray(w.qo_indptr, dtype=np.int32)

    def call(i=0):
        binding.prefill(d.q, d.qo_indptr, d.k, d.v, d.kv_indptr, d.sinks, w.scale, window=window,
                        page_indices=d.page_indices, kv_len=d.kv_len if w.paged else None, out=out, lse=lse,
                        qo_indptr_host=host, kv_len_host=w.kv_len if (w.paged and host_order) else None)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    times = launch_times(call, n, stream, torch, group=group)
    return dict(times=times, out=to_host(out), lse=to_host(lse))


def graph_call_ms(call, n, torch):
    """Per-call time of a few-microsecond call: n calls captured in one HIP
    graph and replayed (the host's launch rate does not enter)."""
    stream = torch.cuda.current_stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n):
            call()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


# The sources each kernel is built from: a traffic record (HBM bytes per
# launch from rocprofv3 FETCH_SIZE / WRITE_SIZE runs) holds their hash and is
# used only while it matches.
KERNEL_SOURCES = {
    "decode_paged_kernel": ("decode.hip", "decode_common.hpp"),
    "decode_balanced_kernel": ("decode_balanced.hip",),
    "prefill_kernel": ("prefill.hip", "mfma_tile.hpp"),
    "verify_kernel": ("verify.hip", "decode_common.hpp", "mfma_tile.hpp"),
}


def kernel_source_hash(kernel):
    import hashlib
    csrc = os.path.join(ROOT, "gqa_attention_sinks_amd", "csrc")
    files = [os.path.join(csrc, f) for f in (*KERNEL_SOURCES[kernel], "device_common.hpp", "kernel_args.hpp")]
    return hashlib.sha256(b"".join(open(f, "rb").read() for f in files)).hexdigest()


def measured_traffic(kernel, workload, splits=None):
    """HBM bytes per launch of ``kernel`` on ``workload`` from the committed
    FETCH_SIZE/WRITE_SIZE runs (profiles/traffic.json), or None when there is
    no record or the kernel's sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path) or kernel not in KERNEL_SOURCES:
        return None
    rec = json.load(open(path)).get(f"{kernel}@{workload}")
    if not rec or rec.get("source_sha256") != kernel_source_hash(kernel) or \
            (splits is not None and rec.get("num_splits") != splits):
        return None
    return int(round(rec["bytes"]))


# ---------------------------------------------------------------------------
# per-workload GPU legs
# ---------------------------------------------------------------------------

DESCR = {
    "tiny_prefill": "tiny prefill: batch 1, 4 query / 1 KV head, head_dim 64, causal 128, contiguous KV, "
                    "sinks N(0, 1), seed 0",
    "paged_decode": "paged decode: batch 64, one query token each, KV lengths uniform in [1, 4096], 64 query / "
                    "8 KV heads, head_dim 64, page size 16, pages permuted in a shared pool, sinks N(0, 2), seed 0",
    "causal_prefill": "causal prefill: batch 4 x 8192 tokens, 64 query / 8 KV heads, head_dim 64, contiguous KV, "
                      "scale 1/8, sinks N(0, 2), full causal, seed 0",
    "long_split_decode": "long split decode: batch 8, 131072 keys each, 64 query / 8 KV heads, paged (page 16), "
                         "16 chunks with the sink in chunk 0 only, then the LSE merge; sinks N(0, 2) with -inf "
                         "and +20 outliers, seed 0",
    "skewed_decode": "skewed decode (beyond the five workloads): batch 64, request 0 with 131072 keys, the others "
                     "uniform in [1, 4096], 64 query / 8 KV heads, paged (page 16), sinks N(0, 2), seed 0",
    "mixed_batch": "mixed batch: 16 prefill chunks of 512 tokens on prefixes uniform in [0, 16384] + 240 decode "
                   "rows with KV lengths uniform in [1, 16384] in one call, 64 query / 8 KV heads, paged "
                   "(page 16), sinks N(0, 2), seed 0",
    "verify_decode": "verify decode (NEXT row): batch 64, KV lengths uniform in [8, 4096], query rows per request "
                     "uniform in [2, 8], 64 query / 8 KV heads, paged (page 16), sinks N(0, 2), seed 0",
    "verify_tree": "draft-tree verify (NEXT row): the verify batch with a random draft tree (custom mask) per "
                   "request, seed 0",
    "append_rope": "paged KV append with rotary embedding (NEXT row): 16 chunks of 512 new tokens on prefixes "
                   "uniform in [0, 16384], 64 query / 8 KV heads, random pages, seed 0",
    "moe_topk": "MoE routing weights (NEXT row): 65536 tokens x 128 experts of bf16 logits N(0, 1), top 4, seed 0",
}


def leg_tiny(w, args, torch, dev, oc):
    import gqa_attention_sinks_amd as sa
    d = Dev(w, torch, dev)
    r = time_prefill(w, max(args.steps, 200), args.warmup, torch, dev, d=d)
    out = torch.empty_like(d.q)
    host = np.ascontiguousarray(w.qo_indptr, dtype=np.int32)
    graph_ms = graph_call_ms(lambda: sa.prefill(d.q, d.qo_indptr, d.k, d.v, d.kv_indptr, d.sinks, w.scale,
                                                 out=out, qo_indptr_host=host), 100, torch)
    flops = prefill_flops(w)
    st = stats_ms(r["times"])
    return {"workload": DESCR["tiny_prefill"], "bound": "latency (launch)",
            "kernels": {"prefill_kernel": {"ms": st, "algorithmic_flops": flops,
                                           "roofline": roofline_entry("prefill_kernel", "mfma", flops, st["mean"],
                                                                      measured_traffic("prefill_kernel", "tiny_prefill"))}},
            "call_ms_graph_replay": round(graph_ms, 5),
            "parity": parity_from_oracle(oc, "tiny_prefill", w, r["out"], r["lse"]),
            "cpu_baseline": oc.baselines.get("tiny_prefill") if oc else None}


def leg_causal_prefill(w, args, torch, dev, oc):
    r = time_prefill(w, 40, 3, torch, dev, group=2)
    flops = prefill_flops(w)
    st = stats_ms(r["times"])
    return {"workload": DESCR["causal_prefill"], "bound": "mfma",
            "kernels": {"prefill_kernel": {"ms": st, "algorithmic_flops": flops,
                                           "roofline": roofline_entry("prefill_kernel", "mfma", flops, st["mean"],
                                                                      measured_traffic("prefill_kernel", "causal_prefill"))}},
            "parity": parity_from_oracle(oc, "causal_prefill", w, r["out"], r["lse"]),
            "cpu_baseline": oc.baselines.get("causal_prefill") if oc else None}


def leg_decode(name, w, args, torch, dev, oc, mode):
    res = time_decode(w, args, torch, dev, mode=mode)
    nbytes = decode_bytes(w)
    dst, mst = stats_ms(res["decode"]), stats_ms(res["merge"])
    kname = "decode_balanced_kernel" if mode == "balanced" else "decode_paged_kernel"
    kernels = {kname: {"ms": dst, "algorithmic_bytes": nbytes,
                       "roofline": roofline_entry(kname, "hbm", nbytes, dst["mean"],
                                                  measured_traffic(kname, name, res["splits"]))}}
    if mode == "balanced":
        kernels["merge_balanced_kernel"] = {"ms": mst}
    elif res["splits"] > 1:
        part = 2 * w.batch * w.num_qo_heads * res["splits"] * (w.head_dim + 1) * 4
        kernels["merge_kernel"] = {"ms": mst, "partials_bytes": part}
    entry = {"workload": DESCR[name], "bound": "hbm", "decode_path": mode,
             ("num_segments" if mode == "balanced" else "num_splits"): res["splits"],
             "step_ms_graph": round(res["step_ms"], 5), "step_ms_eager": round(res["step_ms_eager"], 5),
             "step_GBs": round(nbytes / (res["step_ms"] * 1e-3) / 1e9, 1),
             "kernels": kernels,
             "parity": parity_from_oracle(oc, name, w, res["out"], res["lse"]),
             "cpu_baseline": oc.baselines.get(name) if oc else None}
    return entry, res


def leg_mixed(w, window, args, torch, dev, oc):
    """The mixed batch under one window: the whole call (prefill kernel, then
    the decode kernel for the single-row requests), and each part alone as
    its own call over the same pool (the prefill requests through
    sinkattn_prefill, the decode rows through sinkattn_decode_paged)."""
    import ctypes
    import gqa_attention_sinks_amd as sa
    from gqa_attention_sinks_amd import binding
    name = "mixed_batch_w128" if window else "mixed_batch_full"
    n_pre = int(w.meta["n_prefill"])
    d = Dev(w, torch, dev)
    n, group = (40, 2) if window == 0 else (200, 10)
    ho = not args.no_host_order
    whole = time_prefill(w, n, 3, torch, dev, window=window, d=d, group=group, host_order=ho)
    pre_w = sub_batch(w, range(n_pre))
    dp = Dev.__new__(Dev)
    dp.__dict__ = dict(d.__dict__)
    dp.q = d.q[:int(w.qo_indptr[n_pre])]
    dp.qo_indptr = d.qo_indptr[:n_pre + 1]
    dp.kv_indptr = d.kv_indptr[:n_pre + 1]
    dp.kv_len = d.kv_len[:n_pre]
    pre = time_prefill(pre_w, n, 3, torch, dev, window=window, d=dp, group=group, host_order=ho)
    # decode rows: request b >= n_pre owns row qo_indptr[b] = d0 + (b - n_pre)
    d0 = int(w.qo_indptr[n_pre])
    dec_w = sub_batch(w, range(n_pre, w.batch))
    q_dec = d.q[d0:]
    out_dec = torch.empty_like(q_dec)
    kv = binding.kv_descriptor(d.k, d.v, d.kv_indptr[n_pre:], d.page_indices, d.kv_len[n_pre:],
                               w.kv_len[n_pre:] if ho else None)
    lib = sa.load_library()
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = ctypes.c_void_p
    nd = w.batch - n_pre

    def dec_call(i=0):
        st = lib.sinkattn_decode_paged(P(q_dec.data_ptr()), ctypes.byref(kv), P(d.sinks.data_ptr()), 1,
                                       P(out_dec.data_ptr()), None, None, None, nd, w.num_qo_heads,
                                       w.num_kv_heads, 64, ctypes.c_float(w.scale), window, sp)
        if st != 0:
            raise RuntimeError(lib.sinkattn_last_error().decode())

    for _ in range(3):
        dec_call()
    dec_t = launch_times(dec_call, n, stream, torch, group=group)
    torch.cuda.synchronize()
    same = bool(np.array_equal(to_host(out_dec), whole["out"][d0:]))
    flops = prefill_flops(pre_w, window)
    nbytes = decode_bytes(dec_w, window)
    wst, pst, dst = stats_ms(whole["times"]), stats_ms(pre["times"]), stats_ms(dec_t)
    bound_ms = flops / (MFMA_PEAK_TFLOPS * 1e12) * 1e3 + nbytes / (HBM_PEAK_GBS * 1e9) * 1e3
    return {"workload": DESCR["mixed_batch"] + f"; window {window or 'none (full causal)'}",
            "bound": "mfma (prefill part) + hbm (decode part)" if window == 0 else "latency",
            "call_ms": wst,
            "sum_of_roofline_ms": round(bound_ms, 5),
            "call_frac_of_sum_bound": round(bound_ms / wst["mean"], 4),
            "kernels": {
                "prefill_kernel": {"ms": pst, "algorithmic_flops": flops, "rows": d0,
                                   "roofline": roofline_entry("prefill_kernel", "mfma", flops, pst["mean"],
                                                              measured_traffic("prefill_kernel", name))},
                "decode_paged_kernel": {"ms": dst, "algorithmic_bytes": nbytes, "rows": nd,
                                        "roofline": roofline_entry("decode_paged_kernel", "hbm", nbytes,
                                                                   dst["mean"],
                                                                   measured_traffic("decode_paged_kernel", name))}},
            "decode_rows_alone_equal_whole_call": same,
            "parity": parity_from_oracle(oc, name, w, whole["out"], whole["lse"]),
            "cpu_baseline": oc.baselines.get(name) if oc else None}


def leg_verify(name, w, args, torch, dev, oc):
    """Several query rows per request (sinkattn_decode_paged_multi), with or
    without draft-tree masks: the decode kernel per launch (replicas
    rotated), the whole call (decode + merge) by wall clock, parity of one
    whole call against the oracle."""
    res = time_verify(w, args, torch, dev)
    nbytes = decode_bytes(w)
    return {"workload": DESCR[name], "bound": "hbm", "num_splits": res["splits"],
            "rows": int(w.qo_indptr[-1]), "step_ms_wall": round(res["step_ms"], 5),
            "kernels": {"verify_kernel": {"ms": res["decode"], "algorithmic_bytes": nbytes,
                                          "roofline": roofline_entry("verify_kernel", "hbm", nbytes,
                                                                     res["decode"]["mean"],
                                                                     measured_traffic("verify_kernel", name,
                                                                                      res["splits"]))}},
            "parity": parity_from_oracle(oc, name, w, res["out"], res["lse"]),
            "cpu_baseline": oc.baselines.get(name) if oc else None}


def leg_bytes(name, r):
    """A bandwidth-bound NEXT-row kernel timed by graph replay (its parity
    against the oracle is covered by the GPU tests)."""
    return {"workload": DESCR[name], "bound": "hbm", "ms_per_call_graph": round(r["ms"], 5),
            "kernels": {name: {"ms": {"mean": round(r["ms"], 5)}, "algorithmic_bytes": r["bytes"],
                               "roofline": roofline_entry(name, "hbm", r["bytes"], r["ms"])}},
            "parity": None}


# ---------------------------------------------------------------------------
# main
# ---------------------------------------------------------------------------

def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); sharding the path over several "
              "GPUs is not built", file=sys.stderr)
        sys.exit(2)
    if args.workload is not None:
        return profile_only(args)
    from gqa_attention_sinks_amd import workloads as wl
    t_start = time.perf_counter()
    log("generating workloads")
    ws = {n: getattr(wl, n)() for n in ["tiny_prefill", "paged_decode", "causal_prefill", "long_split_decode",
                                         "mixed_batch", "skewed_decode", "verify_decode", "verify_tree"]}
    cores = len(os.sched_getaffinity(0))
    oc = None
    if not args.no_cpu:
        log(f"oracle on {cores} host cores ({cpu_model()})")
        oc = run_oracles(ws, cores)       # before the GPU is touched: the pool forks
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import gqa_attention_sinks_amd as sa
    if not os.path.exists(sa.library_path()):
        import __graft_entry__
        __graft_entry__.build()
    sa.load_library()
    dev = torch.device("cuda:0")

    configs = {}
    other = "split" if args.decode == "balanced" else "balanced"
    log(f"paged_decode ({args.decode}, then {other})")
    head, res = leg_decode("paged_decode", ws["paged_decode"], args, torch, dev, oc, args.decode)
    configs["paged_decode"] = head
    configs[f"paged_decode_{other}"], _ = leg_decode("paged_decode", ws["paged_decode"], args, torch, dev, oc, other)
    torch.cuda.empty_cache()
    log("tiny_prefill")
    configs["tiny_prefill"] = leg_tiny(ws["tiny_prefill"], args, torch, dev, oc)
    log("causal_prefill")
    configs["causal_prefill"] = leg_causal_prefill(ws["causal_prefill"], args, torch, dev, oc)
    torch.cuda.empty_cache()
    log("long_split_decode")
    configs["long_split_decode"], _ = leg_decode("long_split_decode", ws["long_split_decode"], args, torch,
                                                 dev, oc, "split")
    configs["long_split_decode_balanced"], _ = leg_decode("long_split_decode", ws["long_split_decode"], args,
                                                          torch, dev, oc, "balanced")
    torch.cuda.empty_cache()
    log("skewed_decode")
    configs["skewed_decode_balanced"], _ = leg_decode("skewed_decode", ws["skewed_decode"], args, torch, dev, oc,
                                                      "balanced")
    configs["skewed_decode_split"], _ = leg_decode("skewed_decode", ws["skewed_decode"], args, torch, dev, oc,
                                                   "split")
    torch.cuda.empty_cache()
    for name in ("verify_decode", "verify_tree"):
        log(name)
        configs[name] = leg_verify(name, ws[name], args, torch, dev, oc)
    log("append_rope, moe_topk")
    configs["append_rope"] = leg_bytes("append_rope", time_append(args, torch, dev))
    configs["moe_topk"] = leg_bytes("moe_topk", time_moe(args, torch, dev))
    torch.cuda.empty_cache()
    for window in (128, 0):
        log(f"mixed_batch window={window}")
        configs["mixed_batch_w128" if window else "mixed_batch_full"] = leg_mixed(ws["mixed_batch"], window,
                                                                                  args, torch, dev, oc)
        torch.cuda.empty_cache()

    w = ws["paged_decode"]
    nbytes = decode_bytes(w)
    value = nbytes / (res["step_ms"] * 1e-3) / 1e9
    kname = "decode_balanced_kernel" if args.decode == "balanced" else "decode_paged_kernel"
    mname = "merge_balanced_kernel" if args.decode == "balanced" else "merge_kernel"
    dmean = head["kernels"][kname]["ms"]["mean"]
    roof = roofline_entry(kname, "hbm", nbytes, dmean,
                          measured_traffic(kname, "paged_decode", res["splits"]))
    pre = configs["causal_prefill"]["kernels"]["prefill_kernel"]
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
            "workload": DESCR["paged_decode"],
            "decode_path": args.decode,
            ("num_segments" if args.decode == "balanced" else "num_splits"): res["splits"],
            "work_order": "longest request first, "
                          + ("ranked by the kernel" if args.no_host_order else "ordered on the host"),
            "kv_replicas_rotated": args.replicas,
            "algorithmic_bytes": nbytes,
            "compute": "bf16 Q.K^T and fp16 P.V on MFMA, fp32 accumulation",
            "step": "K steps (decode + merge launches) captured in one HIP graph, replayed",
            "ms_per_step_eager": round(res["step_ms_eager"], 5),
            "decode_kernel_ms": head["kernels"][kname]["ms"],
            "merge_kernel_ms": head["kernels"].get(mname, {}).get("ms"),
            "pct_hbm_peak_step": round(100 * value / HBM_PEAK_GBS, 2),
        },
        "roofline": roof,
        "prefill": {
            "workload": DESCR["causal_prefill"],
            "value": pre["roofline"]["achieved"],
            "unit": "TFLOP/s",
            "ms_per_call": pre["ms"]["mean"],
            "algorithmic_flops": pre["algorithmic_flops"],
            "roofline": pre["roofline"],
        },
        "configs": configs,
    }
    if oc is not None:
        cb = dict(oc.baselines["paged_decode"])
        cb.pop("seconds", None)
        cb["cpu_model"] = cpu_model()
        cb["configs"] = {k: v for k, v in oc.baselines.items()}
        line["cpu_baseline"] = cb
        line["parity"] = head["parity"]
        line["parity_all_within_tol"] = all(c["parity"]["within_tol"] for c in configs.values() if c.get("parity"))
    line["bench_seconds"] = round(time.perf_counter() - t_start, 1)
    print(json.dumps(line), flush=True)


# ---------------------------------------------------------------------------
# one workload only (for rocprofv3 runs)
# ---------------------------------------------------------------------------

def time_verify(w, args, torch, dev):
    """Several query rows per request (sinkattn_decode_paged_multi): the
    decode kernel alone per launch, replicas rotated, and the whole step
    (decode + merge) by wall clock."""
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
    host_len = None if args.no_host_order else w.kv_len
    kvs = [binding.kv_descriptor(r.k, r.v, r.kv_indptr, r.page_indices, r.kv_len, host_len) for r in reps]
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
    dec = launch_times(lambda i: call(i, False), max(args.steps, 100), stream, torch)
    # one whole call (decode + merge) on replica 0 with its LSE, for parity
    r0 = reps[0]
    out0 = torch.empty_like(r0.q)
    lse0 = torch.empty((TQ, H), dtype=torch.float32, device=dev)
    st = lib.sinkattn_decode_paged_multi(P(r0.q.data_ptr()), P(r0.qo_indptr.data_ptr()), mask, mask_ptr,
                                         ctypes.byref(kvs[0]), P(r0.sinks.data_ptr()), s, P(out0.data_ptr()),
                                         opart if s > 1 else None, lpart if s > 1 else None, P(lse0.data_ptr()),
                                         B, TQ, R, H, HKV, 64, scale, 0, sp)
    if st != 0:
        raise RuntimeError(lib.sinkattn_last_error().decode())
    torch.cuda.synchronize()
    return dict(step_ms=wall * 1e3, decode=stats_ms(dec), splits=s, out=to_host(out0), lse=to_host(lse0))


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
    call = lambda: sa.append_paged_kv_rope(*args_, q=q, q_out=q_out)
    for _ in range(args.warmup):
        call()
    ms = graph_call_ms(call, args.steps, torch)
    nbytes = t * (2 * hq * 128 + 4 * hkv * 128 + 256) + 4 * (len(page_indices) + 3 * 17)
    return dict(tokens=t, ms=ms, bytes=nbytes, GBs=nbytes / (ms * 1e-3) / 1e9)


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
    call = lambda: sa.moe_topk_softmax(logits, k, idx, w)
    for _ in range(args.warmup):
        call()
    ms = graph_call_ms(call, args.steps, torch)
    nbytes = t * (e * 2 + k * 6)
    return dict(tokens=t, experts=e, top_k=k, ms=ms, bytes=nbytes, GBs=nbytes / (ms * 1e-3) / 1e9)


def profile_only(args):
    """Time one named workload only (for rocprofv3 runs)."""
    import torch
    import gqa_attention_sinks_amd as sa
    from gqa_attention_sinks_amd import workloads as wl
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    sa.load_library()
    dev = torch.device("cuda:0")
    name = args.workload
    if name == "copy_calibration":
        n = 256 << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / args.steps
        print(json.dumps({"workload": name, "bytes_read": n, "bytes_written": n, "ms": dt * 1e3,
                          "GBs_rw": 2 * n / dt / 1e9}))
        return
    if name == "moe_topk":
        r = time_moe(args, torch, dev)
        print(json.dumps({"workload": name, **r, "frac": r["GBs"] / HBM_PEAK_GBS}))
        return
    if name == "append_rope":
        r = time_append(args, torch, dev)
        print(json.dumps({"workload": name, **r, "frac": r["GBs"] / HBM_PEAK_GBS}))
        return
    w = getattr(wl, name)()
    log(f"timing {name}")
    if name in ("verify_decode", "verify_tree"):
        res = time_verify(w, args, torch, dev)
        gbs = decode_bytes(w) / (res["decode"]["mean"] * 1e-3) / 1e9
        print(json.dumps({"workload": name, "rows": int(w.qo_indptr[-1]), "splits": res["splits"],
                          "step_ms": res["step_ms"], "decode_ms": res["decode"], "decode_GBs": gbs,
                          "frac": gbs / HBM_PEAK_GBS}))
        return
    if name in ("paged_decode", "long_split_decode", "skewed_decode"):
        entry, _ = leg_decode(name, w, args, torch, dev, None, args.decode)
        print(json.dumps({"workload": name, **entry}))
        return
    if name == "tiny_prefill":
        print(json.dumps({"workload": name, **leg_tiny(w, args, torch, dev, None)}))
        return
    if name == "causal_prefill":
        print(json.dumps({"workload": name, **leg_causal_prefill(w, args, torch, dev, None)}))
        return
    for window in w.windows:                   # mixed_batch
        print(json.dumps({"workload": name, "window": window, **leg_mixed(w, window, args, torch, dev, None)}))


if __name__ == "__main__":
    main()
