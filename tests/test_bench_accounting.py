"""The benchmark's algorithmic work, against brute-force counts (CPU only).

The roofline figures divide these counts by measured kernel times, so they
are pinned here independently of the formulas in bench.py:
  * decode bytes: every live key's K and V row once per KV head (head_dim
    bf16 values each), every query row's Q and output (bf16), and the int32
    page ids plus the two per-request metadata arrays;
  * prefill flops: 4 * head_dim per visible (query, key, head), where row t of
    a request with n_q rows over n_k keys sits at n_k - n_q + t and sees the
    keys at or before it (and, with a window W, its last W positions).
"""

import subprocess
import sys

import numpy as np

import bench
from gqa_attention_sinks_amd import workloads as wl


def _decode_bytes_brute(w, window=0):
    total = 0
    for b in range(w.batch):
        n_q, n_k = int(w.qo_len[b]), int(w.kv_len[b])
        for key in range(n_k):
            # the key counts when some query row of the request sees it
            seen = any(key <= n_k - n_q + t and (window == 0 or key > n_k - n_q + t - window) for t in range(n_q))
            if not seen:
                continue
            for _g in range(w.num_kv_heads):
                total += 2 * w.head_dim * 2          # one K row and one V row, bf16
    rows = int(w.qo_indptr[-1])
    total += rows * w.num_qo_heads * w.head_dim * 2   # Q
    total += rows * w.num_qo_heads * w.head_dim * 2   # output
    total += 4 * len(w.page_indices)                  # page ids
    total += 4 * (w.batch + 1) + 4 * w.batch          # page offsets and KV lengths
    return total


def _prefill_flops_brute(w, window):
    visible = 0
    for b in range(w.batch):
        n_q, n_k = int(w.qo_len[b]), int(w.kv_len[b])
        for t in range(n_q):
            pos = n_k - n_q + t
            for j in range(n_k):
                if j <= pos and (window == 0 or j > pos - window):
                    visible += 1
    return 4 * w.head_dim * visible * w.num_qo_heads


def test_decode_bytes_small_batch():
    w = wl.paged_decode(seed=4, batch=5, max_len=300, num_qo_heads=8, num_kv_heads=2)
    assert bench.decode_bytes(w) == _decode_bytes_brute(w)


def test_decode_bytes_several_rows():
    w = wl.verify_decode(seed=2, batch=4, max_len=200, num_qo_heads=16, num_kv_heads=2)
    assert bench.decode_bytes(w) == _decode_bytes_brute(w)


def test_decode_bytes_under_a_window():
    w = wl.verify_decode(seed=3, batch=5, max_len=300, num_qo_heads=16, num_kv_heads=2)
    for window in (1, 7, 128, 1000):
        assert bench.decode_bytes(w, window) == _decode_bytes_brute(w, window), window


def test_headline_decode_bytes():
    """The figure the profiles and the benchmark line quote."""
    assert bench.decode_bytes(wl.paged_decode()) == 274_846_980


def test_prefill_flops_causal_and_window():
    w = wl.make_contiguous("acct", [70, 33, 5], [70, 20, 5], 8, 2, rng=np.random.default_rng(3))
    for window in (0, 1, 16, 128):
        assert bench.prefill_flops(w, window) == _prefill_flops_brute(w, window), window


def test_headline_prefill_flops():
    """4 x 8192 causal rows, 64 heads: 4 * 64 * 64 * 4 * (8192 * 8193 / 2)."""
    assert bench.prefill_flops(wl.causal_prefill()) == 4 * 64 * 64 * 4 * (8192 * 8193 // 2)


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr


def test_host_order_flag():
    """The headline's decode calls pass the host copy of kv_len unless the
    flag asks for the kernels' own ordering."""
    argv = sys.argv
    try:
        sys.argv = ["bench.py"]
        assert bench.parse().no_host_order is False
        sys.argv = ["bench.py", "--no-host-order"]
        assert bench.parse().no_host_order is True
    finally:
        sys.argv = argv


def test_oracle_legs_cover_the_rows_they_claim():
    """The benchmark's oracle samples (sub-batches, (request, KV head)
    units, split partials) reproduce the oracle's whole-call results on the
    rows they cover: the parity summaries compare like with like."""
    import oracle
    ws = {
        "tiny_prefill": wl.tiny_prefill(),
        "paged_decode": wl.paged_decode(batch=6, max_len=200),
        "causal_prefill": wl.causal_prefill(batch=2, seq=96, num_qo_heads=8, num_kv_heads=2),
        "long_split_decode": wl.long_split_decode(batch=2, kv_len=700, num_splits=4, num_qo_heads=16,
                                                  num_kv_heads=2),
        "mixed_batch": wl.mixed_batch(n_prefill=3, chunk=40, max_prefix=100, n_decode=5, max_decode_len=300,
                                      num_qo_heads=8, num_kv_heads=2),
        "skewed_decode": wl.skewed_decode(batch=5, long_len=900, max_len=100, num_qo_heads=8, num_kv_heads=2),
    }
    oc = bench.run_oracles(ws, 3)
    assert set(oc.baselines) == {"tiny_prefill", "paged_decode", "causal_prefill", "long_split_decode",
                                 "mixed_batch_w128", "mixed_batch_full", "skewed_decode"}
    for name, b in oc.baselines.items():
        assert b["kind"] == "oracle" and b["value"] > 0 and 1 <= b["cores"] <= 3, name

    def whole(w, window):
        kv = (oracle.KVCache(k=w.k, v=w.v, kv_indptr=w.kv_indptr, paged=True, page_indices=w.page_indices,
                             kv_len=w.kv_len) if w.paged else oracle.KVCache(k=w.k, v=w.v, kv_indptr=w.kv_indptr))
        return oracle.sink_attention_ref(w.q, w.qo_indptr, kv, w.sinks, w.scale, window)

    for name, key, window in [("tiny_prefill", "tiny_prefill", 0), ("paged_decode", "paged_decode", 0),
                              ("causal_prefill", "causal_prefill", 0), ("long_split_decode", "long_split_decode", 0),
                              ("mixed_batch_w128", "mixed_batch", 128), ("mixed_batch_full", "mixed_batch", 0),
                              ("skewed_decode", "skewed_decode", 0)]:
        w = ws[key]
        out, lse = whole(w, window)
        # the oracle's own results pass through the parity summary exactly
        p = bench.parity_from_oracle(oc, name, w, out.astype(np.float32), lse.astype(np.float32))
        assert p["within_tol"] and p["max_abs"] == 0.0 and p["lse_max_abs"] == 0.0, (name, p)
        assert p["rows"] > 0
    # the causal-prefill sample is every (request, KV head) unit
    assert [k for k, _, _ in oc.results["causal_prefill"]] == [(0, 0), (0, 1), (1, 0), (1, 1)]
