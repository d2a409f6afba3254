"""Randomised parity sweep: many small seeded batches, each drawn with its own
shape -- head counts and GQA group, request count, key and query-row
counts, window, paged or contiguous KV, split count, with or without the
optional host copies -- compared element by element (and every LSE) with
the fp64 oracle.  The fixed cases elsewhere pin the edges one at a time;
this sweep checks that their combinations hold too.

What is being checked (Perplexity blog "GPT-OSS on day 0", section "Kernels
for GPT-OSS > Sink attention"): one sink logit per head in the softmax
denominator, the streaming softmax seeded with it, and under a KV split the
sink in the first chunk only.
"""

import numpy as np
import pytest

from gqa_attention_sinks_amd import workloads as wl
from tests._gpu import DeviceWorkload, assert_parity, oracle_full, say, to_host

pytestmark = pytest.mark.gpu

HEADS = [(8, 8), (12, 3), (16, 2), (8, 1), (32, 2), (64, 8)]   # GQA groups 1, 4, 8, 8, 16, 8
WINDOWS = [0, 0, 1, 17, 64, 100, 128, 129, 300, 5000]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_attention_sinks_amd as sa
    sa.load_library()


def _draw(seed, max_rows, paged=True, max_batch=8, max_keys=700, max_columns=None):
    rng = np.random.default_rng(seed)
    hq, hkv = HEADS[rng.integers(len(HEADS))]
    if max_columns is not None:   # G x rows <= max_columns a request
        max_rows = min(max_rows, max_columns // (hq // hkv))
    batch = int(rng.integers(1, max_batch + 1))
    kv_len = rng.integers(1, max_keys + 1, size=batch)
    qo_len = np.minimum(rng.integers(1, max_rows + 1, size=batch), kv_len)
    window = int(WINDOWS[rng.integers(len(WINDOWS))])
    outliers = rng.random() < 0.3   # some sinks -inf and +20
    if paged:
        w = wl.make_paged(f"random{seed}", kv_len, qo_len, hq, hkv, rng=rng)
    else:
        w = wl.make_contiguous(f"random{seed}", kv_len, qo_len, hq, hkv, rng=rng)
    if outliers:
        w.sinks = wl.outlier_sinks(w.sinks)
    return w, window, rng


@pytest.mark.parametrize("seed", range(24))
def test_random_prefill(seed):
    rng0 = np.random.default_rng(1000 + seed)
    paged = bool(rng0.integers(2))
    w, window, rng = _draw(1000 + seed, max_rows=400, paged=paged)
    host_plan = bool(rng.integers(2))
    kv_len_host = w.kv_len if (paged and rng.integers(2)) else None
    say(f"random prefill seed={seed}: B={w.batch} H={w.num_qo_heads}/{w.num_kv_heads} paged={paged} W={window} "
        f"qo={list(np.diff(w.qo_indptr))} kv={list(w.kv_len)} plan={host_plan} kv_host={kv_len_host is not None}")
    out, lse = DeviceWorkload(w).prefill(window=window, host_plan=host_plan, kv_len_host=kv_len_host)
    ro, rl = oracle_full(w, window)
    assert_parity(to_host(out), ro, f"random prefill {seed}", to_host(lse), rl)


@pytest.mark.parametrize("seed", range(16))
def test_random_decode(seed):
    w, window, rng = _draw(2000 + seed, max_rows=1, max_batch=40, max_keys=3000)
    splits = int(rng.integers(1, 9))
    kv_len_host = w.kv_len if rng.integers(2) else None
    say(f"random decode seed={seed}: B={w.batch} H={w.num_qo_heads}/{w.num_kv_heads} W={window} S={splits} "
        f"kv_host={kv_len_host is not None}")
    out, lse = DeviceWorkload(w).decode(splits, window=window, kv_len_host=kv_len_host)
    ro, rl = oracle_full(w, window)
    assert_parity(to_host(out), ro, f"random decode {seed}", to_host(lse), rl)


@pytest.mark.parametrize("seed", range(12))
def test_random_verify(seed):
    w, window, rng = _draw(3000 + seed, max_rows=8, max_batch=16, max_keys=2000, max_columns=64)
    splits = int(rng.integers(1, 4))
    kv_len_host = w.kv_len if rng.integers(2) else None
    say(f"random verify seed={seed}: B={w.batch} H={w.num_qo_heads}/{w.num_kv_heads} W={window} S={splits} "
        f"qo={list(np.diff(w.qo_indptr))}")
    max_rows = min(8, 64 // (w.num_qo_heads // w.num_kv_heads))
    out, lse = DeviceWorkload(w).decode_multi(splits, max_rows, window=window, kv_len_host=kv_len_host)
    ro, rl = oracle_full(w, window)
    assert_parity(to_host(out), ro, f"random verify {seed}", to_host(lse), rl)


@pytest.mark.parametrize("seed", range(8))
def test_random_balanced_decode(seed):
    import torch
    import gqa_attention_sinks_amd as sa
    w, window, rng = _draw(4000 + seed, max_rows=1, max_batch=40, max_keys=3000)
    n = int(rng.choice([1, 7, 48, 192]))
    d = DeviceWorkload(w)
    ws = torch.full((sa.decode_balanced_workspace_bytes(w.batch, w.num_qo_heads, n),), 0xFF, dtype=torch.uint8,
                    device=d.q.device)                  # NaN-filled: a partial that is not written shows
    say(f"random balanced decode seed={seed}: B={w.batch} H={w.num_qo_heads}/{w.num_kv_heads} W={window} N={n}")
    out, lse = sa.decode_paged_balanced(d.q, d.k, d.v, d.kv_indptr, d.page_indices, d.kv_len, d.sinks, w.scale,
                                        num_segments=n, window=window, workspace=ws, return_lse=True)
    ro, rl = oracle_full(w, window)
    assert_parity(to_host(out), ro, f"random balanced decode {seed}", to_host(lse), rl)
