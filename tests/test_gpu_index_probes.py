"""Bit-exact checks of the split rule and the paged gathers on the GPU.

* One-hot probes: with an all-ones query, a target key scoring +60 and every
  other key -60 (scale 1/8, D = 64) and no sink, exp(-120) underflows to 0 in
  fp32, so a softmax range holding one target returns that target's V row
  exactly; V rows hold integer codes of their logical position, so a gather
  from a wrong page or slot shows as a wrong code.
* Count probes: zero queries and no sink make every score 0, so a chunk's
  partial LSE is ln(number of keys it holds); the rounded exp must equal the
  chunk size from the chunk rule exactly, and empty chunks give -inf.
* Permutation: the same logical cache under two physical page permutations
  gives bitwise identical outputs.
The chunk rule (whole pages, ceil split, sink in chunk 0 only) follows the
"Kernels for GPT-OSS > Sink attention" section of the Perplexity blog post
"GPT-OSS on day 0".
"""

import numpy as np
import pytest

import oracle
from gqa_attention_sinks_amd import workloads as wl
from tests._gpu import DeviceWorkload, assert_parity, oracle_full, say, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _codes(pos, d=64):
    return wl.value_code(np.asarray(pos), np.arange(d)).astype(np.float64)


def _decode_base(lengths, seed):
    rng = np.random.default_rng(seed)
    return wl.make_paged("probe", lengths, np.ones(len(lengths)), 16, 2, rng=rng, decode=True)


@pytest.mark.parametrize("num_splits", [2, 5, 16])
def test_one_hot_target_per_chunk(num_splits):
    lengths = np.array([1, 16, 17, 1000, 4096, 4095, 333])
    base = _decode_base(lengths, 40 + num_splits)
    bounds = oracle.split_bounds_ref(lengths, num_splits)
    rng = np.random.default_rng(7)
    targets = []
    for b in range(len(lengths)):
        tb = []
        for c in range(num_splits):
            lo, hi = bounds[b, c]
            if hi > lo:
                tb.append(int(rng.integers(lo, hi)))
        targets.append(tb)
    w = wl.one_hot_probe(base, targets)
    say(f"one-hot per chunk S={num_splits}")
    o_part, lse_part = DeviceWorkload(w).decode(num_splits, merge=False)
    o_part = to_host(o_part)
    lse_part = to_host(lse_part)
    for b in range(len(lengths)):
        k = 0
        for c in range(num_splits):
            lo, hi = bounds[b, c]
            if hi > lo:
                expect = _codes(targets[b][k])
                k += 1
                assert np.array_equal(o_part[b, :, c, :], np.broadcast_to(expect, o_part[b, :, c, :].shape)), \
                    f"request {b} chunk {c}: wrong gather"
            else:
                assert np.all(o_part[b, :, c, :] == 0) and np.all(np.isneginf(lse_part[b, :, c]))


@pytest.mark.parametrize("num_splits", [1, 3, 16])
def test_one_hot_single_target_merged_output_is_exact(num_splits):
    lengths = np.array([5, 64, 65, 2047, 4096, 1])
    base = _decode_base(lengths, 60 + num_splits)
    rng = np.random.default_rng(8)
    targets = [[int(rng.integers(0, l))] for l in lengths]
    w = wl.one_hot_probe(base, targets)
    say(f"one-hot merged S={num_splits}")
    out = to_host(DeviceWorkload(w).decode(num_splits, return_lse=False))
    for b, t in enumerate(targets):
        assert np.array_equal(out[b], np.broadcast_to(_codes(t[0]), out[b].shape)), f"request {b}"


@pytest.mark.parametrize("window", [0, 128])
def test_one_hot_prefill_paged_gather(window):
    """Mixed batch (prefill chunks + decode rows) over a permuted pool: rows
    that can see their request's target must return its code exactly."""
    base = wl.mixed_batch(n_prefill=3, chunk=160, max_prefix=600, n_decode=12, max_decode_len=900)
    rng = np.random.default_rng(9)
    targets = []
    for b in range(base.batch):
        n_k, n_q = int(base.kv_len[b]), int(base.qo_len[b])
        targets.append([int(rng.integers(max(0, n_k - n_q - 40), n_k))])
    w = wl.one_hot_probe(base, targets)
    say(f"one-hot prefill window={window}")
    out = to_host(DeviceWorkload(w).prefill(window=window, return_lse=False))
    checked = 0
    for b in range(w.batch):
        n_k, n_q = int(w.kv_len[b]), int(w.qo_len[b])
        j = targets[b][0]
        for t in range(n_q):
            p = n_k - n_q + t
            lo = max(0, p - window + 1) if window > 0 else 0
            if lo <= j <= p:
                r = int(w.qo_indptr[b]) + t
                assert np.array_equal(out[r], np.broadcast_to(_codes(j), out[r].shape)), f"req {b} row {t}"
                checked += 1
    assert checked > 100


@pytest.mark.parametrize("window", [0, 100])
def test_count_probe_chunk_sizes(window):
    lengths = np.array([1, 15, 16, 17, 31, 32, 33, 500, 4096, 1234])
    s = 5
    w = wl.zero_query_probe(_decode_base(lengths, 77))
    say(f"count probe window={window}")
    _, lse_part = DeviceWorkload(w).decode(s, window=window, merge=False)
    lse_part = to_host(lse_part)
    bounds = oracle.split_bounds_ref(lengths, s)
    for b, n in enumerate(lengths):
        lo_vis = max(0, n - window) if window > 0 else 0
        for c in range(s):
            cnt = max(0, min(bounds[b, c, 1], n) - max(bounds[b, c, 0], lo_vis))
            got = lse_part[b, :, c]
            if cnt == 0:
                assert np.all(np.isneginf(got)), (b, c)
            else:
                assert np.all(np.round(np.exp(got)) == cnt), (b, c, cnt, np.exp(got[:2]))


def test_maximum_split_count():
    """num_splits = 256, the library's maximum: a 4096-key request gets one
    page per chunk and the short ones leave most chunks empty.  The count
    probe gives every chunk's size exactly, and on random data the merged
    output matches the oracle."""
    lengths = np.array([1, 17, 4096, 300, 4095])
    s = 256
    w = wl.zero_query_probe(_decode_base(lengths, 78))
    say("count probe, 256 chunks")
    _, lse_part = DeviceWorkload(w).decode(s, merge=False)
    lse_part = to_host(lse_part)
    bounds = oracle.split_bounds_ref(lengths, s)
    for b, n in enumerate(lengths):
        for c in range(s):
            cnt = max(0, min(bounds[b, c, 1], n) - bounds[b, c, 0])
            got = lse_part[b, :, c]
            if cnt == 0:
                assert np.all(np.isneginf(got)), (b, c)
            else:
                assert np.all(np.round(np.exp(got)) == cnt), (b, c, cnt)
    rng = np.random.default_rng(79)
    w2 = wl.make_paged("max_splits", lengths, np.ones_like(lengths), 16, 2, rng=rng, decode=True,
                       sink_overrides=wl.outlier_sinks)
    say("decode parity, 256 chunks")
    out, lse = DeviceWorkload(w2).decode(s)
    ro, rl = oracle_full(w2, 0)
    assert_parity(to_host(out), ro, "decode S=256", to_host(lse), rl)


def test_page_permutation_is_bitwise_invisible():
    base = wl.paged_decode(batch=16, max_len=2000)
    other = wl.repermute(base, seed=99)
    say("permutation invariance")
    d1, d2 = DeviceWorkload(base), DeviceWorkload(other)
    for s in [1, 4]:
        a = to_host(d1.decode(s, return_lse=False))
        b = to_host(d2.decode(s, return_lse=False))
        assert np.array_equal(a, b)
    mb = wl.mixed_batch(n_prefill=2, chunk=150, max_prefix=500, n_decode=10, max_decode_len=700)
    mo = wl.repermute(mb, seed=5)
    for window in [0, 128]:
        a = to_host(DeviceWorkload(mb).prefill(window=window, return_lse=False))
        b = to_host(DeviceWorkload(mo).prefill(window=window, return_lse=False))
        assert np.array_equal(a, b)
