"""GPU parity: the HIP library (through its C ABI binding) against the fp64
oracle on the same seeded inputs.

What is being checked (Perplexity blog "GPT-OSS on day 0", section "Kernels
for GPT-OSS > Sink attention"): one sink logit per head in the softmax
denominator with no value row, the streaming softmax seeded with it, and under
a KV split the sink in the first chunk only.

Sizes: small cases compare every element; the GPT-OSS-shaped workloads run at
their full sizes in the launch configuration the benchmark times and are
compared element by element too (every output and every LSE), the oracle
spread over all host cores.
"""

import numpy as np
import pytest

import gqa_attention_sinks_amd as sa
import oracle
from gqa_attention_sinks_amd import workloads as wl
from tests._gpu import (DeviceWorkload, assert_parity, assert_parity_by_request, host_workers, kv_cache,
                        oracle_full, say, to_host)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_attention_sinks_amd as sa
    sa.load_library()


# ---------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------

def test_tiny_prefill_full():
    w = wl.tiny_prefill()
    say("tiny_prefill: B=1 Hq=4 Hkv=1 n=128 contiguous")
    d = DeviceWorkload(w)
    out, lse = d.prefill(window=0)
    ro, rl = oracle_full(w, 0)
    assert_parity(to_host(out), ro, "tiny_prefill", to_host(lse), rl)


@pytest.mark.parametrize("window", [0, 1, 37, 128, 129])
@pytest.mark.parametrize("paged", [False, True])
def test_prefill_ragged_small(window, paged):
    """Ragged requests spanning several tiles, chunked prefill (n_q < n_k),
    GQA 8:1, windows around a tile edge, paged and contiguous KV."""
    rng = np.random.default_rng(11)
    kv_len = np.array([1, 130, 300, 77, 513])
    qo_len = np.array([1, 130, 129, 20, 257])
    maker = wl.make_paged if paged else wl.make_contiguous
    w = maker("ragged", kv_len, qo_len, 16, 2, rng=rng)
    say(f"prefill ragged paged={paged} window={window} qo={list(qo_len)} kv={list(kv_len)}")
    out, lse = DeviceWorkload(w).prefill(window=window)
    ro, rl = oracle_full(w, window)
    assert_parity(to_host(out), ro, f"prefill ragged w={window} paged={paged}", to_host(lse), rl)


@pytest.mark.parametrize("paged", [False, True])
def test_prefill_host_plan_is_invisible(paged):
    """The exact launch from the host copy of qo_indptr and the upper-bound
    launch without it give bitwise identical results."""
    rng = np.random.default_rng(21)
    kv_len = np.array([300, 1, 77, 513, 2])
    qo_len = np.array([300, 1, 20, 257, 1])
    maker = wl.make_paged if paged else wl.make_contiguous
    w = maker("plan", kv_len, qo_len, 16, 2, rng=rng)
    say(f"prefill host plan paged={paged}")
    d = DeviceWorkload(w)
    for window in [0, 128]:
        a_out, a_lse = d.prefill(window=window, host_plan=True)
        b_out, b_lse = d.prefill(window=window, host_plan=False)
        assert np.array_equal(to_host(a_out), to_host(b_out))
        assert np.array_equal(to_host(a_lse), to_host(b_lse))
        if paged:
            # a tile order ranked on the host from kv_len, and one from a
            # wrong copy of kv_len (order only): the same bits
            for name, host in [("exact", w.kv_len), ("reversed", np.ascontiguousarray(w.kv_len[::-1]))]:
                c_out, c_lse = d.prefill(window=window, kv_len_host=host)
                assert np.array_equal(to_host(c_out), to_host(b_out)), name
                assert np.array_equal(to_host(c_lse), to_host(b_lse)), name


@pytest.mark.parametrize("case", ["rank_256", "rank_257", "plan_512", "plan_513", "one_request"])
def test_prefill_host_plan_at_its_limits(case):
    """Launches at the limits of the host-built tile order: up to 256 tiles
    of differently shaped requests are ranked by key count (257: request by
    request), up to 512 tiles take their (request, tile) from the host plan
    (513: the kernel's own scan); a single request over contiguous KV is
    planned with no key counts on the host (nothing to rank).  Planned and
    unplanned launches give the same bits."""
    rng = np.random.default_rng(31)
    if case == "one_request":
        qo_len = np.array([300], dtype=np.int64)
        w = wl.make_contiguous("one", np.array([1000]), qo_len, 16, 2, rng=rng)
        windows = [0, 128]
        host = None
    elif case.startswith("rank"):
        # paged, unbounded window: 64-row tiles (16 query / 2 KV heads)
        n = int(case.split("_")[1])
        qo_len = np.array([64 * (n - 3), 64, 64, 64, 1, 1], dtype=np.int64)   # single rows: decode kernel
        kv_len = qo_len + np.array([0, 3000, 10, 700, 5, 900])
        w = wl.make_paged("rank", kv_len, qo_len, 16, 2, rng=rng)
        windows = [0, 3000]   # ranked also under a window longer than 2048 keys
        host = w.kv_len
    else:
        # contiguous, 128-key window (no ranking): 512 tiles, or 513 with one more row
        qo_len = np.array([64 * 256, 64 * 256] + ([1] if case == "plan_513" else []), dtype=np.int64)
        w = wl.make_contiguous("plan", qo_len, qo_len, 16, 2, rng=rng)
        windows = [128]
        host = None
    say(f"prefill host plan limit {case}: qo={list(qo_len)}")
    d = DeviceWorkload(w)
    for window in windows:
        a_out, a_lse = d.prefill(window=window, kv_len_host=host)
        b_out, b_lse = d.prefill(window=window, host_plan=False)
        assert np.array_equal(to_host(a_out), to_host(b_out))
        assert np.array_equal(to_host(a_lse), to_host(b_lse))


@pytest.mark.parametrize("group", [1, 4, 16])
def test_prefill_group_sizes_and_no_sinks(group):
    rng = np.random.default_rng(12 + group)
    hkv = 2
    w = wl.make_contiguous("groups", [200, 64], [200, 33], hkv * group, hkv, rng=rng)
    say(f"prefill group={group}")
    d = DeviceWorkload(w)
    out, lse = d.prefill(window=0)
    ro, rl = oracle_full(w, 0)
    assert_parity(to_host(out), ro, f"prefill group {group}", to_host(lse), rl)
    out, lse = d.prefill(window=0, sinks=False)
    ro, rl = oracle_full(w, 0, sinks=False)
    assert_parity(to_host(out), ro, f"prefill group {group} no sinks", to_host(lse), rl)


@pytest.mark.parametrize("window", [37, 100])
@pytest.mark.parametrize("group", [1, 2, 8])
def test_prefill_group_sizes_under_windows(group, window):
    """Groups that do not split into fours put 256 consecutive rows of one
    head in a workgroup: under a window the later waves skip the
    workgroup's first key tiles and meet their first visible keys later."""
    rng = np.random.default_rng(40 + group + window)
    hkv = 2
    w = wl.make_paged("groups_w", [700, 90], [600, 90], hkv * group, hkv, rng=rng)
    say(f"prefill group={group} window={window}")
    out, lse = DeviceWorkload(w).prefill(window=window)
    ro, rl = oracle_full(w, window)
    assert_parity(to_host(out), ro, f"prefill group {group} window {window}", to_host(lse), rl)


def test_prefill_outlier_sinks():
    rng = np.random.default_rng(13)
    w = wl.make_paged("outliers", [300, 64], [300, 64], 16, 2, rng=rng, sink_overrides=wl.outlier_sinks)
    say("prefill with -inf / +20 sinks")
    out, lse = DeviceWorkload(w).prefill(window=0)
    ro, rl = oracle_full(w, 0)
    assert_parity(to_host(out), ro, "prefill outlier sinks", to_host(lse), rl)


def test_causal_prefill_full_size():
    """4 x 8192 causal prefill, 64/8 heads, in the benchmark's launch: every
    output element and every LSE against the oracle."""
    w = wl.causal_prefill()
    say(f"causal_prefill full size: B=4 n=8192 Hq=64 Hkv=8, oracle on {host_workers()} threads")
    out, lse = DeviceWorkload(w).prefill(window=0)
    g, gl = to_host(out), to_host(lse)
    del out, lse
    ro, rl = oracle_full(w, 0)
    assert_parity_by_request(w, g, ro, "causal_prefill", gl, rl)


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("num_splits", [1, 2, 4, 5, 16])
def test_paged_decode_full(num_splits):
    """Full size at several split counts, including the library's own pick for
    this batch (4), which is what the benchmark times."""
    import gqa_attention_sinks_amd as sa
    w = wl.paged_decode()
    assert sa.pick_num_splits(w.kv_len, w.num_kv_heads) == 4
    say(f"paged_decode full size: B=64 kv~U[1,4096] S={num_splits}")
    d = DeviceWorkload(w)
    out, lse = d.decode(num_splits)
    ro, rl = oracle_full(w, 0)
    assert_parity(to_host(out), ro, f"paged_decode S={num_splits}", to_host(lse), rl)


@pytest.mark.parametrize("length", [1, 15, 16, 17, 4095, 4096])
@pytest.mark.parametrize("window", [0, 1, 127, 128, 129, 3000])
def test_decode_edge_lengths_windows(length, window):
    """Lengths around a page and near the largest, windows around 128; the
    kernel ranks requests by length unless a window of at most 2048 keys
    makes their work alike (3000: ranked and windowed)."""
    rng = np.random.default_rng(length * 7 + window)
    w = wl.make_paged("edge", [length, max(1, length // 2)], [1, 1], 16, 2, rng=rng, decode=True,
                      sink_overrides=wl.outlier_sinks)
    say(f"decode edge length={length} window={window}")
    d = DeviceWorkload(w)
    ro, rl = oracle_full(w, window)
    for s in [1, 3, 16]:
        out, lse = d.decode(s, window=window)
        assert_parity(to_host(out), ro, f"decode L={length} W={window} S={s}", to_host(lse), rl)


@pytest.mark.parametrize("heads", [(4, 4), (4, 2), (16, 1)])
def test_decode_group_sizes_and_no_sinks(heads):
    """GQA groups of 1, 2 and 16 query heads per KV head (the MFMA columns a
    page load serves), with and without sinks."""
    hq, hkv = heads
    rng = np.random.default_rng(17 + hq * 4 + hkv)
    w = wl.make_paged("groups", [1, 40, 700, 16], [1, 1, 1, 1], hq, hkv, rng=rng, decode=True)
    say(f"decode group={hq // hkv}")
    d = DeviceWorkload(w)
    for sinks in [True, False]:
        ro, rl = oracle_full(w, 0, sinks=sinks)
        for s in [1, 3]:
            out, lse = d.decode(s, sinks=sinks)
            assert_parity(to_host(out), ro, f"decode group {hq // hkv} S={s} sinks={sinks}", to_host(lse), rl)


def test_decode_partials_sink_only_in_chunk_zero():
    """The partials themselves: chunk 0 carries the sink, the others do not."""
    w = wl.paged_decode(batch=6, max_len=700)
    w.sinks = wl.outlier_sinks(w.sinks)
    say("decode partials S=4")
    o_part, lse_part = DeviceWorkload(w).decode(4, merge=False)
    ro, rl = oracle.split_partials_ref(w.q, kv_cache(w), w.sinks, w.scale, 4)
    assert_parity(to_host(o_part), ro, "o_part", to_host(lse_part), rl)


def test_long_split_decode_full_size():
    """8 x 131072 keys, 16 chunks, sinks with -inf and +20 outliers."""
    w = wl.long_split_decode()
    say("long_split_decode full size: B=8 L=131072 S=16")
    d = DeviceWorkload(w)
    o_part, lse_part = d.decode(16, merge=False)
    out, lse = d.decode(16)
    kv = kv_cache(w)
    rp, rlp = oracle.split_partials_ref(w.q, kv, w.sinks, w.scale, 16, workers=host_workers())
    assert_parity(to_host(o_part), rp, "long decode partials", to_host(lse_part), rlp)
    ro, rl = oracle.merge_ref(rp, rlp)
    assert_parity(to_host(out), ro, "long decode merged", to_host(lse), rl)


# ---------------------------------------------------------------------------
# mixed batch
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("window", [128, 0])
def test_mixed_batch_small_full(window):
    w = wl.mixed_batch(n_prefill=4, chunk=200, max_prefix=900, n_decode=30, max_decode_len=1500)
    say(f"mixed small window={window}")
    out, lse = DeviceWorkload(w).prefill(window=window)
    ro, rl = oracle_full(w, window)
    assert_parity(to_host(out), ro, f"mixed small W={window}", to_host(lse), rl)


@pytest.mark.parametrize("window", [128, 0])
def test_mixed_batch_full_size(window):
    """16 x 512-token prefill chunks + 240 decode rows in one call: every
    output element and LSE of every row against the oracle."""
    w = wl.mixed_batch()
    say(f"mixed_batch full size window={window}, oracle on {host_workers()} threads")
    out, lse = DeviceWorkload(w).prefill(window=window)
    g, gl = to_host(out), to_host(lse)
    del out, lse
    ro, rl = oracle_full(w, window)
    n_pre = w.meta["n_prefill"]
    assert_parity_by_request(w, g, ro, f"mixed full W={window} prefill", gl, rl, requests=range(n_pre))
    d0 = int(w.qo_indptr[n_pre])
    assert_parity(g[d0:], ro[d0:], f"mixed full W={window} decode rows", gl[d0:], rl[d0:])


# ---------------------------------------------------------------------------
# scheduling paths: the work-order logic differs by batch shape, the results
# must not
# ---------------------------------------------------------------------------

def test_decode_large_batch_unranked():
    """300 requests: above the size the decode kernel ranks by length, so
    units run in natural order."""
    rng = np.random.default_rng(31)
    kv_len = rng.integers(1, 300, size=300)
    w = wl.make_paged("big_batch", kv_len, np.ones(300), 16, 2, rng=rng, decode=True,
                      sink_overrides=wl.outlier_sinks)
    say("decode 300 requests (unranked), S in {1, 3}")
    d = DeviceWorkload(w)
    ro, rl = oracle_full(w, 0)
    for s in [1, 3]:
        out, lse = d.decode(s)
        assert_parity(to_host(out), ro, f"decode B=300 S={s}", to_host(lse), rl)


@pytest.mark.parametrize("uniform", [False, True])
def test_prefill_many_tiles_request_major(uniform):
    """More than 256 query tiles (uneven or equal requests): the prefill
    takes tiles request by request instead of ranking them."""
    rng = np.random.default_rng(32)
    n = 130
    qo_len = np.full(n, 300) if uniform else rng.integers(257, 400, size=n)
    kv_len = qo_len + (0 if uniform else rng.integers(0, 64, size=n))
    w = wl.make_contiguous("many_tiles", kv_len, qo_len, 4, 1, rng=rng)
    say(f"prefill {n} requests, {int(np.sum((qo_len + 255) // 256))} tiles, uniform={uniform}")
    out, lse = DeviceWorkload(w).prefill(window=0)
    ro, rl = oracle_full(w, 0)
    assert_parity(to_host(out), ro, f"prefill many tiles uniform={uniform}", to_host(lse), rl)


def test_prefill_uneven_ranked_order_windowed():
    """Uneven requests with at most 256 tiles take the ranked order without a
    window and under a window longer than 2048 keys; under a short window
    (200) they take request order."""
    rng = np.random.default_rng(33)
    qo_len = np.array([600, 20, 513, 256, 1000, 3])
    kv_len = qo_len + np.array([0, 700, 5, 300, 0, 2000])
    w = wl.make_paged("ranked", kv_len, qo_len, 8, 2, rng=rng)
    say("prefill uneven requests, windows 0, 200 and 3000")
    d = DeviceWorkload(w)
    for window in [0, 200, 3000]:
        out, lse = d.prefill(window=window)
        ro, rl = oracle_full(w, window)
        assert_parity(to_host(out), ro, f"prefill ranked W={window}", to_host(lse), rl)


# ---------------------------------------------------------------------------
# merge entry point
# ---------------------------------------------------------------------------

def _host_copies(w):
    """The right host copy of kv_len, a reversed (wrong) one and a constant one:
    each orders the work differently, none may change a result."""
    lens = np.asarray(w.kv_len, dtype=np.int32)
    return {"right": lens, "reversed": lens[::-1].copy(), "constant": np.zeros_like(lens)}


def _same(a, b, what):
    for x, y in zip(a, b):
        assert np.array_equal(to_host(x), to_host(y)), f"{what}: results differ"


@pytest.mark.parametrize("window", [0, 128, 3000])
def test_decode_host_order_is_invisible(window):
    """Work ordered on the host from a copy of kv_len (right or wrong) and by
    the kernels' own ranking give bitwise identical results; the planned path
    meets the parity bar."""
    w = wl.paged_decode(batch=40, max_len=3000)
    d = DeviceWorkload(w)
    ro, rl = oracle_full(w, window)
    for s in [1, 4]:
        say(f"decode host order window={window} S={s}")
        base = d.decode(s, window=window)
        for name, host in _host_copies(w).items():
            got = d.decode(s, window=window, kv_len_host=host)
            _same(got, base, f"decode host copy {name} W={window} S={s}")
        assert_parity(to_host(got[0]), ro, f"decode planned W={window} S={s}", to_host(got[1]), rl)


@pytest.mark.parametrize("batch,window", [(2, 0), (256, 0), (257, 0), (40, 2048), (40, 2049)])
def test_decode_host_order_at_its_limits(batch, window):
    """The host order applies to batches of 2..256 requests and windows of
    none or over 2048 keys; at and across each limit the results equal the
    kernels' own ordering bit for bit."""
    rng = np.random.default_rng(batch * 7 + window)
    kv_len = rng.integers(1, 2600, size=batch)
    w = wl.make_paged("order_limits", kv_len, np.ones(batch), 16, 2, rng=rng, decode=True)
    d = DeviceWorkload(w)
    say(f"decode host order limits batch={batch} window={window}")
    for s in [1, 3]:
        base = d.decode(s, window=window)
        for name, host in _host_copies(w).items():
            _same(d.decode(s, window=window, kv_len_host=host), base, f"B={batch} W={window} S={s} {name}")


def test_decode_host_order_large_batch_and_noalloc():
    """Above 256 requests the host copy is ignored; the no-allocation entry
    point takes it like the allocating one."""
    rng = np.random.default_rng(32)
    kv_len = rng.integers(1, 300, size=300)
    w = wl.make_paged("big_batch", kv_len, np.ones(300), 16, 2, rng=rng, decode=True)
    d = DeviceWorkload(w)
    say("decode B=300 with a host copy; noalloc with a host copy")
    _same(d.decode(3, kv_len_host=w.kv_len), d.decode(3), "decode B=300 host copy")
    v = wl.paged_decode(batch=24, max_len=2000)
    e = DeviceWorkload(v)
    for name, host in _host_copies(v).items():
        a = sa.decode_paged_noalloc(e.q, e.k, e.v, e.kv_indptr, e.page_indices, e.kv_len, e.sinks, v.scale,
                                    num_splits=4, return_lse=True, kv_len_host=host)
        _same(a, e.decode(4), f"noalloc host copy {name}")


# ---------------------------------------------------------------------------
# several query rows per request (speculative verify) over paged KV
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("num_splits", [1, 3, 16])
def test_verify_decode_full(num_splits):
    w = wl.verify_decode()
    say(f"verify_decode full size: B=64 rows~U[2,8] kv~U[8,4096] S={num_splits}")
    out, lse = DeviceWorkload(w).decode_multi(num_splits, 8)
    ro, rl = oracle_full(w, 0)
    assert_parity(to_host(out), ro, f"verify_decode S={num_splits}", to_host(lse), rl)


@pytest.mark.parametrize("heads,max_rows", [((64, 8), 2), ((4, 1), 8), ((16, 1), 4), ((64, 8), 5)])
@pytest.mark.parametrize("window", [0, 1, 3, 128, 3000])
def test_verify_decode_shapes_windows(heads, max_rows, window):
    hq, hkv = heads
    rng = np.random.default_rng(hq * 100 + max_rows * 10 + window)
    kv_len = np.array([1, 2, 15, 16, 17, 33, 200, 1000, max_rows, 4097])
    qo_len = np.minimum(rng.integers(1, max_rows + 1, size=len(kv_len)), kv_len)
    w = wl.make_paged("verify_edge", kv_len, qo_len, hq, hkv, rng=rng, sink_overrides=wl.outlier_sinks)
    say(f"verify edges heads={heads} max_rows={max_rows} window={window}")
    d = DeviceWorkload(w)
    ro, rl = oracle_full(w, window)
    for s in [1, 3, 16]:
        out, lse = d.decode_multi(s, max_rows, window=window)
        assert_parity(to_host(out), ro, f"verify {heads} R={max_rows} W={window} S={s}", to_host(lse), rl)


def test_verify_decode_partials_and_rows_before_the_first_key():
    """Partials per row (sink only in chunk 0); a request with fewer cached
    keys than query rows has rows that see no key: out 0, lse = sink."""
    rng = np.random.default_rng(77)
    w = wl.make_paged("verify_partials", [300, 40, 5, 700], [4, 7, 5, 1], 64, 8, rng=rng,
                      sink_overrides=wl.outlier_sinks)
    w.kv_len = w.kv_len.copy()
    w.kv_len[2] = 2                      # 5 query rows over 2 keys: rows 0..2 sit before key 0
    say("verify partials S=4 and rows before the first key")
    d = DeviceWorkload(w)
    o_part, lse_part = d.decode_multi(4, 8, merge=False)
    ro, rl = oracle.split_partials_ref(w.q, kv_cache(w), w.sinks, w.scale, 4, qo_indptr=w.qo_indptr)
    assert_parity(to_host(o_part), ro, "verify o_part", to_host(lse_part), rl)
    out, lse = d.decode_multi(1, 8)
    fo, fl = oracle_full(w, 0)
    assert_parity(to_host(out), fo, "verify unsplit", to_host(lse), fl)


def test_verify_decode_one_row_matches_the_decode_kernel():
    """With one row per request the multi-row kernel (whose softmax reference
    moves only on overflow) and the single-token kernel (running maximum)
    both meet the parity bar and agree with each other to it."""
    w = wl.paged_decode(batch=20, max_len=3000)
    d = DeviceWorkload(w)
    ro, rl = oracle_full(w, 0)
    say("verify one-row vs decode S=1,5")
    for s in [1, 5]:
        a, la = d.decode(s)
        b, lb = d.decode_multi(s, 1)
        assert_parity(to_host(b), ro, f"one-row multi S={s}", to_host(lb), rl)
        assert_parity(to_host(a), ro, f"decode S={s}", to_host(la), rl)
        assert_parity(to_host(b), to_host(a), f"multi vs decode S={s}", to_host(lb), to_host(la))


# ---------------------------------------------------------------------------
# custom masks: a draft tree per request verified in one step
# ---------------------------------------------------------------------------

def _oracle_masked(w, masks):
    return oracle.sink_attention_ref(w.q, w.qo_indptr, kv_cache(w), w.sinks, w.scale, 0,
                                     workers=host_workers(), custom_mask=masks)


@pytest.mark.parametrize("num_splits", [1, 3, 16])
def test_tree_verify_full(num_splits):
    w = wl.verify_tree()
    say(f"verify_tree full size: B=64 rows~U[2,8] random draft trees S={num_splits}")
    out, lse = DeviceWorkload(w).decode_multi(num_splits, 8, masks=w.meta["masks"])
    ro, rl = _oracle_masked(w, w.meta["masks"])
    assert_parity(to_host(out), ro, f"verify_tree S={num_splits}", to_host(lse), rl)


@pytest.mark.parametrize("heads,max_rows", [((64, 8), 8), ((4, 1), 8), ((16, 1), 4), ((64, 8), 2)])
def test_custom_mask_random_and_edges(heads, max_rows):
    hq, hkv = heads
    rng = np.random.default_rng(hq * 1000 + max_rows)
    kv_len = np.array([1, 2, 15, 16, 17, 33, 200, 1000, max_rows, 4097])
    qo_len = np.minimum(rng.integers(1, max_rows + 1, size=len(kv_len)), kv_len)
    w = wl.make_paged("mask_edge", kv_len, qo_len, hq, hkv, rng=rng, sink_overrides=wl.outlier_sinks)
    masks = [rng.random((int(q), int(k))) < 0.5 for q, k in zip(qo_len, kv_len)]
    masks[3][0, :] = False            # a row that sees no key: out 0, lse = sink
    say(f"random masks heads={heads} max_rows={max_rows}")
    d = DeviceWorkload(w)
    ro, rl = _oracle_masked(w, masks)
    for s in [1, 3]:
        out, lse = d.decode_multi(s, max_rows, masks=masks)
        assert_parity(to_host(out), ro, f"mask {heads} R={max_rows} S={s}", to_host(lse), rl)
    o_part, lse_part = d.decode_multi(4, max_rows, merge=False, masks=masks)
    po, pl = oracle.split_partials_ref(w.q, kv_cache(w), w.sinks, w.scale, 4, qo_indptr=w.qo_indptr,
                                       custom_mask=masks)
    assert_parity(to_host(o_part), po, f"mask partials {heads}", to_host(lse_part), pl)


@pytest.mark.parametrize("masked", [False, True])
def test_verify_host_order_is_invisible(masked):
    w = wl.verify_tree() if masked else wl.verify_decode(batch=24)
    masks = w.meta.get("masks") if masked else None
    d = DeviceWorkload(w)
    for s in [1, 3]:
        say(f"verify host order masked={masked} S={s}")
        base = d.decode_multi(s, 8, masks=masks)
        for name, host in _host_copies(w).items():
            _same(d.decode_multi(s, 8, masks=masks, kv_len_host=host), base,
                  f"verify host copy {name} masked={masked} S={s}")


@pytest.mark.parametrize("window", [3, 3000])
def test_verify_host_order_under_windows(window):
    """Windows of at most 2048 keys leave the order to the kernels, longer
    ones use the host order: both give the kernels' own results bit for bit."""
    w = wl.verify_decode(batch=24)
    d = DeviceWorkload(w)
    say(f"verify host order window={window}")
    base = d.decode_multi(3, 8, window=window)
    for name, host in _host_copies(w).items():
        _same(d.decode_multi(3, 8, window=window, kv_len_host=host), base, f"verify W={window} {name}")


@pytest.mark.parametrize("window", [0, 128])
def test_mixed_batch_host_order_is_invisible(window):
    w = wl.mixed_batch(n_prefill=4, chunk=200, max_prefix=900, n_decode=30, max_decode_len=1500)
    d = DeviceWorkload(w)
    say(f"mixed host order window={window}")
    base = d.prefill(window=window)
    for name, host in _host_copies(w).items():
        _same(d.prefill(window=window, kv_len_host=host), base, f"mixed host copy {name} W={window}")


def test_chain_mask_is_the_causal_kernel():
    """A chain-shaped draft tree is the causal rule: the masked kernel gives
    the unmasked one's results bit for bit."""
    w = wl.verify_decode(batch=24, max_len=3000)
    masks = wl.tree_masks(np.random.default_rng(5), w.kv_len, np.diff(w.qo_indptr), chain=True)
    d = DeviceWorkload(w)
    say("chain mask vs causal S=1,4")
    for s in [1, 4]:
        a, la = d.decode_multi(s, 8)
        b, lb = d.decode_multi(s, 8, masks=masks)
        assert np.array_equal(to_host(a), to_host(b)), f"S={s}: outputs differ"
        assert np.array_equal(to_host(la), to_host(lb)), f"S={s}: LSE differ"


def test_merge_entry_point():
    import torch
    import gqa_attention_sinks_amd as sa
    rng = np.random.default_rng(3)
    rows, heads, s = 5, 8, 7
    o = rng.normal(size=(rows, heads, s, 64)).astype(np.float32)
    l = rng.normal(0, 3, size=(rows, heads, s)).astype(np.float32)
    l[0, 0, :] = -np.inf
    o[0, 0, :] = 0
    l[1, :, 3:] = -np.inf
    l[2, 1, 0] = 40.0
    say("merge entry point")
    dev = torch.device("cuda:0")
    out, lse = sa.merge(torch.from_numpy(o).to(dev), torch.from_numpy(l).to(dev), return_lse=True)
    ro, rl = oracle.merge_ref(o, l)
    assert_parity(to_host(out)[1:], ro[1:], "merge", to_host(lse), rl)
    assert np.all(to_host(out)[0, 0] == 0)


@pytest.mark.parametrize("rows,heads,s", [(127, 64, 3), (129, 64, 3), (129, 64, 17), (520, 64, 2), (135, 61, 4)])
def test_merge_both_launch_shapes(rows, heads, s):
    """Launches of 8192 (row, head) pairs or more pack four pairs into a
    wave, smaller ones one: both against the oracle, with empty, sink-only and
    dominant chunks among the inputs, and a ragged last group of pairs."""
    import torch
    rng = np.random.default_rng(rows * 31 + heads * 7 + s)
    o = rng.normal(size=(rows, heads, s, 64)).astype(np.float32)
    l = rng.normal(0, 3, size=(rows, heads, s)).astype(np.float32)
    l[0, 0, :] = -np.inf
    o[0, 0, :] = 0
    l[1, :, 1:] = -np.inf
    l[2, 5, 0] = 40.0
    l[rows - 1, heads - 1, s - 1] = 30.0
    say(f"merge launch shapes rows={rows} heads={heads} S={s} pairs={rows * heads}")
    dev = torch.device("cuda:0")
    out, lse = sa.merge(torch.from_numpy(o).to(dev), torch.from_numpy(l).to(dev), return_lse=True)
    ro, rl = oracle.merge_ref(o, l)
    g, gl = to_host(out), to_host(lse)
    assert np.all(g[0, 0] == 0) and gl[0, 0] == -np.inf
    g[0, 0] = ro[0, 0] = 0
    assert_parity(g, ro, f"merge rows={rows} heads={heads} S={s}", gl, rl)
