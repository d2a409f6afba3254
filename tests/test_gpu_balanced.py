"""The balanced paged decode (sinkattn_decode_paged_balanced) on the GPU.

What it computes is what sinkattn_decode_paged computes; the split differs:
the batch's live pages, request after request, are cut into equal segments
(Perplexity blog "GPT-OSS on day 0", section "Kernels for GPT-OSS > Sink
attention": attention split into blocks along the KV sequence, the sink in
each request's first block only, the blocks merged).  Checked against the
fp64 oracle: outputs and LSE at full size and at edge shapes, the workspace
partials of every multi-segment request against the oracle's pieces (the
sink in the first piece only), and the segment rule and paged gathers bit
for bit with count, one-hot and permutation probes.
"""

import numpy as np
import pytest

import oracle
from gqa_attention_sinks_amd import workloads as wl
from tests._gpu import (DeviceWorkload, assert_parity, bits_to_dev, kv_cache, oracle_full, say, to_host)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_attention_sinks_amd as sa
    sa.load_library()


def _run(d, num_segments, window=0, sinks=True):
    """Balanced decode through the binding; returns out, lse and the workspace."""
    import torch
    import gqa_attention_sinks_amd as sa
    w = d.w
    n = num_segments or sa.pick_num_segments(w.num_kv_heads)
    ws = torch.full((sa.decode_balanced_workspace_bytes(w.batch, w.num_qo_heads, n),), 0xFF, dtype=torch.uint8,
                    device=d.q.device)                  # NaN-filled: a partial that is not written shows
    out, lse = sa.decode_paged_balanced(d.q, d.k, d.v, d.kv_indptr, d.page_indices, d.kv_len,
                                        d.sinks if sinks else None, w.scale, num_segments=n, window=window,
                                        workspace=ws, return_lse=True)
    return out, lse, ws, n


def _pieces_check(w, ws, n, window, what):
    """Every multi-segment request's pieces in the workspace against the
    oracle's pieces (sink in the first piece only)."""
    import gqa_attention_sinks_amd as sa
    plan, lse_ws, o_ws = sa.balanced_workspace_views(ws, w.batch, w.num_qo_heads, n)
    pieces = oracle.balanced_pieces_ref(w.kv_len, n, window)
    first, n_pages, _ = oracle.live_pages_ref(w.kv_len, window)
    np.testing.assert_array_equal(plan.cpu().numpy(), np.concatenate([[0], np.cumsum(n_pages)]))
    segs = sa.balanced_workspace_segments(ws, w.batch).cpu().numpy()
    np.testing.assert_array_equal(segs, sa.balanced_segments(w.kv_len, n, window))
    parts = oracle.pieces_partials_ref(w.q, kv_cache(w), w.sinks, w.scale, pieces, window)
    lse_h, o_h = to_host(lse_ws), to_host(o_ws)
    checked = 0
    for b, pb in enumerate(pieces):
        if len(pb) < 2:
            continue
        for i, (s, _, _) in enumerate(pb):
            slot = s + b
            ro, rl = parts[b][0][:, i, :], parts[b][1][:, i]
            assert_parity(o_h[slot], ro, f"{what} request {b} piece {i}", lse_h[slot], rl)
            checked += 1
    return checked


def test_paged_decode_full_size():
    """64 requests, KV lengths uniform in [1, 4096], the library's segment
    count: every output and LSE, and every workspace partial."""
    w = wl.paged_decode()
    say("balanced decode full size: B=64 kv~U[1,4096]")
    out, lse, ws, n = _run(DeviceWorkload(w), 0)
    ro, rl = oracle_full(w, 0)
    assert_parity(to_host(out), ro, f"balanced paged_decode N={n}", to_host(lse), rl)
    assert _pieces_check(w, ws, n, 0, "balanced paged_decode") > 0


def test_long_split_decode_full_size():
    """8 requests of 131072 keys with -inf and +20 sinks: each request
    spans many segments."""
    w = wl.long_split_decode()
    say("balanced decode long: B=8 L=131072")
    out, lse, ws, n = _run(DeviceWorkload(w), 0)
    ro, rl = oracle_full(w, 0)
    assert_parity(to_host(out), ro, f"balanced long decode N={n}", to_host(lse), rl)


@pytest.mark.parametrize("num_segments", [1, 2, 7, 64, 192, 1000])
@pytest.mark.parametrize("window", [0, 1, 37, 128, 3000])
def test_edge_lengths_segments_windows(num_segments, window):
    """Lengths around a page edge, a request with no key, more segments than
    pages; sinks with -inf and +20 outliers."""
    rng = np.random.default_rng(num_segments * 10 + window)
    lengths = np.array([1, 15, 16, 17, 700, 4095, 4096, 33, 2, 1500])
    w = wl.make_paged("bal_edge", lengths, np.ones(len(lengths)), 16, 2, rng=rng, decode=True,
                      sink_overrides=wl.outlier_sinks)
    w.kv_len = w.kv_len.copy()
    w.kv_len[8] = 0                      # a request without keys: out 0, lse = sink
    say(f"balanced edges N={num_segments} W={window}")
    d = DeviceWorkload(w)
    out, lse, ws, n = _run(d, num_segments, window)
    ro, rl = oracle_full(w, window)
    assert_parity(to_host(out), ro, f"balanced edges N={num_segments} W={window}", to_host(lse), rl)
    _pieces_check(w, ws, n, window, f"balanced edges N={num_segments} W={window}")


@pytest.mark.parametrize("heads", [(4, 4), (16, 1), (64, 8)])
def test_group_sizes_and_no_sinks(heads):
    hq, hkv = heads
    rng = np.random.default_rng(hq + hkv)
    w = wl.make_paged("bal_groups", [1, 40, 700, 16, 3000], np.ones(5), hq, hkv, rng=rng, decode=True)
    d = DeviceWorkload(w)
    say(f"balanced groups {heads}")
    for sinks in (True, False):
        out, lse, _, n = _run(d, 13, 0, sinks=sinks)
        ro, rl = oracle_full(w, 0, sinks=sinks)
        assert_parity(to_host(out), ro, f"balanced group {hq // hkv} sinks={sinks}", to_host(lse), rl)


def test_largest_batch():
    w = wl.paged_decode(seed=9, batch=256, max_len=300)
    say("balanced decode B=256")
    out, lse, _, n = _run(DeviceWorkload(w), 0)
    ro, rl = oracle_full(w, 0)
    assert_parity(to_host(out), ro, "balanced B=256", to_host(lse), rl)


# ---------------------------------------------------------------------------
# bit-exact probes of the segment rule and the gathers
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("num_segments", [3, 29, 192])
@pytest.mark.parametrize("window", [0, 100])
def test_count_probe_piece_sizes(num_segments, window):
    """Zero queries and no sink: every piece's LSE is ln(its key count), so
    exp(lse) rounds to the exact count of the oracle's piece (the keys of the
    piece inside the row's window)."""
    lengths = np.array([1, 16, 17, 1000, 4096, 4095, 333, 48])
    base = wl.make_paged("bal_count", lengths, np.ones(len(lengths)), 16, 2,
                         rng=np.random.default_rng(5), decode=True)
    w = wl.zero_query_probe(base)
    say(f"balanced count probe N={num_segments} W={window}")
    out, lse, ws, n = _run(DeviceWorkload(w), num_segments, window)
    import gqa_attention_sinks_amd as sa
    _, lse_ws, _ = sa.balanced_workspace_views(ws, w.batch, w.num_qo_heads, n)
    lse_h, lse_out = to_host(lse_ws), to_host(lse)
    pieces = oracle.balanced_pieces_ref(lengths, n, window)
    for b, pb in enumerate(pieces):
        n_k = int(lengths[b])
        lo = max(0, n_k - window) if window else 0
        assert int(round(float(np.exp(lse_out[b, 0])))) == n_k - lo, (b, lse_out[b, 0])
        if len(pb) < 2:
            continue
        for s, a, e in pb:
            counts = np.rint(np.exp(lse_h[s + b])).astype(np.int64)
            assert np.all(counts == e - a), (b, s, a, e, counts[:4])


@pytest.mark.parametrize("num_segments", [5, 192])
def test_one_hot_target_per_piece(num_segments):
    """One target key per request: the merged bf16 output equals the target's
    V code bit for bit (any wrong page, slot or segment shows)."""
    lengths = np.array([1, 16, 17, 1000, 4096, 4095, 333])
    base = wl.make_paged("bal_onehot", lengths, np.ones(len(lengths)), 16, 2,
                         rng=np.random.default_rng(6), decode=True)
    rng = np.random.default_rng(8)
    targets = [[int(rng.integers(0, l))] for l in lengths]
    w = wl.one_hot_probe(base, targets)
    say(f"balanced one-hot N={num_segments}")
    out, _, _, _ = _run(DeviceWorkload(w), num_segments)
    g = to_host(out)
    for b, (t,) in enumerate(targets):
        want = wl.value_code(np.array([t]), np.arange(64))[0].astype(np.float64)
        for h in range(w.num_qo_heads):
            np.testing.assert_array_equal(g[b, h], want, err_msg=f"request {b} head {h} target {t}")


def test_page_permutation_is_invisible():
    w = wl.paged_decode(seed=11, batch=40, max_len=2000)
    w2 = wl.repermute(w, seed=3)
    say("balanced permutation")
    a, la, _, _ = _run(DeviceWorkload(w), 0)
    b, lb, _, _ = _run(DeviceWorkload(w2), 0)
    assert np.array_equal(to_host(a), to_host(b))
    assert np.array_equal(to_host(la), to_host(lb))


def test_skewed_batch():
    """One request of 131072 keys among 63 short ones: the long request spans
    most segments."""
    w = wl.skewed_decode()
    say("balanced skewed decode: one 131072-key request + 63 in [1, 4096]")
    d = DeviceWorkload(w)
    out, lse, ws, n = _run(d, 0)
    ro, rl = oracle_full(w, 0)
    assert_parity(to_host(out), ro, f"balanced skewed N={n}", to_host(lse), rl)
    # and the split path on the same batch
    o2, l2 = d.decode(4)
    assert_parity(to_host(o2), ro, "split skewed S=4", to_host(l2), rl)
