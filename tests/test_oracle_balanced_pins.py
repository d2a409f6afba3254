"""Pins of the oracle's balanced split of a decode batch (reading R24).

Perplexity blog "GPT-OSS on day 0", section "Kernels for GPT-OSS > Sink
attention": attention may be split into blocks along the KV sequence, only
the first block carries the sink, and the blocks' softmaxes combine into
the whole one.  The balanced split cuts the batch's live pages (request after
request) into equal segments, so a segment may hold pieces of several
requests.  Pinned here against a token-by-token brute force of the rule and
of the piece softmaxes (tests/_loops.py), against the unsplit oracle
(split == unsplit for every segment count, with a negative control that
seeds every piece), and by the rule's invariants.
"""

import numpy as np
import pytest

import oracle
from tests import _loops
from tests.test_oracle_pins import _tiny_problem


def _spec_kv_len(p):
    return np.asarray(p["spec"]["kv_len"], dtype=np.int64)


@pytest.mark.parametrize("seed", range(12))
def test_pieces_and_partials_match_token_brute_force(seed):
    rng = np.random.default_rng(31000 + seed)
    p = _tiny_problem(rng, paged=True, batch=int(rng.integers(1, 5)), max_len=40, page_size=4,
                      qo_mode="decode", sink_kind="mixed" if seed % 3 == 0 else "normal")
    kv_len = _spec_kv_len(p)
    for n_seg in (1, 2, 3, int(rng.integers(4, 30))):
        pieces = oracle.balanced_pieces_ref(kv_len, n_seg, p["window"], page_size=4)
        parts = oracle.pieces_partials_ref(p["q"], p["kv"], p["sinks"], p["scale"], pieces, p["window"])
        brute = _loops.brute_balanced(p["q"].tolist(), p["spec"], p["sinks"].tolist(), p["scale"], p["window"],
                                      p["hkv"], n_seg)
        for b in range(len(kv_len)):
            assert [(s, lo, hi) for s, lo, hi, _, _ in brute[b]] == pieces[b], (b, n_seg)
            o, l = parts[b]
            np.testing.assert_allclose(o, np.array([e[3] for e in brute[b]]).transpose(1, 0, 2),
                                       rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(l, np.array([e[4] for e in brute[b]]).T, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("seed", range(8))
def test_balanced_split_equals_unsplit_with_negative_control(seed):
    rng = np.random.default_rng(32000 + seed)
    p = _tiny_problem(rng, paged=True, batch=int(rng.integers(2, 5)), max_len=90, page_size=4,
                      qo_mode="decode")
    kv_len = _spec_kv_len(p)
    full_o, full_l = oracle.sink_attention_ref(p["q"], p["qo_indptr"], p["kv"], p["sinks"], p["scale"],
                                               p["window"])
    for n_seg in (1, 2, 3, 5, 8, 17, 64):
        pieces = oracle.balanced_pieces_ref(kv_len, n_seg, p["window"], page_size=4)
        parts = oracle.pieces_partials_ref(p["q"], p["kv"], p["sinks"], p["scale"], pieces, p["window"])
        bad = oracle.pieces_partials_ref(p["q"], p["kv"], p["sinks"], p["scale"], pieces, p["window"],
                                         sink_in_every_piece=True)
        for b in range(len(kv_len)):
            out, lse = oracle.merge_ref(*parts[b])
            np.testing.assert_allclose(out, full_o[b], rtol=1e-13, atol=1e-13)
            np.testing.assert_allclose(lse, full_l[b], rtol=1e-13, atol=1e-13)
            # negative control: every extra seeded piece adds one more sink mass
            _, lb = oracle.merge_ref(*bad[b])
            extra = len(pieces[b]) - 1
            expect = np.log(np.exp(full_l[b]) + extra * np.exp(p["sinks"]))
            np.testing.assert_allclose(lb, expect, rtol=1e-12)
            if extra:     # the control has teeth: the extra masses move the LSE
                assert np.max(np.abs(lb - full_l[b])) > 1e-9


def test_a_request_without_keys_is_the_sink_alone():
    rng = np.random.default_rng(33000)
    p = _tiny_problem(rng, paged=True, batch=3, max_len=30, page_size=4, qo_mode="decode")
    kv = p["kv"]
    kv.kv_len = np.array([kv.kv_len[0], 0, kv.kv_len[2]])
    pieces = oracle.balanced_pieces_ref(kv.kv_len, 4, 0, page_size=4)
    assert pieces[1] == [(-1, 0, 0)]
    o, l = oracle.pieces_partials_ref(p["q"], kv, p["sinks"], p["scale"], pieces)[1]
    assert np.all(o == 0.0)
    np.testing.assert_array_equal(l[:, 0], p["sinks"])


def test_segment_rule_invariants():
    """Pieces cover each request's live keys once, in order, on whole pages
    (cut only at page edges); segments hold floor or ceil of T / N pages;
    consecutive requests' pieces share at most the segment where one ends and
    the next begins."""
    rng = np.random.default_rng(34000)
    for _ in range(300):
        batch = int(rng.integers(1, 40))
        kv_len = rng.integers(0, 3000, size=batch)
        kv_len[rng.random(batch) < 0.1] = 0
        window = int(rng.choice([0, 0, 1, 16, 100, 5000]))
        n_seg = int(rng.integers(1, 300))
        pieces = oracle.balanced_pieces_ref(kv_len, n_seg, window)
        first, n_pages, lo = oracle.live_pages_ref(kv_len, window)
        total = int(n_pages.sum())
        seg_pages = np.zeros(n_seg, dtype=np.int64)
        last_seg = -1
        for b in range(batch):
            if kv_len[b] == 0:
                assert pieces[b] == [(-1, 0, 0)]
                continue
            segs = [s for s, _, _ in pieces[b]]
            assert segs == sorted(set(segs))
            assert segs[0] >= last_seg
            last_seg = segs[-1]
            assert pieces[b][0][1] == lo[b] and pieces[b][-1][2] == kv_len[b]
            for (s0, _, h0), (s1, l1, _) in zip(pieces[b], pieces[b][1:]):
                assert h0 == l1 and l1 % 16 == 0
            for s, a, e in pieces[b]:
                seg_pages[s] += -(-e // 16) - a // 16
        assert seg_pages.sum() == total
        assert seg_pages.max() - seg_pages.min() <= 1
