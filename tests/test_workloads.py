"""The seeded input generators: determinism, page tables, poisoning, shapes."""

import numpy as np

from gqa_attention_sinks_amd import workloads as wl


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -9, -2.5, 3.0e38, np.nan], dtype=np.float32)
    bits = wl.bf16_bits(x)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa (1.0) wins
    assert bits[0] == 0x3F80 and bits[1] == 0x3F80
    assert bits[2] == 0x3F81            # 1 + 3*2^-9 = 1 + 0.75 ulp rounds up to 1 + 2^-7
    assert bits[3] == 0xC020
    assert bits[5] == 0x7FC0


def test_generators_are_deterministic():
    a = wl.paged_decode(batch=4, max_len=100)
    b = wl.paged_decode(batch=4, max_len=100)
    for f in ["q", "k", "v", "kv_len", "page_indices", "sinks"]:
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))


def test_page_tables_and_poison():
    w = wl.paged_decode(batch=6, max_len=70)
    assert w.num_pages == int(np.ceil(w.kv_indptr[-1] * 1.01))
    assert len(np.unique(w.page_indices)) == len(w.page_indices)
    live = np.zeros((w.num_pages, 16), dtype=bool)
    for b in range(w.batch):
        pages = w.page_indices[w.kv_indptr[b]:w.kv_indptr[b + 1]]
        assert len(pages) == -(-int(w.kv_len[b]) // 16)
        for j in range(int(w.kv_len[b])):
            live[pages[j // 16], j % 16] = True
    nan_k = np.isnan(wl_widen(w.k)).all(axis=(1, 3))      # [pages, slots]
    assert np.array_equal(nan_k, ~live)
    assert not np.isnan(wl_widen(w.q)).any()


def wl_widen(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def test_named_small_shapes():
    t = wl.tiny_prefill()
    assert t.q.shape == (128, 4, 64) and t.k.shape == (128, 1, 64) and not t.paged
    m = wl.mixed_batch(n_prefill=2, chunk=32, max_prefix=64, n_decode=5, max_decode_len=80)
    assert list(m.qo_len) == [32, 32, 1, 1, 1, 1, 1]
    assert m.windows == (128, 0)
    d = wl.long_split_decode(batch=2, kv_len=4096, num_splits=4)
    assert np.isneginf(d.sinks[::8]).all() and (d.sinks[7::8] == 20.0).all()


def test_repermute_keeps_logical_rows():
    w = wl.paged_decode(batch=3, max_len=50)
    w2 = wl.repermute(w, seed=5)
    for b in range(w.batch):
        for j in range(int(w.kv_len[b])):
            p1 = w.page_indices[w.kv_indptr[b] + j // 16]
            p2 = w2.page_indices[w2.kv_indptr[b] + j // 16]
            np.testing.assert_array_equal(w.k[p1, :, j % 16], w2.k[p2, :, j % 16])
