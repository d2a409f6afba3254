"""Seeded synthetic inputs for sink attention (shared by tests, bench, smoke).

This module holds input generation only: random draws, rounding of the drawn
fp32 values to bf16 bit patterns, page-table construction and NaN poisoning of
unused cache slots.  It contains none of the attention arithmetic, imports
nothing from the HIP binding or from the oracle, and needs only numpy.

Recipe (every workload):

* ``np.random.default_rng(seed)``, seed 0 unless stated; a fresh generator per
  workload and a fixed draw order: KV lengths -> prefix lengths -> page
  permutation -> Q -> K -> V -> sinks.
* Q/K/V are fp32 ``standard_normal`` draws rounded to bf16 (round to nearest,
  ties to even), held as uint16 bit patterns.
* Paged caches ([SONAR-INF]: per-request KV pages with page metadata) are
  pools ``[num_pages, Hkv, page_size, D]`` holding exactly the pages the
  requests need plus 1% spare pages; physical page ids are a random
  permutation of the pool, handed out in logical order.  Slots past a
  request's last key and all spare pages hold NaN, so any read of them shows.
* Sinks are fp32, ``normal(0, std)`` per head.

The named workloads follow GPT-OSS attention shapes: 64 query heads sharing 8
KV heads, head_dim 64, page size 16, softmax scale 1/sqrt(64).
"""

from __future__ import annotations

import math
import os
from dataclasses import dataclass, field
from typing import Optional, Sequence, Tuple

import numpy as np

BF16_NAN = np.uint16(0x7FC0)
PAGE_SIZE = 16
HEAD_DIM = 64


def bf16_bits(x) -> np.ndarray:
    """fp32 values -> bf16 bit patterns, round to nearest even; NaN stays NaN."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        r[nan] = BF16_NAN
    return r


def _normal_bf16(rng, shape, chunk=1 << 22) -> np.ndarray:
    """fp32 standard-normal draws rounded to bf16, in chunks of ``chunk``
    values.  Chunk i draws from its own PCG64 stream, seeded with
    (key_i, i) where the keys are one draw of ``rng`` (so the result depends
    only on ``rng``'s state, not on the thread count); the chunks are filled
    by a thread pool, which keeps the multi-GB paged pools quick to build."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    nchunks = max(1, -(-n // chunk))
    keys = rng.integers(0, 1 << 62, size=nchunks)

    def fill(i):
        s = i * chunk
        e = min(n, s + chunk)
        sub = np.random.default_rng([int(keys[i]), i])
        out[s:e] = bf16_bits(sub.standard_normal(e - s, dtype=np.float32))

    if nchunks == 1:
        fill(0)
    else:
        from concurrent.futures import ThreadPoolExecutor
        try:
            cores = len(os.sched_getaffinity(0))
        except AttributeError:          # pragma: no cover
            cores = os.cpu_count() or 1
        with ThreadPoolExecutor(max_workers=max(1, min(16, cores, nchunks))) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


@dataclass
class Workload:
    """One attention call's inputs, host-side.

    ``q``: uint16 ``[total_q, Hq, D]``; ``qo_indptr``: int32 ``[B+1]``.
    Contiguous KV: ``k``/``v`` uint16 ``[total_kv, Hkv, D]``, ``kv_indptr`` row
    offsets.  Paged KV: ``k``/``v`` uint16 ``[num_pages, Hkv, page_size, D]``,
    ``kv_indptr`` offsets into ``page_indices``.  ``kv_len`` int32 ``[B]``.
    ``windows``: the window of each call in the workload (0 = full causal).
    ``num_splits``: KV chunks per request for split decode (None: unsplit).
    """

    name: str
    q: np.ndarray
    qo_indptr: np.ndarray
    k: np.ndarray
    v: np.ndarray
    paged: bool
    kv_indptr: np.ndarray
    kv_len: np.ndarray
    sinks: np.ndarray
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int = HEAD_DIM
    page_indices: Optional[np.ndarray] = None
    page_size: int = PAGE_SIZE
    scale: float = 1.0 / math.sqrt(HEAD_DIM)
    windows: Tuple[int, ...] = (0,)
    num_splits: Optional[int] = None
    decode: bool = False
    meta: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return len(self.kv_len)

    @property
    def total_q(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_pages(self) -> int:
        return int(self.k.shape[0]) if self.paged else 0

    @property
    def qo_len(self) -> np.ndarray:
        return np.diff(self.qo_indptr)


def _page_tables(rng, kv_len, page_size=PAGE_SIZE, spare_frac=0.01):
    """Pages per request, pool size with 1% spare, permuted physical ids."""
    n_pages = (np.asarray(kv_len, dtype=np.int64) + page_size - 1) // page_size
    page_indptr = np.zeros(len(kv_len) + 1, dtype=np.int64)
    page_indptr[1:] = np.cumsum(n_pages)
    needed = int(page_indptr[-1])
    pool = needed + int(math.ceil(needed * spare_frac))
    perm = rng.permutation(pool)
    page_indices = perm[:needed].astype(np.int32)
    return page_indptr.astype(np.int32), page_indices, pool


def _poison_pool(pool_bits, kv_len, page_indptr, page_indices, page_size=PAGE_SIZE):
    """NaN into every slot that holds no live key (tails of last pages, spare pages)."""
    used = np.zeros((pool_bits.shape[0], page_size), dtype=bool)
    for b, length in enumerate(np.asarray(kv_len)):
        length = int(length)
        if length == 0:
            continue
        pages = page_indices[page_indptr[b]: page_indptr[b + 1]]
        used[pages[:-1], :] = True
        used[pages[-1], : length - (len(pages) - 1) * page_size] = True
    # pool layout [num_pages, Hkv, page_size, D]
    mask = ~used
    pool_bits.transpose(0, 2, 1, 3)[mask] = BF16_NAN


def make_paged(name, kv_len, qo_len, num_qo_heads, num_kv_heads, seed=0, sink_std=2.0,
               windows=(0,), num_splits=None, prefix_first=None, rng=None, head_dim=HEAD_DIM,
               sink_overrides=None, decode=False, meta=None) -> Workload:
    """A paged-KV workload.  ``kv_len``/``qo_len`` are per-request arrays (the
    caller drew them from ``rng`` first, keeping the draw order)."""
    rng = np.random.default_rng(seed) if rng is None else rng
    kv_len = np.asarray(kv_len, dtype=np.int32)
    qo_len = np.asarray(qo_len, dtype=np.int32)
    assert np.all(qo_len <= kv_len) and np.all(qo_len >= 1)
    page_indptr, page_indices, pool = _page_tables(rng, kv_len)
    total_q = int(qo_len.sum())
    q = _normal_bf16(rng, (total_q, num_qo_heads, head_dim))
    k = _normal_bf16(rng, (pool, num_kv_heads, PAGE_SIZE, head_dim))
    v = _normal_bf16(rng, (pool, num_kv_heads, PAGE_SIZE, head_dim))
    sinks = rng.normal(0.0, sink_std, size=num_qo_heads).astype(np.float32)
    if sink_overrides is not None:
        sinks = sink_overrides(sinks)
    _poison_pool(k, kv_len, page_indptr, page_indices)
    _poison_pool(v, kv_len, page_indptr, page_indices)
    qo_indptr = np.zeros(len(qo_len) + 1, dtype=np.int32)
    qo_indptr[1:] = np.cumsum(qo_len)
    return Workload(name=name, q=q, qo_indptr=qo_indptr, k=k, v=v, paged=True,
                    kv_indptr=page_indptr, kv_len=kv_len, sinks=sinks,
                    num_qo_heads=num_qo_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
                    page_indices=page_indices, windows=tuple(windows), num_splits=num_splits,
                    decode=decode, meta=dict(meta or {}))


def make_contiguous(name, kv_len, qo_len, num_qo_heads, num_kv_heads, seed=0, sink_std=2.0,
                    windows=(0,), rng=None, head_dim=HEAD_DIM, meta=None) -> Workload:
    """A contiguous-KV workload (K/V rows of every request packed back to back)."""
    rng = np.random.default_rng(seed) if rng is None else rng
    kv_len = np.asarray(kv_len, dtype=np.int32)
    qo_len = np.asarray(qo_len, dtype=np.int32)
    assert np.all(qo_len <= kv_len) and np.all(qo_len >= 1)
    total_q, total_kv = int(qo_len.sum()), int(kv_len.sum())
    q = _normal_bf16(rng, (total_q, num_qo_heads, head_dim))
    k = _normal_bf16(rng, (total_kv, num_kv_heads, head_dim))
    v = _normal_bf16(rng, (total_kv, num_kv_heads, head_dim))
    sinks = rng.normal(0.0, sink_std, size=num_qo_heads).astype(np.float32)
    qo_indptr = np.zeros(len(qo_len) + 1, dtype=np.int32)
    qo_indptr[1:] = np.cumsum(qo_len)
    kv_indptr = np.zeros(len(kv_len) + 1, dtype=np.int32)
    kv_indptr[1:] = np.cumsum(kv_len)
    return Workload(name=name, q=q, qo_indptr=qo_indptr, k=k, v=v, paged=False,
                    kv_indptr=kv_indptr, kv_len=kv_len, sinks=sinks,
                    num_qo_heads=num_qo_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
                    windows=tuple(windows), meta=dict(meta or {}))


# --------------------------------------------------------------------------
# Named workloads (GPT-OSS attention shapes)
# --------------------------------------------------------------------------

def tiny_prefill(seed=0) -> Workload:
    """Batch 1, 4 query heads on 1 KV head, head_dim 64, causal 128 tokens,
    contiguous KV, sinks N(0, 1)."""
    rng = np.random.default_rng(seed)
    return make_contiguous("tiny_prefill", [128], [128], 4, 1, rng=rng, sink_std=1.0)


def paged_decode(seed=0, batch=64, max_len=4096, num_qo_heads=64, num_kv_heads=8) -> Workload:
    """64 requests, one query token each, KV lengths uniform in [1, 4096],
    64/8 heads, page size 16, permuted shared pool, sinks N(0, 2)."""
    rng = np.random.default_rng(seed)
    kv_len = rng.integers(1, max_len + 1, size=batch)
    return make_paged("paged_decode", kv_len, np.ones(batch), num_qo_heads, num_kv_heads,
                      rng=rng, decode=True)


def skewed_decode(seed=0, batch=64, long_len=131072, max_len=4096, num_qo_heads=64, num_kv_heads=8) -> Workload:
    """A decode batch with one very long request: request 0 holds 131072 keys,
    the other 63 hold KV lengths uniform in [1, 4096]; 64/8 heads, page size
    16, permuted shared pool, sinks N(0, 2).  A split into a fixed number of
    chunks per request leaves the long request to a few workgroups; the
    balanced split does not."""
    rng = np.random.default_rng(seed)
    kv_len = rng.integers(1, max_len + 1, size=batch)
    kv_len[0] = long_len
    return make_paged("skewed_decode", kv_len, np.ones(batch), num_qo_heads, num_kv_heads, rng=rng, decode=True)


def causal_prefill(seed=0, batch=4, seq=8192, num_qo_heads=64, num_kv_heads=8) -> Workload:
    """4 sequences of 8192 tokens, full causal, 64/8 heads, contiguous KV,
    scale 1/sqrt(64), sinks N(0, 2)."""
    rng = np.random.default_rng(seed)
    return make_contiguous("causal_prefill", [seq] * batch, [seq] * batch, num_qo_heads,
                           num_kv_heads, rng=rng)


def outlier_sinks(sinks: np.ndarray) -> np.ndarray:
    """Every KV group mixes a -inf sink (head % 8 == 0), a +20 sink
    (head % 8 == 7) and ordinary N(0, 2) sinks."""
    s = sinks.copy()
    h = np.arange(len(s))
    s[h % 8 == 0] = -np.inf
    s[h % 8 == 7] = 20.0
    return s


def long_split_decode(seed=0, batch=8, kv_len=131072, num_splits=16, num_qo_heads=64,
                      num_kv_heads=8) -> Workload:
    """8 requests with 131072 cached keys, one query token each, KV split into
    16 chunks (sink in chunk 0 only) then merged; paged, page size 16; sinks
    N(0, 2) with -inf and +20 outliers."""
    rng = np.random.default_rng(seed)
    lens = np.full(batch, kv_len)
    return make_paged("long_split_decode", lens, np.ones(batch), num_qo_heads, num_kv_heads,
                      rng=rng, num_splits=num_splits, sink_overrides=outlier_sinks,
                      decode=True)


def mixed_batch(seed=0, n_prefill=16, chunk=512, max_prefix=16384, n_decode=240,
                max_decode_len=16384, num_qo_heads=64, num_kv_heads=8) -> Workload:
    """One call over 16 prefill chunks of 512 tokens on prefixes uniform in
    [0, 16384] followed by 240 decode rows with KV lengths uniform in
    [1, 16384]; paged, page size 16; calls alternate a 128-token sliding window
    and full causal."""
    rng = np.random.default_rng(seed)
    dec_len = rng.integers(1, max_decode_len + 1, size=n_decode)
    prefix = rng.integers(0, max_prefix + 1, size=n_prefill)
    kv_len = np.concatenate([prefix + chunk, dec_len])
    qo_len = np.concatenate([np.full(n_prefill, chunk), np.ones(n_decode, dtype=np.int64)])
    return make_paged("mixed_batch", kv_len, qo_len, num_qo_heads, num_kv_heads, rng=rng,
                      windows=(128, 0), meta={"n_prefill": n_prefill, "n_decode": n_decode})


def verify_decode(seed=0, batch=64, max_len=4096, min_rows=2, max_rows=8, num_qo_heads=64,
                  num_kv_heads=8) -> Workload:
    """A speculative verify step: 64 requests with KV lengths uniform in
    [max_rows, 4096] (the proposed tokens' keys already cached), each scoring
    a number of query rows uniform in [2, 8]; 64/8 heads, paged, page size 16."""
    rng = np.random.default_rng(seed)
    kv_len = rng.integers(max_rows, max_len + 1, size=batch)
    qo_len = rng.integers(min_rows, max_rows + 1, size=batch)
    return make_paged("verify_decode", kv_len, qo_len, num_qo_heads, num_kv_heads, rng=rng,
                      meta={"max_rows": max_rows})


def verify_tree(seed=0) -> Workload:
    """The verify batch of ``verify_decode`` with a random draft tree per
    request (its custom mask in ``meta["masks"]``)."""
    w = verify_decode(seed)
    rng = np.random.default_rng(seed + 1)
    w.meta["masks"] = tree_masks(rng, w.kv_len, np.diff(w.qo_indptr))
    return w


def tree_masks(rng, kv_len, qo_len, chain: bool = False):
    """Draft-tree masks for a verify step (EAGLE-style tree attention): the
    n_q draft tokens of request b are the last n_q keys of its cache and form
    a tree (node i's parent a uniformly drawn earlier node, or the prefix);
    row t sees every prefix key and the draft keys on its own root path.
    ``chain`` makes every node's parent the previous one (a causal chain).
    Returns one boolean ``[n_q, n_k]`` array per request."""
    masks = []
    for n_k, n_q in zip(np.asarray(kv_len), np.asarray(qo_len)):
        n_k, n_q = int(n_k), int(n_q)
        parent = [i - 1 if chain else int(rng.integers(-1, i)) for i in range(n_q)]
        m = np.zeros((n_q, n_k), dtype=bool)
        base = n_k - n_q
        m[:, :max(base, 0)] = True
        for t in range(n_q):
            i = t
            while i >= 0:
                if base + i >= 0:
                    m[t, base + i] = True
                i = parent[i]
        masks.append(m)
    return masks


def pack_masks(masks):
    """Bit-pack boolean masks for the library: request b's ``[n_q, n_k]`` mask
    flattened row-major, bit i of the flat index in byte i // 8 at bit i % 8
    (little-endian), each request starting on a whole byte.  Returns
    ``(bits uint8 [nbytes], indptr int32 [B+1])`` with byte offsets."""
    chunks, indptr = [], [0]
    for m in masks:
        packed = np.packbits(np.asarray(m, dtype=bool).reshape(-1), bitorder="little")
        chunks.append(packed)
        indptr.append(indptr[-1] + len(packed))
    bits = np.concatenate(chunks) if chunks else np.zeros(0, dtype=np.uint8)
    return bits.astype(np.uint8), np.asarray(indptr, dtype=np.int32)


NAMED = {
    "tiny_prefill": tiny_prefill,
    "paged_decode": paged_decode,
    "skewed_decode": skewed_decode,
    "causal_prefill": causal_prefill,
    "long_split_decode": long_split_decode,
    "mixed_batch": mixed_batch,
    "verify_decode": verify_decode,
    "verify_tree": verify_tree,
}


# --------------------------------------------------------------------------
# Structured probes for bit-exact index checks
# --------------------------------------------------------------------------

def value_code(pos: np.ndarray, dim: np.ndarray) -> np.ndarray:
    """Integer code of logical key ``pos`` at dimension ``dim``: exact in bf16
    (|code| <= 254), and rows of nearby positions differ."""
    return (((pos[..., None] + 31 * dim[None, :] + 7 * (pos[..., None] // 509)) % 509) - 254
            ).astype(np.float32)


def one_hot_probe(base: Workload, targets: Sequence[Sequence[int]], hot=7.5) -> Workload:
    """Rewrite a paged workload so that, for request ``b``, the keys listed in
    ``targets[b]`` score +60 and every other live key scores -60 against an
    all-ones query (scale 1/8, D = 64), with every sink at -inf; each V row
    holds the integer code of its logical position.  exp(-120) underflows to 0
    in fp32, so each softmax range with one target returns that target's V
    row exactly."""
    assert base.paged
    w = Workload(**{**base.__dict__})
    d = base.head_dim
    w.q = np.full(base.q.shape, bf16_bits(np.float32(1.0)), dtype=np.uint16)
    k = base.k.copy()
    v = base.v.copy()
    dims = np.arange(d)
    for b in range(base.batch):
        length = int(base.kv_len[b])
        pos = np.arange(length)
        page = base.page_indices[base.kv_indptr[b] + pos // base.page_size]
        slot = pos % base.page_size
        hotmask = np.isin(pos, np.asarray(targets[b], dtype=np.int64))
        kval = np.where(hotmask, hot, -hot).astype(np.float32)
        kb = bf16_bits(np.broadcast_to(kval[:, None], (length, d)))
        vb = bf16_bits(value_code(pos, dims))
        for g in range(base.num_kv_heads):
            k[page, g, slot, :] = kb
            v[page, g, slot, :] = vb
    w.k, w.v = k, v
    w.sinks = np.full(base.num_qo_heads, -np.inf, dtype=np.float32)
    w.name = base.name + "+onehot"
    return w


def zero_query_probe(base: Workload) -> Workload:
    """All-zero queries and -inf sinks: every visible score is 0, so each
    softmax range's log-sum-exp is ln(number of keys in it)."""
    w = Workload(**{**base.__dict__})
    w.q = np.zeros_like(base.q)
    w.sinks = np.full(base.num_qo_heads, -np.inf, dtype=np.float32)
    w.name = base.name + "+zeroq"
    return w


def repermute(base: Workload, seed: int) -> Workload:
    """Same logical KV under a different physical page permutation."""
    assert base.paged
    rng = np.random.default_rng(seed)
    pool = base.num_pages
    perm = rng.permutation(pool).astype(np.int32)
    # physical page x moves to perm[x]
    k = np.full_like(base.k, BF16_NAN)
    v = np.full_like(base.v, BF16_NAN)
    k[perm] = base.k
    v[perm] = base.v
    w = Workload(**{**base.__dict__})
    w.k, w.v = k, v
    w.page_indices = perm[base.page_indices]
    w.name = base.name + f"+perm{seed}"
    return w
