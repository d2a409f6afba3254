"""Plain fp64 reference for sink attention (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may use this module.  It is deliberately slow and
obvious: numpy fp64 matrix products and ``exp``, no blocking beyond splitting
query rows into groups to bound memory, no fusion, no reordering of the
definition.

What is computed ([DAY0-SINK], [DAY0-HOPPER]; see ``oracle/__init__.py``):
for request ``b`` with ``n_q`` query rows and ``n_k`` cached keys, query row
``t`` and query head ``h``::

    p      = n_k - n_q + t                       (bottom-right causal position)
    g      = h // G,  G = Hq / Hkv               (GQA head mapping)
    V(p)   = {j : lo <= j <= p},  lo = max(0, p - W + 1) if W > 0 else 0
    s_j    = scale * <q[t, h], k[j, g]>          for j in V(p)
    Z      = exp(sink[h]) + sum_{j in V(p)} exp(s_j)
    o[t,h] = sum_{j in V(p)} exp(s_j) / Z * v[j, g]
    lse    = ln Z

i.e. ordinary softmax attention with one extra virtual key whose logit is the
head's sink and whose value row is zero.

Readings of points the pages leave open (each enforced by a test):

* R1  the lost sink formula: the sink is one more logit in the softmax
      denominator with no value row.  A constant added to every Q.K product
      would cancel in the softmax, and the pages start the running max at the
      sink value, so the sink is compared with the (scaled) logits directly.
* R2  the softmax scale multiplies only q.k, never the sink.
* R3  the pages start the scale ``d`` at 1: with ``m = sink`` that 1 is the
      sink's own mass exp(sink - m).
* R4  under a KV split the sink enters exactly once per row, in chunk 0.
* R5  GQA mapping g = h // (Hq / Hkv).
* R6  causal alignment is bottom-right: row t of a request sits at position
      n_k - n_q + t and its own key is already cached.
* R7  a window W > 0 counts visible keys including the query's own position;
      W = 0 means unlimited (plain causal).
* R9  split rule: n_pages = ceil(L / page_size), ppc = ceil(n_pages / S),
      chunk c covers pages [c*ppc, min((c+1)*ppc, n_pages)), i.e. tokens
      [c*ppc*page_size, min((c+1)*ppc*page_size, L)); chunks may be empty.
* R10 lse is the natural log of Z and includes the sink.
* R14 no visible key: o = 0 and lse = sink; sink = +inf: o = 0, lse = +inf;
      sink = -inf and no visible key: o = 0, lse = -inf.
* R24 balanced split of a decode batch (one query row per request, at
      n_k - 1): the keys a row reads are [lo, n_k), lo = max(0, n_k - W)
      under a window W > 0, else 0, i.e. its live pages floor(lo / 16) ..
      ceil(n_k / 16) - 1.  The requests' live pages, request after request,
      form one list of T pages; segment s of N holds the list positions
      [floor(s T / N), floor((s + 1) T / N)).  A request's piece in a
      segment is the part of its live pages there (its keys clipped to
      [lo, n_k)); each request's first piece carries the sink.  A request
      with no key has one empty piece (o = 0, lse = sink).
* R18 custom masks (a draft tree verified in one step): when a boolean mask
      ``[n_q, n_k]`` is given for a request, key j is visible to row t
      exactly when ``mask[t, j]``; it replaces the causal rule and the window,
      and the sink is unchanged (it is no key and is never masked).
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Optional

import numpy as np

_NEG_INF = -math.inf


def widen_bf16(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact fp64 values.

    A bf16 number is the upper half of an IEEE binary32, so shifting the 16
    bits into the top of a 32-bit word gives the same value exactly.
    """
    u = np.asarray(bits, dtype=np.uint16)
    return (u.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _as_f64(x) -> np.ndarray:
    a = np.asarray(x)
    if a.dtype == np.uint16:
        return widen_bf16(a)
    return a.astype(np.float64)


@dataclass
class KVCache:
    """Where the keys and values of every request live.

    Contiguous:  ``k``/``v`` are ``[total_kv, Hkv, D]``; request ``b`` owns
    rows ``kv_indptr[b] : kv_indptr[b+1]``.

    Paged ([SONAR-INF]: per-request KV pages plus page metadata):  ``k``/``v``
    are pools ``[num_pages, Hkv, page_size, D]``; request ``b``'s logical key
    ``j`` is slot ``j % page_size`` of physical page
    ``page_indices[kv_indptr[b] + j // page_size]``; ``kv_len[b]`` gives the
    number of keys.

    ``k`` and ``v`` may hold bf16 bit patterns (uint16) or floats.
    """

    k: np.ndarray
    v: np.ndarray
    kv_indptr: np.ndarray
    paged: bool = False
    page_indices: Optional[np.ndarray] = None
    kv_len: Optional[np.ndarray] = None
    page_size: int = 16

    def length(self, b: int) -> int:
        if self.paged:
            return int(self.kv_len[b])
        return int(self.kv_indptr[b + 1] - self.kv_indptr[b])

    def rows(self, b: int, g: int, lo: int = 0, hi: Optional[int] = None):
        """Logical keys ``lo..hi-1`` of request ``b``, KV head ``g`` as fp64."""
        n = self.length(b)
        hi = n if hi is None else hi
        if hi <= lo:
            d = self.k.shape[-1]
            return np.zeros((0, d)), np.zeros((0, d))
        if self.paged:
            j = np.arange(lo, hi)
            page = np.asarray(self.page_indices)[int(self.kv_indptr[b]) + j // self.page_size]
            slot = j % self.page_size
            kk = self.k[page, g, slot, :]
            vv = self.v[page, g, slot, :]
        else:
            base = int(self.kv_indptr[b])
            kk = self.k[base + lo: base + hi, g, :]
            vv = self.v[base + lo: base + hi, g, :]
        return _as_f64(kk), _as_f64(vv)


def visible_range(n_q: int, n_k: int, t, window: int):
    """Keys visible to query row ``t`` (R6, R7): returns inclusive ``(lo, p)``."""
    t = np.asarray(t)
    p = n_k - n_q + t
    if window > 0:
        lo = np.maximum(0, p - window + 1)
    else:
        lo = np.zeros_like(p)
    return lo, p


def _softmax_with_sink(s: np.ndarray, vis: np.ndarray, sink: np.ndarray, vals: np.ndarray):
    """One block of rows: logits ``s`` [R, n], visibility ``vis`` [R, n],
    sink logit per row [R], value rows [n, D] -> (o [R, D], lse [R]).

    Max subtraction is only for fp64 range safety; Z is the definition's.
    """
    s = np.where(vis, s, _NEG_INF)
    row_max = s.max(axis=1) if s.shape[1] else np.full(s.shape[0], _NEG_INF)
    m = np.maximum(sink, row_max)
    o = np.zeros((s.shape[0], vals.shape[1]))
    lse = np.empty(s.shape[0])
    fin = np.isfinite(m)
    # rows with M = -inf: no visible key and sink = -inf; M = +inf: sink = +inf
    lse[~fin] = m[~fin]
    if fin.any():
        sf, mf = s[fin], m[fin]
        e = np.exp(sf - mf[:, None])            # exp(-inf) = 0 on masked keys
        e_sink = np.exp(sink[fin] - mf)
        z = e_sink + e.sum(axis=1)
        o[fin] = (e @ vals) / z[:, None]
        lse[fin] = mf + np.log(z)
    return o, lse


def _attend_request_group(q_b, kv: KVCache, b: int, g: int, heads, sinks, scale, window, row_block,
                          mask=None):
    """All query rows of request ``b`` for the query heads ``heads`` that read
    KV head ``g``.  ``q_b`` is fp64 [n_q, Hq, D]; ``mask`` (optional, bool
    [n_q, n_k]) replaces the causal / window rule (R18)."""
    n_q = q_b.shape[0]
    n_k = kv.length(b)
    d = q_b.shape[2]
    gq = len(heads)
    out = np.zeros((n_q, gq, d))
    lse = np.empty((n_q, gq))
    for r0 in range(0, n_q, row_block):
        r1 = min(n_q, r0 + row_block)
        t = np.arange(r0, r1)
        if mask is None:
            lo, p = visible_range(n_q, n_k, t, window)
            k_lo = int(max(0, lo.min()))
            k_hi = int(min(n_k, p.max() + 1))
        else:
            k_lo, k_hi = 0, n_k
        kk, vv = kv.rows(b, g, k_lo, max(k_lo, k_hi))
        j = np.arange(k_lo, k_lo + kk.shape[0])
        if mask is None:
            vis = (j[None, :] >= lo[:, None]) & (j[None, :] <= p[:, None])   # [rows, n]
        else:
            vis = np.asarray(mask, dtype=bool)[r0:r1, k_lo:k_lo + kk.shape[0]]
        for i, h in enumerate(heads):
            s = scale * (q_b[r0:r1, h, :] @ kk.T)
            sink = np.full(r1 - r0, sinks[h])
            o_blk, l_blk = _softmax_with_sink(s, vis, sink, vv)
            out[r0:r1, i, :] = o_blk
            lse[r0:r1, i] = l_blk
    return out, lse


def _sinks_f64(sinks, hq):
    if sinks is None:                 # no sinks: plain softmax attention (sink = -inf)
        return np.full(hq, _NEG_INF)
    s = np.asarray(sinks, dtype=np.float64)
    assert s.shape == (hq,)
    return s


def sink_attention_ref(q, qo_indptr, kv: KVCache, sinks, scale: float, window: int = 0,
                       workers: int = 1, row_block: int = 256, custom_mask=None):
    """Unsplit sink attention, the plain definition ([DAY0-SINK], [DAY0-HOPPER]).

    ``q`` is ``[total_q, Hq, D]`` (bf16 bits or floats), ``qo_indptr`` the
    ``[B+1]`` row offsets of each request.  ``custom_mask`` (optional) is one
    boolean ``[n_q, n_k]`` array per request that replaces the causal rule
    (R18; ``window`` must then be 0).  Returns fp64 ``out [total_q, Hq, D]``
    and ``lse [total_q, Hq]`` (natural log, sink included).  ``workers`` > 1
    spreads (request, KV head) units over threads, BLAS held to one thread.
    """
    qf = _as_f64(q)
    total_q, hq, d = qf.shape
    hkv = kv.k.shape[1]
    assert hq % hkv == 0
    assert custom_mask is None or window == 0
    group = hq // hkv
    sk = _sinks_f64(sinks, hq)
    qo_indptr = np.asarray(qo_indptr, dtype=np.int64)
    batch = len(qo_indptr) - 1
    out = np.zeros((total_q, hq, d))
    lse = np.empty((total_q, hq))

    def unit(bg):
        b, g = bg
        r0, r1 = int(qo_indptr[b]), int(qo_indptr[b + 1])
        if r1 == r0:
            return
        heads = list(range(g * group, (g + 1) * group))
        mask = None if custom_mask is None else custom_mask[b]
        o, l = _attend_request_group(qf[r0:r1], kv, b, g, heads, sk, scale, window, row_block, mask)
        out[r0:r1, g * group:(g + 1) * group, :] = o
        lse[r0:r1, g * group:(g + 1) * group] = l

    units = [(b, g) for b in range(batch) for g in range(hkv)]
    _run_units(unit, units, workers)
    return out, lse


def _run_units(fn, units, workers):
    if workers <= 1:
        for u in units:
            fn(u)
        return
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:                     # pragma: no cover
        threadpool_limits = None
    limiter = threadpool_limits(limits=1) if threadpool_limits else None
    try:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(fn, units))
    finally:
        if limiter is not None:
            limiter.restore_original_limits()


def split_bounds_ref(kv_len, num_splits: int, page_size: int = 16) -> np.ndarray:
    """Token range ``[lo, hi)`` of every chunk of every request (reading R9).

    Chunks are whole pages: a request of L keys has ceil(L / page_size)
    pages, each chunk takes ceil(pages / S) of them in order, and the last
    chunks may be short or empty.  Returns int64 ``[B, S, 2]``.
    """
    kv_len = np.asarray(kv_len, dtype=np.int64)
    out = np.zeros((len(kv_len), num_splits, 2), dtype=np.int64)
    for b, length in enumerate(kv_len):
        n_pages = -(-int(length) // page_size)
        per_chunk = -(-n_pages // num_splits)
        for c in range(num_splits):
            first = min(c * per_chunk, n_pages)
            last = min((c + 1) * per_chunk, n_pages)
            out[b, c, 0] = min(first * page_size, int(length))
            out[b, c, 1] = min(last * page_size, int(length))
    return out


def split_partials_ref(q, kv: KVCache, sinks, scale: float, num_splits: int, window: int = 0,
                       sink_in_every_chunk: bool = False, workers: int = 1, qo_indptr=None,
                       custom_mask=None):
    """Per-chunk partial results of a decode step ([DAY0-SINK]: the KV sequence
    is split into blocks and only the first block carries the sink).

    Without ``qo_indptr``, ``q`` is ``[B, Hq, D]``: one query per request, at
    position ``kv_len[b] - 1``.  With ``qo_indptr`` ([B+1] row offsets), ``q``
    is ``[total_q, Hq, D]`` and request ``b`` owns rows ``qo_indptr[b]`` ..
    ``qo_indptr[b+1] - 1``; its row ``t`` sits at ``kv_len[b] - n_q + t`` (R6),
    as in a speculative-decoding verify step ([SONAR-INF]: the target model
    scores several proposed tokens in one pass).  For chunk ``c`` with keys
    ``[lo_c, hi_c)`` (R9, the request's pages, the same for all its rows)
    intersected with the row's visible range (R7), the chunk is attended on
    its own, its softmax seeded with the sink only when ``c == 0``.  Returns
    ``o_part [rows, Hq, S, D]`` (each chunk normalised by its own Z_c) and
    ``lse_part [rows, Hq, S]`` = ln Z_c, rows being B or total_q.  An empty
    chunk gives o = 0 with lse = -inf, or lse = sink for chunk 0.

    ``custom_mask`` (with ``qo_indptr``): one boolean ``[n_q, n_k]`` array per
    request replacing the row's visible range (R18); the chunks stay the
    request's pages.

    ``sink_in_every_chunk`` exists only as the negative control for tests.
    """
    qf = _as_f64(q)
    rows, hq, d = qf.shape
    assert custom_mask is None or (qo_indptr is not None and window == 0)
    hkv = kv.k.shape[1]
    group = hq // hkv
    sk = _sinks_f64(sinks, hq)
    if qo_indptr is None:
        qo_indptr = np.arange(rows + 1, dtype=np.int64)
    qo_indptr = np.asarray(qo_indptr, dtype=np.int64)
    batch = len(qo_indptr) - 1
    assert int(qo_indptr[-1]) == rows
    kv_len = np.array([kv.length(b) for b in range(batch)])
    bounds = split_bounds_ref(kv_len, num_splits, kv.page_size)
    o_part = np.zeros((rows, hq, num_splits, d))
    lse_part = np.empty((rows, hq, num_splits))

    def unit(bg):
        b, g = bg
        n_k = int(kv_len[b])
        r0, r1 = int(qo_indptr[b]), int(qo_indptr[b + 1])
        for t in range(r1 - r0):
            if custom_mask is None:
                lo_vis, p = visible_range(r1 - r0, n_k, t, window)
                lo_vis, p = int(lo_vis), int(p)
            else:
                lo_vis, p = 0, n_k - 1
            for c in range(num_splits):
                lo = max(int(bounds[b, c, 0]), lo_vis)
                hi = min(int(bounds[b, c, 1]), p + 1)
                kk, vv = kv.rows(b, g, lo, max(lo, hi))
                for h in range(g * group, (g + 1) * group):
                    seeded = (c == 0) or sink_in_every_chunk
                    sink = np.array([sk[h] if seeded else _NEG_INF])
                    s = scale * (kk @ qf[r0 + t, h, :])[None, :]
                    if custom_mask is None:
                        vis = np.ones_like(s, dtype=bool)
                    else:
                        vis = np.asarray(custom_mask[b], dtype=bool)[t, lo:lo + kk.shape[0]][None, :]
                    o, l = _softmax_with_sink(s, vis, sink, vv)
                    o_part[r0 + t, h, c, :] = o[0]
                    lse_part[r0 + t, h, c] = l[0]

    _run_units(unit, [(b, g) for b in range(batch) for g in range(hkv)], workers)
    return o_part, lse_part


def live_pages_ref(kv_len, window: int = 0, page_size: int = 16):
    """The pages one query row at position n_k - 1 reads (R24): keys
    [lo, n_k) with lo = max(0, n_k - W) for a window W > 0, else 0, on pages
    floor(lo / page_size) .. ceil(n_k / page_size) - 1.  Returns int64
    arrays (first_page, n_pages, lo), one entry per request."""
    n_k = np.asarray(kv_len, dtype=np.int64)
    lo = np.maximum(0, n_k - window) if window > 0 else np.zeros_like(n_k)
    first = lo // page_size
    end = -(-n_k // page_size)
    return first, np.maximum(0, end - first), lo


def balanced_pieces_ref(kv_len, num_segments: int, window: int = 0, page_size: int = 16):
    """The balanced split of a decode batch into ``num_segments`` segments
    (R24; [DAY0-SINK]: attention split into blocks along the KV sequence).
    Returns one list per request of pieces ``(segment, lo_token, hi_token)``
    in key order; a request with no key gets ``[(-1, 0, 0)]``."""
    n_k = np.asarray(kv_len, dtype=np.int64)
    first, n_pages, lo = live_pages_ref(n_k, window, page_size)
    total = int(n_pages.sum())
    starts = [(s * total) // num_segments for s in range(num_segments + 1)]
    pieces = []
    pos = 0                                   # list position of the request's first live page
    for b in range(len(n_k)):
        mine = []
        for s in range(num_segments):
            a = max(pos, starts[s])
            e = min(pos + int(n_pages[b]), starts[s + 1])
            if a >= e:
                continue
            p0 = int(first[b]) + (a - pos)    # the request's own page numbers
            p1 = int(first[b]) + (e - pos)
            mine.append((s, max(p0 * page_size, int(lo[b])), min(p1 * page_size, int(n_k[b]))))
        pieces.append(mine if mine else [(-1, 0, 0)])
        pos += int(n_pages[b])
    return pieces


def pieces_partials_ref(q, kv: KVCache, sinks, scale: float, pieces, window: int = 0,
                        sink_in_every_piece: bool = False):
    """Partial results of a decode step split into arbitrary pieces of each
    request's keys ([DAY0-SINK]: only the first block carries the sink).
    ``q`` is ``[B, Hq, D]`` (one query row per request, at ``kv_len[b] - 1``);
    ``pieces[b]`` lists ``(segment, lo, hi)`` token ranges in key order (as
    ``balanced_pieces_ref`` returns).  Each piece is attended on its own,
    over its keys inside the row's visible range (R7), its softmax seeded
    with the sink only when it is the request's first piece.  Returns one
    ``(o [Hq, n_pieces, D], lse [Hq, n_pieces])`` pair per request, each
    piece normalised by its own denominator (``merge_ref`` combines them).

    ``sink_in_every_piece`` exists only as the negative control for tests."""
    qf = _as_f64(q)
    batch, hq, d = qf.shape
    hkv = kv.k.shape[1]
    group = hq // hkv
    sk = _sinks_f64(sinks, hq)
    out = []
    for b in range(batch):
        n_k = kv.length(b)
        lo_vis, p = visible_range(1, n_k, 0, window)
        lo_vis, p = int(lo_vis), int(p)
        o_b = np.zeros((hq, len(pieces[b]), d))
        l_b = np.empty((hq, len(pieces[b])))
        for i, (_seg, lo, hi) in enumerate(pieces[b]):
            a, e = max(lo, lo_vis), min(hi, p + 1)
            for g in range(hkv):
                kk, vv = kv.rows(b, g, a, max(a, e))
                for h in range(g * group, (g + 1) * group):
                    seeded = i == 0 or sink_in_every_piece
                    sink = np.array([sk[h] if seeded else _NEG_INF])
                    s_row = scale * (kk @ qf[b, h, :])[None, :]
                    o, l = _softmax_with_sink(s_row, np.ones_like(s_row, dtype=bool), sink, vv)
                    o_b[h, i, :] = o[0]
                    l_b[h, i] = l[0]
        out.append((o_b, l_b))
    return out


def merge_ref(o_part, lse_part):
    """Combine chunk partials into the full softmax (log-sum-exp merge).

    Each chunk's o_c is its own weighted mean with total mass exp(lse_c); the
    union's mass is the sum of the masses, so
    o = sum_c exp(lse_c) o_c / sum_c exp(lse_c) and lse = ln sum_c exp(lse_c),
    evaluated after subtracting M = max_c lse_c.  ``o_part [..., S, D]``,
    ``lse_part [..., S]``.
    """
    o_part = np.asarray(o_part, dtype=np.float64)
    lse_part = np.asarray(lse_part, dtype=np.float64)
    m = lse_part.max(axis=-1)
    out = np.zeros(o_part.shape[:-2] + o_part.shape[-1:])
    lse = np.array(m, dtype=np.float64, copy=True)
    fin = np.isfinite(m)
    if fin.any():
        w = np.exp(lse_part[fin] - m[fin][..., None])            # [..., S]
        wsum = w.sum(axis=-1)
        out[fin] = (w[..., None] * o_part[fin]).sum(axis=-2) / wsum[..., None]
        lse[fin] = m[fin] + np.log(wsum)
    pos_inf = np.isposinf(m)
    if pos_inf.any():
        # only a +inf sink produces lse = +inf; its chunk carries o = 0
        w = np.isposinf(lse_part[pos_inf]).astype(np.float64)
        out[pos_inf] = (w[..., None] * o_part[pos_inf]).sum(axis=-2) / w.sum(axis=-1)[..., None]
    return out, lse


def attention_weights_ref(q_row, keys, sink: float, scale: float):
    """Attention weights of one query row over ``keys`` [n, D] plus the sink's
    own weight: returns (p [n], p_sink).  For the mass-conservation pin."""
    q = _as_f64(q_row)
    k = _as_f64(keys)
    s = scale * (k @ q)
    m = max(sink, s.max() if s.size else _NEG_INF)
    e = np.exp(s - m)
    e_sink = math.exp(sink - m)
    z = e_sink + e.sum()
    return e / z, e_sink / z


def default_workers() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:                  # pragma: no cover
        return os.cpu_count() or 1
