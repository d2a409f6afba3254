"""Pure-Python brute force of sink attention, written from the definition
(Perplexity blog "GPT-OSS on day 0", section "Kernels for GPT-OSS > Sink
attention": the per-head sink is one more term of the softmax denominator).

Independent of ``oracle/``: its own gather, its own causal/window rule, no
max subtraction, ``math.fsum`` for every sum.  Used only on tiny inputs to pin
the oracle.  ``mp_attention`` repeats it in 50-digit mpmath arithmetic.
"""

import math


def _key_rows(kvspec, b, g):
    """List of (k_row, v_row) of request b, KV head g, in logical order."""
    if kvspec["paged"]:
        rows = []
        start = kvspec["page_indptr"][b]
        for j in range(kvspec["kv_len"][b]):
            page = kvspec["page_indices"][start + j // kvspec["page_size"]]
            slot = j % kvspec["page_size"]
            rows.append((list(kvspec["k"][page][g][slot]), list(kvspec["v"][page][g][slot])))
        return rows
    lo, hi = kvspec["kv_indptr"][b], kvspec["kv_indptr"][b + 1]
    return [(list(kvspec["k"][r][g]), list(kvspec["v"][r][g])) for r in range(lo, hi)]


def brute_attention(q, qo_indptr, kvspec, sinks, scale, window, num_kv_heads):
    """Returns (out, lse) as nested lists: out[row][head][dim], lse[row][head]."""
    n_heads = len(sinks)
    group = n_heads // num_kv_heads
    out, lse = [], []
    for b in range(len(qo_indptr) - 1):
        n_q = qo_indptr[b + 1] - qo_indptr[b]
        for t in range(n_q):
            row = qo_indptr[b] + t
            o_row, l_row = [], []
            for h in range(n_heads):
                g = h // group
                keys = _key_rows(kvspec, b, g)
                n_k = len(keys)
                pos = n_k - n_q + t
                first = max(0, pos - window + 1) if window > 0 else 0
                weights, vals = [], []
                for j in range(first, pos + 1):
                    kr, vr = keys[j]
                    s = scale * math.fsum(a * c for a, c in zip(q[row][h], kr))
                    weights.append(math.exp(s))
                    vals.append(vr)
                z = math.fsum(weights + [math.exp(sinks[h])])
                d = len(q[row][h])
                o_row.append([math.fsum(w * v[i] for w, v in zip(weights, vals)) / z for i in range(d)])
                l_row.append(math.log(z))
            out.append(o_row)
            lse.append(l_row)
    return out, lse


def mp_attention(q, qo_indptr, kvspec, sinks, scale, window, num_kv_heads, dps=50):
    import mpmath
    mpmath.mp.dps = dps
    n_heads = len(sinks)
    group = n_heads // num_kv_heads
    out, lse = [], []
    for b in range(len(qo_indptr) - 1):
        n_q = qo_indptr[b + 1] - qo_indptr[b]
        for t in range(n_q):
            row = qo_indptr[b] + t
            o_row, l_row = [], []
            for h in range(n_heads):
                g = h // group
                keys = _key_rows(kvspec, b, g)
                n_k = len(keys)
                pos = n_k - n_q + t
                first = max(0, pos - window + 1) if window > 0 else 0
                z = mpmath.exp(mpmath.mpf(sinks[h])) if sinks[h] != -math.inf else mpmath.mpf(0)
                acc = [mpmath.mpf(0)] * len(q[row][h])
                for j in range(first, pos + 1):
                    kr, vr = keys[j]
                    s = mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(a) * mpmath.mpf(c) for a, c in zip(q[row][h], kr))
                    e = mpmath.exp(s)
                    z += e
                    acc = [a + e * mpmath.mpf(v) for a, v in zip(acc, vr)]
                o_row.append([float(a / z) for a in acc])
                l_row.append(float(mpmath.log(z)))
            out.append(o_row)
            lse.append(l_row)
    return out, lse


def brute_split_partials(q, qo_indptr, kvspec, sinks, scale, window, num_kv_heads, num_splits):
    """Chunk partials of every query row, from the definition: request b's
    n_pages = ceil(L / page_size) pages are dealt out in order, ceil(n_pages /
    S) to a chunk; chunk c attends to its own keys that the row can see, with
    the sink's mass only in chunk 0.  Returns (o_part[row][head][c][dim],
    lse_part[row][head][c]); a chunk with no mass gives o = 0, lse = -inf."""
    n_heads = len(sinks)
    group = n_heads // num_kv_heads
    ps = kvspec["page_size"]
    o_part, lse_part = [], []
    for b in range(len(qo_indptr) - 1):
        n_q = qo_indptr[b + 1] - qo_indptr[b]
        n_k = kvspec["kv_len"][b]
        n_pages = -(-n_k // ps)
        per = -(-n_pages // num_splits)
        for t in range(n_q):
            row = qo_indptr[b] + t
            pos = n_k - n_q + t
            first = max(0, pos - window + 1) if window > 0 else 0
            o_row, l_row = [], []
            for h in range(n_heads):
                keys = _key_rows(kvspec, b, h // group)
                o_h, l_h = [], []
                for c in range(num_splits):
                    weights, vals = [], []
                    for j in range(n_k):
                        if not (c * per <= j // ps < (c + 1) * per) or not (first <= j <= pos):
                            continue
                        kr, vr = keys[j]
                        weights.append(math.exp(scale * math.fsum(a * e for a, e in zip(q[row][h], kr))))
                        vals.append(vr)
                    z = math.fsum(weights + ([math.exp(sinks[h])] if c == 0 else []))
                    d = len(q[row][h])
                    if z == 0.0:
                        o_h.append([0.0] * d)
                        l_h.append(-math.inf)
                    else:
                        o_h.append([math.fsum(w * v[i] for w, v in zip(weights, vals)) / z for i in range(d)])
                        l_h.append(math.log(z))
                o_row.append(o_h)
                l_row.append(l_h)
            o_part.append(o_row)
            lse_part.append(l_row)
    return o_part, lse_part


def brute_attention_masked(q, qo_indptr, kvspec, sinks, scale, masks, num_kv_heads):
    """Like brute_attention, with row t of request b seeing key j exactly when
    masks[b][t][j] (a custom mask replaces the causal rule)."""
    n_heads = len(sinks)
    group = n_heads // num_kv_heads
    out, lse = [], []
    for b in range(len(qo_indptr) - 1):
        n_q = qo_indptr[b + 1] - qo_indptr[b]
        for t in range(n_q):
            row = qo_indptr[b] + t
            o_row, l_row = [], []
            for h in range(n_heads):
                keys = _key_rows(kvspec, b, h // group)
                weights, vals = [], []
                for j, (kr, vr) in enumerate(keys):
                    if not masks[b][t][j]:
                        continue
                    weights.append(math.exp(scale * math.fsum(a * c for a, c in zip(q[row][h], kr))))
                    vals.append(vr)
                z = math.fsum(weights + [math.exp(sinks[h])])
                d = len(q[row][h])
                o_row.append([math.fsum(w * v[i] for w, v in zip(weights, vals)) / z for i in range(d)])
                l_row.append(math.log(z))
            out.append(o_row)
            lse.append(l_row)
    return out, lse


def brute_balanced(q, kvspec, sinks, scale, window, num_kv_heads, num_segments):
    """The balanced split of a decode batch, token by token: one query row per
    request at position n_k - 1 sees keys max(0, n_k - W) .. n_k - 1 (all of
    them without a window); the pages holding those keys, request after
    request, are numbered 0 .. T - 1, and page number i belongs to the first
    segment s with i < floor((s + 1) T / N).  Each request's keys are grouped
    by segment, every group attended on its own, the first one with the sink.
    Returns per request a list of (segment, first key, last key + 1,
    o[h][d], lse[h]); a request with no key gets one empty group (segment
    -1) holding o = 0 and lse = sink."""
    ps = kvspec["page_size"]
    n_heads = len(sinks)
    group = n_heads // num_kv_heads
    live = []                                       # per request: its visible keys
    for b in range(len(kvspec["kv_len"])):
        n_k = kvspec["kv_len"][b]
        first = max(0, n_k - window) if window > 0 else 0
        live.append(list(range(first, n_k)))
    numbers, total = [], 0                          # per request: page -> list number
    for keys in live:
        pages = sorted(set(j // ps for j in keys))
        numbers.append({p: total + i for i, p in enumerate(pages)})
        total += len(pages)

    def segment_of(i):
        s = 0
        while not i < ((s + 1) * total) // num_segments:
            s += 1
        return s

    result = []
    for b, keys in enumerate(live):
        groups = {}
        for j in keys:
            groups.setdefault(segment_of(numbers[b][j // ps]), []).append(j)
        entries = []
        for n, s in enumerate(sorted(groups)):
            js = groups[s]
            o_h, l_h = [], []
            for h in range(n_heads):
                rows = _key_rows(kvspec, b, h // group)
                weights = [math.exp(scale * math.fsum(x * y for x, y in zip(q[b][h], rows[j][0]))) for j in js]
                sink_w = [math.exp(sinks[h])] if n == 0 else []
                z = math.fsum(weights + sink_w)
                d = len(q[b][h])
                if z == 0.0:
                    o_h.append([0.0] * d)
                    l_h.append(-math.inf)
                    continue
                o_h.append([math.fsum(w * rows[j][1][i] for w, j in zip(weights, js)) / z for i in range(d)])
                l_h.append(math.log(z))
            entries.append((s, js[0], js[-1] + 1, o_h, l_h))
        if not entries:
            d = len(q[b][0])
            entries.append((-1, 0, 0, [[0.0] * d for _ in range(n_heads)], [float(x) for x in sinks]))
        result.append(entries)
    return result
