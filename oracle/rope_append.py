"""Plain fp64 reference for appending new keys/values to a paged KV cache with
rotary position embedding applied to the new queries and keys (TEST
INFRASTRUCTURE ONLY: used by ``tests/`` alone; shares nothing with the HIP
library).

Sources: "GPT-OSS on day 0", section "GPT-OSS on Hopper" (the models use
YaRN rotary position encoding, as DeepSeek-V3 does); "Accelerating Sonar
through speculation", section "Inference with speculative decoding" (KV-cache
pages are allocated per request and the page tables travel to the GPU as
metadata).  The pages give neither the YaRN constants nor the pairing of the
rotated dimensions, so:

* R19 the rotation angles come from the caller as a table ``cos_sin[pos, 64]``
      (cos of the 32 frequency pairs in columns 0..31, sin in 32..63), so any
      frequency scaling (YaRN's included) lives in the table;
* R20 pairs are (x[f], x[f + 32]) ("half" layout) or (x[2f], x[2f + 1])
      ("interleaved"), chosen by the caller; pair f at position p rotates by
      the table's angle: (a, b) -> (a cos - b sin, b cos + a sin);
* R21 request b appends n_b tokens that take logical positions
      kv_len[b] - n_b .. kv_len[b] - 1 (kv_len counts them already, as the
      attention call that follows sees them); position p lives in page
      page_indices[page_indptr[b] + p // 16], slot p % 16.  A token whose
      position lies outside the table ([0, max_pos)) has no angle: nothing of
      it is written (its query row is left undefined, NaN here).
"""

from __future__ import annotations

import numpy as np

HALF = 32


def _pairs(d: int, interleaved: bool):
    """Index arrays (first, second) of the 32 rotated pairs."""
    f = np.arange(d // 2)
    if interleaved:
        return 2 * f, 2 * f + 1
    return f, f + d // 2


def rotate(x, pos, cos_sin, interleaved: bool):
    """Rotate vectors ``x [..., D]`` (fp64) at integer positions ``pos [...]``."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    i, j = _pairs(d, interleaved)
    c = np.asarray(cos_sin, dtype=np.float64)[np.asarray(pos)][..., :d // 2]
    s = np.asarray(cos_sin, dtype=np.float64)[np.asarray(pos)][..., d // 2:]
    out = x.copy()
    out[..., i] = x[..., i] * c - x[..., j] * s
    out[..., j] = x[..., j] * c + x[..., i] * s
    return out


def append_positions(append_indptr, kv_len):
    """(request, logical position) of every appended token, in order (R21)."""
    append_indptr = np.asarray(append_indptr, dtype=np.int64)
    kv_len = np.asarray(kv_len, dtype=np.int64)
    req, pos = [], []
    for b in range(len(append_indptr) - 1):
        n = int(append_indptr[b + 1] - append_indptr[b])
        for i in range(n):
            req.append(b)
            pos.append(int(kv_len[b]) - n + i)
    return np.asarray(req, dtype=np.int64), np.asarray(pos, dtype=np.int64)


def append_rope_ref(q, k_new, v_new, append_indptr, kv_len, page_indptr, page_indices, k_pool, v_pool,
                    cos_sin, interleaved: bool = False):
    """Returns ``(q_out [T, Hq, D], k_pool', v_pool')`` in fp64: the new
    queries and keys rotated at their positions, the new keys and values
    written to their page slots, every other pool entry unchanged.  Inputs
    may be bf16 bit patterns (uint16) or floats."""
    from .sink_attention import _as_f64
    qf, kf, vf = _as_f64(q), _as_f64(k_new), _as_f64(v_new)
    kp, vp = _as_f64(k_pool).copy(), _as_f64(v_pool).copy()
    req, pos = append_positions(append_indptr, kv_len)
    ok = (pos >= 0) & (pos < np.asarray(cos_sin).shape[0])
    safe = np.where(ok, pos, 0)
    q_out = rotate(qf, safe[:, None], cos_sin, interleaved)
    q_out[~ok] = np.nan
    k_rot = rotate(kf, safe[:, None], cos_sin, interleaved)
    page_size = kp.shape[2]
    for t, (b, p) in enumerate(zip(req, pos)):
        if not ok[t]:
            continue
        page = int(np.asarray(page_indices)[int(page_indptr[b]) + p // page_size])
        kp[page, :, p % page_size, :] = k_rot[t]
        vp[page, :, p % page_size, :] = vf[t]
    return q_out, kp, vp
