"""Plain fp64 reference for GPT-OSS's MoE routing weights (TEST
INFRASTRUCTURE ONLY: used by ``tests/`` alone; shares nothing with the HIP
library).

Source: "GPT-OSS on day 0", sections "GPT-OSS on Hopper" (the expert weights
take a softmax after the top-K selection) and "Kernels for GPT-OSS > MoE"
(unlike DeepSeek-style models, which take the softmax over all experts,
GPT-OSS takes it over the top-K selected experts only, and the expert
weights must be computed in bfloat16 precision).  Readings:

* R22 the router logits are bf16; the selection compares those bf16 values
      exactly, the K largest first; equal logits rank the lower expert index
      first (the pages give no tie rule);
* R23 "in bfloat16 precision": the softmax over the K selected logits is
      evaluated on the bf16 logits and its result rounded to bf16 (the
      rounding is the library's; this reference returns the exact value).
"""

from __future__ import annotations

import numpy as np


def topk_softmax_ref(logits, k: int):
    """``logits [T, E]`` (bf16 bit patterns or floats) -> ``(idx [T, K] int64,
    w [T, K] fp64)``: the K largest logits of each row in decreasing order
    (ties: lower index first) and the softmax over those K logits alone."""
    from .sink_attention import _as_f64
    x = _as_f64(logits)
    t, e = x.shape
    idx = np.empty((t, k), dtype=np.int64)
    w = np.empty((t, k))
    for r in range(t):
        order = sorted(range(e), key=lambda j: (-x[r, j], j))   # largest first, lower index on ties
        sel = order[:k]
        idx[r] = sel
        v = x[r, sel]
        ex = np.exp(v - v.max())
        w[r] = ex / ex.sum()
    return idx, w
