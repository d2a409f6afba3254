"""fp64 CPU oracle for grouped-query attention with per-head learned sinks.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (``gqa_attention_sinks_amd``) and imports nothing from it.

Sources (the pages are the authority on what is computed):

* [DAY0-SINK]  Perplexity blog post "GPT-OSS on day 0" (read in its French
  rendering "GPT-OSS au jour J" and its Chinese/Icelandic/Turkish
  renderings), section "Kernels for GPT-OSS > Sink attention".  The sink is an
  extra per-head term that joins the softmax next to the Q.K products; the
  streaming softmax keeps a running max ``m`` and a scale ``d``; starting ``m``
  at the head's sink value (with ``d = 1``) makes the sink land in the softmax
  denominator; when attention is split into blocks along the KV sequence, only
  the first block carries it.
* [DAY0-HOPPER] same post, section "GPT-OSS on Hopper": attention is GQA with
  attention sinks, each head owning one pretrained sink parameter that is
  counted in the softmax.
* [SONAR-INF]  Perplexity blog post "Accelerating Sonar through speculation"
  (Greek rendering), section "Inference with speculative decoding": KV-cache
  pages are allocated per request by the scheduler and the page information
  travels to the GPU as metadata built on the CPU.

Where the pages are silent (the formulas themselves were lost in the text of
the pages, causal alignment, window length, split rule, LSE base, head
mapping) the readings used here are listed in the module docstring of
``oracle.sink_attention``.

Pins: every function here is checked by ``tests/test_oracle_pins.py`` against
closed forms, library attention, brute force (float and 50-digit mpmath),
hand-worked examples in ``tests/golden/`` and invariants.  The conventions
that the pages cannot decide (head mapping, window count, chunk rule, LSE
base) are fixed by reading and enforced by tests; they are "parity unpinned"
by the pages themselves.
"""

from .sink_attention import (  # noqa: F401
    KVCache,
    widen_bf16,
    sink_attention_ref,
    split_bounds_ref,
    split_partials_ref,
    merge_ref,
    attention_weights_ref,
    visible_range,
    live_pages_ref,
    balanced_pieces_ref,
    pieces_partials_ref,
)
from .rope_append import append_rope_ref, append_positions, rotate  # noqa: F401
from .moe_routing import topk_softmax_ref  # noqa: F401
