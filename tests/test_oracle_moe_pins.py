"""Pins of the fp64 MoE routing reference (oracle/moe_routing.py): a
hand-worked row, brute force over every K-subset, closed forms (K = E is the
softmax over all experts, K = 1 gives weight 1), invariants (weights sum to
1, a shift of every logit changes nothing) and planted mistakes.

Source: "GPT-OSS on day 0", sections "GPT-OSS on Hopper" and "Kernels for
GPT-OSS > MoE" (softmax over the top-K selected experts only, in bf16).
"""

import itertools
import math

import numpy as np
import pytest
from scipy.special import softmax

import oracle


def test_hand_worked_row_with_ties():
    # logits of 6 experts; K = 3.  Largest are 2.0 (expert 4), then 1.0 twice
    # (experts 1 and 5: the lower index first), then 0.5 (expert 0) drops out.
    logits = np.array([[0.5, 1.0, -1.0, 0.0, 2.0, 1.0]])
    idx, w = oracle.topk_softmax_ref(logits, 3)
    assert idx.tolist() == [[4, 1, 5]]
    z = math.exp(2.0) + 2 * math.exp(1.0)
    np.testing.assert_allclose(w[0], [math.exp(2.0) / z, math.exp(1.0) / z, math.exp(1.0) / z], rtol=1e-15)


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_subsets(seed):
    rng = np.random.default_rng(seed)
    e, k = int(rng.integers(2, 9)), None
    k = int(rng.integers(1, e + 1))
    logits = np.round(rng.normal(size=(20, e)) * 4) / 4     # quarter steps: ties happen
    idx, w = oracle.topk_softmax_ref(logits, k)
    for r in range(len(logits)):
        # the subset with the largest logit sum, ties broken by the smaller sorted index tuple
        best = max(itertools.combinations(range(e), k),
                   key=lambda c: (sum(logits[r, j] for j in c), [-j for j in sorted(c, key=lambda j: (-logits[r, j], j))]))
        assert sorted(idx[r].tolist()) == sorted(best)
        assert all(logits[r, idx[r, i]] >= logits[r, idx[r, i + 1]] for i in range(k - 1))
        ex = [math.exp(logits[r, j]) for j in idx[r]]
        np.testing.assert_allclose(w[r], [x / math.fsum(ex) for x in ex], rtol=1e-14)


def test_closed_forms_and_invariants():
    rng = np.random.default_rng(9)
    logits = rng.normal(size=(50, 16))
    idx, w = oracle.topk_softmax_ref(logits, 16)      # K = E: softmax over all experts, reordered
    np.testing.assert_allclose(w, np.take_along_axis(softmax(logits, axis=1), idx, axis=1), rtol=1e-14)
    idx1, w1 = oracle.topk_softmax_ref(logits, 1)
    assert (idx1[:, 0] == np.argmax(logits, axis=1)).all() and (w1 == 1.0).all()
    idx4, w4 = oracle.topk_softmax_ref(logits, 4)
    np.testing.assert_allclose(w4.sum(axis=1), 1.0, rtol=1e-14)
    idx4s, w4s = oracle.topk_softmax_ref(logits + 3.25, 4)
    assert (idx4s == idx4).all()
    np.testing.assert_allclose(w4s, w4, rtol=1e-13)
    # a softmax over all experts followed by top-K (the other routing family)
    # is a different thing: the planted variant must differ
    all_then_k = np.take_along_axis(softmax(logits, axis=1), idx4, axis=1)
    assert np.max(np.abs(all_then_k - w4)) > 1e-2
