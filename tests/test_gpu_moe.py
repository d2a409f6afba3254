"""GPU parity of the MoE routing weights (sinkattn_moe_topk_softmax) against
the fp64 oracle (oracle/moe_routing.py): the selected expert ids bit for bit
(the selection compares bf16 logits exactly on both sides; equal logits rank
the lower index first), the weights within one bf16 ulp of the exact softmax
over the selected logits (|g - r| <= 2^-8 |r| + 1e-6).  Source: "GPT-OSS on
day 0", sections "GPT-OSS on Hopper" and "Kernels for GPT-OSS > MoE".
"""

import numpy as np
import pytest

import oracle
from gqa_attention_sinks_amd import workloads as wl
from tests._gpu import bits_to_dev, say, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_attention_sinks_amd as sa
    sa.load_library()


def _bf16_bits(x):
    """fp32 values -> bf16 bit patterns, round to nearest even."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _check(bits, k, what):
    import torch
    import gqa_attention_sinks_amd as sa
    idx, w = sa.moe_topk_softmax(bits_to_dev(bits), k)
    torch.cuda.synchronize()
    ri, rw = oracle.topk_softmax_ref(bits, k)
    gi = idx.cpu().numpy()
    bad = np.nonzero((gi != ri).any(axis=1))[0]
    assert bad.size == 0, f"{what}: expert ids differ on {bad.size} tokens, first {bad[0]}: {gi[bad[0]]} vs {ri[bad[0]]}"
    gw = to_host(w)
    err = np.abs(gw - rw)
    say(f"{what}: tokens={len(bits)} max weight err={err.max():.2e}")
    assert (err <= 2.0 ** -8 * np.abs(rw) + 1e-6).all(), f"{what}: weights off by {err.max():.3e}"


@pytest.mark.parametrize("experts,k", [(128, 4), (32, 4), (512, 8), (7, 7), (1, 1), (65, 3), (256, 8), (96, 2),
                                        (288, 5)])
def test_moe_random_logits(experts, k):
    rng = np.random.default_rng(experts * 10 + k)
    _check(wl._normal_bf16(rng, (4096, experts)), k, f"E={experts} K={k}")


def test_moe_ties_and_signed_zeros():
    rng = np.random.default_rng(5)
    logits = rng.integers(-2, 3, size=(2048, 64)).astype(np.float32)   # five values: ties everywhere
    logits[:, :8] = 0.0
    logits[::2, :8] = -0.0                                             # -0 and +0 tie on value
    _check(_bf16_bits(logits), 4, "ties")
    _check(_bf16_bits(logits), 8, "ties K=8")


def test_moe_extreme_magnitudes():
    rng = np.random.default_rng(6)
    logits = rng.normal(size=(1024, 128)).astype(np.float32) * np.float32(1e30)
    logits[:, 5] = 3e38                                                # near the bf16 maximum
    _check(_bf16_bits(logits), 4, "huge")
    _check(_bf16_bits(rng.normal(size=(1024, 128)).astype(np.float32) * np.float32(1e-30)), 4, "tiny")
