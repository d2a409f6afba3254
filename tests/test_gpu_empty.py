"""Empty and degenerate inputs on the GPU, against the fp64 oracle.

A request with no cached key (kv_len = 0) in a decode or verify batch sees
only the sink: out = 0 and LSE = the sink (-inf without one), and in the
split partials chunk 0 carries the sink while every other chunk is empty
("GPT-OSS on day 0", section "Kernels for GPT-OSS > Sink attention": the sink
is part of the first block only).  Calls with no token at all (an append of
zero tokens, MoE routing of zero tokens) read and write nothing, also when
torch hands the library NULL pointers for the empty buffers.
"""

import numpy as np
import pytest

import oracle
from gqa_attention_sinks_amd import workloads as wl
from tests._gpu import (DeviceWorkload, assert_parity, bits_to_dev, i32_to_dev, kv_cache, oracle_full,
                        say, to_host)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_attention_sinks_amd as sa
    sa.load_library()


def _with_empty_requests(w, empty):
    """The workload with the listed requests' caches emptied (their pages stay
    allocated, as a serving engine's would before the first append)."""
    kv_len = w.kv_len.copy()
    kv_len[list(empty)] = 0
    w.kv_len = kv_len
    return w


@pytest.mark.parametrize("num_splits", [1, 4])
def test_decode_requests_without_keys(num_splits):
    rng = np.random.default_rng(31)
    w = wl.make_paged("no_keys", [40, 17, 300, 1, 70], [1, 1, 1, 1, 1], 16, 2, rng=rng, decode=True,
                      sink_overrides=wl.outlier_sinks)
    w = _with_empty_requests(w, [1, 3])
    say(f"decode with empty requests S={num_splits}")
    d = DeviceWorkload(w)
    ro, rl = oracle_full(w, 0)
    assert np.all(ro[[1, 3]] == 0.0)
    out, lse = d.decode(num_splits)
    assert_parity(to_host(out), ro, f"decode empty S={num_splits}", to_host(lse), rl)
    # the LSE of an empty request is the sink itself (through base 2 and back in fp32)
    np.testing.assert_allclose(to_host(lse)[[1, 3]], np.broadcast_to(w.sinks, (2, 16)), rtol=1e-6, atol=1e-6)
    if num_splits > 1:
        o_part, lse_part = d.decode(num_splits, merge=False)
        rp, rlp = oracle.split_partials_ref(w.q, kv_cache(w), w.sinks, w.scale, num_splits)
        assert_parity(to_host(o_part), rp, "decode empty partials", to_host(lse_part), rlp)


def test_verify_requests_without_keys():
    """Verify rows of requests whose cache is empty: every row sits before
    the first key."""
    rng = np.random.default_rng(32)
    w = wl.make_paged("verify_no_keys", [9, 40, 300, 5], [3, 2, 8, 4], 64, 8, rng=rng)
    w = _with_empty_requests(w, [0, 3])
    say("verify with empty requests")
    d = DeviceWorkload(w)
    ro, rl = oracle_full(w, 0)
    for s in [1, 3]:
        out, lse = d.decode_multi(s, 8)
        assert_parity(to_host(out), ro, f"verify empty S={s}", to_host(lse), rl)
    rows0 = slice(int(w.qo_indptr[0]), int(w.qo_indptr[1]))
    assert np.all(to_host(out)[rows0] == 0.0)


def test_append_of_zero_tokens_writes_nothing():
    import torch
    import gqa_attention_sinks_amd as sa
    rng = np.random.default_rng(33)
    kv_len = np.array([20, 33], dtype=np.int32)
    page_indptr = np.array([0, 2, 5], dtype=np.int32)
    k_pool = wl._normal_bf16(rng, (6, 2, 16, 64))
    v_pool = wl._normal_bf16(rng, (6, 2, 16, 64))
    kp, vp = bits_to_dev(k_pool), bits_to_dev(v_pool)
    empty = torch.empty((0, 2, 64), dtype=torch.bfloat16, device="cuda:0")
    table = torch.ones((64, 64), dtype=torch.float32, device="cuda:0")
    say("append of zero tokens")
    sa.append_paged_kv_rope(empty, empty.clone(), i32_to_dev(np.zeros(3, dtype=np.int32)), kp, vp,
                            i32_to_dev(page_indptr), i32_to_dev(np.arange(5, dtype=np.int32)),
                            i32_to_dev(kv_len), table)
    torch.cuda.synchronize()
    for pool, host in [(kp, k_pool), (vp, v_pool)]:   # bit for bit
        np.testing.assert_array_equal(pool.view(torch.int16).cpu().numpy(), host.view(np.int16))


def test_moe_of_zero_tokens():
    import torch
    import gqa_attention_sinks_amd as sa
    say("moe routing of zero tokens")
    logits = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda:0")
    idx, w = sa.moe_topk_softmax(logits, 4)
    torch.cuda.synchronize()
    assert tuple(idx.shape) == (0, 4) and tuple(w.shape) == (0, 4)
