"""The entry points are documented as safe to capture in a HIP graph: they
allocate nothing, never synchronise the host and keep no device state
between calls.  Capture split decode + merge (also with the work ordered
from a host copy of kv_len), the balanced decode + its merge, prefill and
two verify calls (the second large enough for the merge that packs four
(row, head) pairs a wave) into one graph, replay it several times with eager
work in between, and
check every replay against the eager results bit for bit; the same for the
append with rotary embedding and the MoE routing."""

import numpy as np
import pytest

from gqa_attention_sinks_amd import workloads as wl
from tests._gpu import DeviceWorkload, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_attention_sinks_amd as sa
    sa.load_library()


def test_graph_replay_matches_eager():
    import torch
    import gqa_attention_sinks_amd as sa
    dec = DeviceWorkload(wl.paged_decode(batch=24, max_len=2000))
    pre = DeviceWorkload(wl.make_contiguous("graph_prefill", [300, 129], [300, 64], 16, 2,
                                            rng=np.random.default_rng(4)))
    ver = DeviceWorkload(wl.verify_decode(batch=12, max_len=900))
    big = DeviceWorkload(wl.verify_decode())          # 327 rows x 64 heads: the four-pairs-a-wave merge
    dw, pw, vw, bw = dec.w, pre.w, ver.w, big.w

    outs = dict(dec=torch.empty_like(dec.q), pre=torch.empty_like(pre.q), ver=torch.empty_like(ver.q),
                big=torch.empty_like(big.q), bal=torch.empty_like(dec.q), host=torch.empty_like(dec.q))
    o_part = torch.empty((dw.batch, dw.num_qo_heads, 4, 64), dtype=torch.float32, device="cuda:0")
    lse_part = torch.empty((dw.batch, dw.num_qo_heads, 4), dtype=torch.float32, device="cuda:0")
    vo_part = torch.empty((int(vw.qo_indptr[-1]), vw.num_qo_heads, 3, 64), dtype=torch.float32, device="cuda:0")
    vlse_part = torch.empty((int(vw.qo_indptr[-1]), vw.num_qo_heads, 3), dtype=torch.float32, device="cuda:0")
    bo_part = torch.empty((int(bw.qo_indptr[-1]), bw.num_qo_heads, 2, 64), dtype=torch.float32, device="cuda:0")
    blse_part = torch.empty((int(bw.qo_indptr[-1]), bw.num_qo_heads, 2), dtype=torch.float32, device="cuda:0")
    ho_part, hlse_part = torch.empty_like(o_part), torch.empty_like(lse_part)
    ws = torch.empty(sa.decode_balanced_workspace_bytes(dw.batch, dw.num_qo_heads, 37), dtype=torch.uint8,
                     device="cuda:0")

    def work(stream=None):
        sa.decode_paged(dec.q, dec.k, dec.v, dec.kv_indptr, dec.page_indices, dec.kv_len, dec.sinks, dw.scale,
                        num_splits=4, out=outs["dec"], o_part=o_part, lse_part=lse_part, stream=stream)
        sa.prefill(pre.q, pre.qo_indptr, pre.k, pre.v, pre.kv_indptr, pre.sinks, pw.scale, window=0,
                   out=outs["pre"], stream=stream)
        sa.decode_paged_multi(ver.q, ver.qo_indptr, ver.k, ver.v, ver.kv_indptr, ver.page_indices, ver.kv_len,
                              ver.sinks, vw.scale, 8, num_splits=3, out=outs["ver"], o_part=vo_part,
                              lse_part=vlse_part, stream=stream)
        sa.decode_paged_multi(big.q, big.qo_indptr, big.k, big.v, big.kv_indptr, big.page_indices, big.kv_len,
                              big.sinks, bw.scale, 8, num_splits=2, out=outs["big"], o_part=bo_part,
                              lse_part=blse_part, stream=stream)
        sa.decode_paged_balanced(dec.q, dec.k, dec.v, dec.kv_indptr, dec.page_indices, dec.kv_len, dec.sinks,
                                 dw.scale, num_segments=37, out=outs["bal"], workspace=ws, stream=stream)
        sa.decode_paged(dec.q, dec.k, dec.v, dec.kv_indptr, dec.page_indices, dec.kv_len, dec.sinks, dw.scale,
                        num_splits=4, out=outs["host"], o_part=ho_part, lse_part=hlse_part,
                        kv_len_host=dw.kv_len, stream=stream)

    work()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in outs.items()}

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        work(side)                        # warm the side stream once before capture
        side.synchronize()
        with torch.cuda.graph(graph, stream=side):
            work(side)
    torch.cuda.synchronize()
    for rep in range(4):
        for v in outs.values():           # eager work between replays
            v.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in outs.items():
            assert torch.equal(v, eager[k]), f"replay {rep}: {k} differs from the eager result"
    say("graph replays match eager results")


def test_graph_replay_append_and_moe():
    """The append with rotary embedding and the MoE routing (both timed by
    graph replay in the benchmark), captured together and replayed with
    their outputs cleared and the pools restored between replays."""
    import torch
    import gqa_attention_sinks_amd as sa
    from tests._gpu import bits_to_dev, i32_to_dev
    from tests.test_gpu_append import _case
    c = _case(61, [40, 300, 17, 1000], [5, 64, 17, 1], 16, 2)
    q, k, v = bits_to_dev(c["q"]), bits_to_dev(c["k"]), bits_to_dev(c["v"])
    kp0, vp0 = bits_to_dev(c["k_pool"]), bits_to_dev(c["v_pool"])
    kp, vp = kp0.clone(), vp0.clone()
    meta = [i32_to_dev(c[n]) for n in ("append_indptr", "page_indptr", "page_indices", "kv_len")]
    table = torch.from_numpy(c["table"]).to("cuda:0")
    q_out = torch.empty_like(q)
    logits = bits_to_dev(wl._normal_bf16(np.random.default_rng(62), (777, 96)))
    idx = torch.empty((777, 4), dtype=torch.int32, device="cuda:0")
    wts = torch.empty((777, 4), dtype=torch.bfloat16, device="cuda:0")

    def work(stream=None):
        sa.append_paged_kv_rope(k, v, meta[0], kp, vp, meta[1], meta[2], meta[3], table, q=q, q_out=q_out,
                                stream=stream)
        sa.moe_topk_softmax(logits, 4, idx, wts, stream=stream)

    def reset():                          # eager work between replays
        kp.copy_(kp0)
        vp.copy_(vp0)
        for t in (q_out, idx, wts):
            t.zero_()

    work()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (kp, vp, q_out, idx, wts)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        work(side)
        side.synchronize()
        with torch.cuda.graph(graph, stream=side):
            work(side)
    torch.cuda.synchronize()
    for rep in range(3):
        reset()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, ref in zip(("k_pool", "v_pool", "q_out", "topk_idx", "topk_w"),
                                  (kp, vp, q_out, idx, wts), eager):
            assert torch.equal(got, ref), f"replay {rep}: {name} differs from the eager result"
    say("append and MoE graph replays match eager results")
