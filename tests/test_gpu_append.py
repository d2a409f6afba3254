"""GPU parity of the paged KV append with rotary embedding
(sinkattn_append_paged_kv_rope) against the fp64 oracle (oracle/rope_append.py).

Values move bit for bit; rotated keys and queries are fp32 arithmetic rounded
to bf16, checked within |g - r| <= 2^-8 |r| + 1e-5 (one bf16 ulp plus the
fp32 rounding of x1 c - x2 s); every pool slot the append must not touch is
compared bit for bit.  Sources: "GPT-OSS on day 0", section "GPT-OSS on
Hopper" (YaRN rotary encoding); "Accelerating Sonar through speculation",
section "Inference with speculative decoding" (paged KV, CPU-built tables).
"""

import numpy as np
import pytest

import oracle
from gqa_attention_sinks_amd import workloads as wl
from tests._gpu import bits_to_dev, i32_to_dev, say, to_host

pytestmark = pytest.mark.gpu

RTOL, ATOL = 2.0 ** -8, 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_attention_sinks_amd as sa
    sa.load_library()


def rotary_table(max_pos, base=10000.0):
    f = np.arange(32)
    ang = np.arange(max_pos)[:, None] * base ** (-2.0 * f / 64)[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def _case(seed, kv_len, n_new, hq, hkv, max_pos=None):
    rng = np.random.default_rng(seed)
    kv_len = np.asarray(kv_len, dtype=np.int32)
    n_new = np.asarray(n_new, dtype=np.int32)
    append_indptr = np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32)
    n_pages = (kv_len + 15) // 16
    page_indptr = np.concatenate([[0], np.cumsum(n_pages)]).astype(np.int32)
    pool = int(page_indptr[-1]) + 4
    page_indices = rng.permutation(pool)[: page_indptr[-1]].astype(np.int32)
    t = int(append_indptr[-1])
    bf = lambda shape: wl._normal_bf16(rng, shape)
    return dict(q=bf((t, hq, 64)), k=bf((t, hkv, 64)), v=bf((t, hkv, 64)), append_indptr=append_indptr,
                kv_len=kv_len, page_indptr=page_indptr, page_indices=page_indices,
                k_pool=bf((pool, hkv, 16, 64)), v_pool=bf((pool, hkv, 16, 64)),
                table=rotary_table(max_pos or int(kv_len.max()) + 1))


def _run_gpu(c, interleaved, with_q=True, in_place=False):
    import torch
    import gqa_attention_sinks_amd as sa
    kp, vp = bits_to_dev(c["k_pool"]), bits_to_dev(c["v_pool"])
    q = bits_to_dev(c["q"]) if with_q else None
    q_out = q if in_place else None
    table = torch.from_numpy(c["table"]).to("cuda:0")
    out = sa.append_paged_kv_rope(bits_to_dev(c["k"]), bits_to_dev(c["v"]), i32_to_dev(c["append_indptr"]),
                                  kp, vp, i32_to_dev(c["page_indptr"]), i32_to_dev(c["page_indices"]),
                                  i32_to_dev(c["kv_len"]), table, interleaved=interleaved, q=q, q_out=q_out)
    torch.cuda.synchronize()
    raw = lambda x: x.view(torch.int16).cpu().numpy().view(np.uint16)
    return (None if out is None else to_host(out)), raw(kp), raw(vp), kp, vp, out


def _check(c, interleaved, with_q=True, in_place=False):
    q_out, kbits, vbits, _, _, _ = _run_gpu(c, interleaved, with_q, in_place)
    rq, rk, rv = oracle.append_rope_ref(c["q"], c["k"], c["v"], c["append_indptr"], c["kv_len"], c["page_indptr"],
                                        c["page_indices"], c["k_pool"], c["v_pool"], c["table"], interleaved)
    req, pos = oracle.append_positions(c["append_indptr"], c["kv_len"])
    ok = pos < c["table"].shape[0]
    written = np.zeros(c["k_pool"].shape[:1] + c["k_pool"].shape[2:3], dtype=bool)
    for t, (b, p) in enumerate(zip(req, pos)):
        if not ok[t]:
            continue
        page = c["page_indices"][c["page_indptr"][b] + p // 16]
        written[page, p % 16] = True
        np.testing.assert_array_equal(vbits[page, :, p % 16], c["v"][t], err_msg=f"value row of token {t}")
        g = oracle.widen_bf16(kbits[page, :, p % 16])
        err = np.abs(g - rk[page, :, p % 16])
        assert (err <= RTOL * np.abs(rk[page, :, p % 16]) + ATOL).all(), f"key row of token {t}: {err.max():.3e}"
    # every other slot untouched, bit for bit
    for bits, orig in [(kbits, c["k_pool"]), (vbits, c["v_pool"])]:
        keep = ~written
        np.testing.assert_array_equal(bits.transpose(0, 2, 1, 3)[keep], orig.transpose(0, 2, 1, 3)[keep])
    if with_q:
        err = np.abs(q_out[ok] - rq[ok])
        assert (err <= RTOL * np.abs(rq[ok]) + ATOL).all(), f"queries: {err.max():.3e}"
    return int(ok.sum())


@pytest.mark.parametrize("interleaved", [False, True])
@pytest.mark.parametrize("heads", [(64, 8), (4, 1), (16, 1)])
def test_append_rope_shapes(interleaved, heads):
    c = _case(1 + heads[0], [5, 17, 40, 1, 300, 16], [2, 1, 17, 1, 8, 16], *heads)
    n = _check(c, interleaved)
    say(f"append heads={heads} interleaved={interleaved}: {n} tokens")


@pytest.mark.parametrize("seed", range(12))
def test_append_random_shapes(seed):
    """Seeded random batches: head counts, requests, prefix lengths (also
    page-aligned and empty prefixes), new-token counts, pair layout, queries
    rotated in place, kept apart or not given, and a table that may end
    before the last positions."""
    rng = np.random.default_rng(500 + seed)
    hq, hkv = [(64, 8), (8, 8), (16, 2), (4, 1), (32, 4)][rng.integers(5)]
    batch = int(rng.integers(1, 12))
    n_new = rng.integers(1, 70, size=batch)
    prefix = rng.choice([0, 16, 32, 15, 17, 100, 1000, 4095], size=batch)
    kv_len = prefix + n_new
    max_pos = int(kv_len.max()) + 1 if rng.random() < 0.7 else int(rng.integers(1, kv_len.max() + 1))
    c = _case(600 + seed, kv_len, n_new, hq, hkv, max_pos=max_pos)
    interleaved = bool(rng.integers(2))
    mode = int(rng.integers(3))   # 0: queries out of place, 1: in place, 2: keys only
    n = _check(c, interleaved, with_q=mode != 2, in_place=mode == 1)
    say(f"append random seed={seed}: B={batch} H={hq}/{hkv} interleaved={interleaved} mode={mode} "
        f"table={max_pos}: {n} tokens placed")


def test_append_in_place_keys_only_and_out_of_table():
    c = _case(7, [33, 100, 64], [3, 5, 2], 64, 8, max_pos=98)   # request 1's last two positions are past the table
    _check(c, False, in_place=True)
    _check(c, True, with_q=False)


def test_append_many_tokens():
    """16 prefill chunks of 512 tokens on prefixes uniform in [0, 16384]."""
    rng = np.random.default_rng(3)
    prefix = rng.integers(0, 16385, size=16)
    c = _case(3, prefix + 512, np.full(16, 512), 64, 8)
    say("append 16 x 512 tokens")
    _check(c, False)


def test_append_then_decode_reads_what_was_written():
    """Rotate and append the last tokens, then attend over the cache with the
    rotated queries: the decode over the appended pool equals the oracle's
    attention over the oracle's appended pool."""
    import torch
    import gqa_attention_sinks_amd as sa
    c = _case(9, [50, 700, 129, 3000], [1, 4, 2, 8], 64, 8)
    q_out, _, _, kp, vp, qd = _run_gpu(c, False)
    rq, rk, rv = oracle.append_rope_ref(c["q"], c["k"], c["v"], c["append_indptr"], c["kv_len"], c["page_indptr"],
                                        c["page_indices"], c["k_pool"], c["v_pool"], c["table"], False)
    sinks = np.random.default_rng(10).normal(0, 2, size=64).astype(np.float32)
    out = sa.decode_paged_multi(qd, i32_to_dev(c["append_indptr"]), kp, vp, i32_to_dev(c["page_indptr"]),
                                i32_to_dev(c["page_indices"]), i32_to_dev(c["kv_len"]),
                                torch.from_numpy(sinks).to("cuda:0"), 0.125, 8, num_splits=3)
    kv = oracle.KVCache(k=rk, v=rv, kv_indptr=c["page_indptr"], paged=True, page_indices=c["page_indices"],
                        kv_len=c["kv_len"], page_size=16)
    ro, _ = oracle.sink_attention_ref(q_out, c["append_indptr"], kv, sinks, 0.125, 0)
    g = to_host(out)
    err = np.abs(g - ro)
    say(f"append -> decode: max_abs={err.max():.3e}")
    # keys in the pool are the kernel's bf16 rounding of the oracle's fp64 keys
    assert (err <= 2e-2 * np.abs(ro) + 5e-3).all()
