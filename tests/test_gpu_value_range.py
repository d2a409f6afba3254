"""V at the edge of the accepted range (|v| <= 65280, include/sinkattn.h):
the kernels stage V as fp16, and values up to the bound must give the
oracle's results, also when they sit on keys that a window or the causal
rule hides from some rows (those keys are staged with the visible ones and
meet a zero weight).

Each request gets two large V rows (one key each) in every KV head:
+-65280 and +-59904 (bf16 values) in alternating dimensions, so no output
element sums large values of opposite signs (the fp16 weights' relative
rounding then stays far inside the 1 % relative tolerance)."""

import numpy as np
import pytest

from gqa_attention_sinks_amd import workloads as wl
from tests._gpu import DeviceWorkload, assert_parity, oracle_full, say, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_attention_sinks_amd as sa
    sa.load_library()


BIG = (65280.0, 59904.0)


def _with_big_values(w, rng):
    """Put the two large V rows at random logical keys of every request."""
    v = w.v.copy()
    sign = np.where(np.arange(w.head_dim) % 2 == 0, 1.0, -1.0).astype(np.float32)
    for b in range(w.batch):
        n_k = int(w.kv_len[b])
        keys = rng.choice(n_k, size=min(2, n_k), replace=False)
        for key, mag in zip(keys, BIG):
            row = wl.bf16_bits(mag * sign)
            if w.paged:
                page = w.page_indices[w.kv_indptr[b] + key // w.page_size]
                v[page, :, key % w.page_size, :] = row
            else:
                v[int(w.kv_indptr[b]) + key, :, :] = row
    w.v = v
    return w


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("window", [0, 37])
def test_prefill_v_at_the_bound(paged, window):
    rng = np.random.default_rng(40 + window + int(paged))
    kv_len = np.array([130, 300, 77, 513])
    qo_len = np.array([130, 129, 20, 257])
    maker = wl.make_paged if paged else wl.make_contiguous
    w = _with_big_values(maker("vrange", kv_len, qo_len, 16, 2, rng=rng), rng)
    say(f"prefill |v| up to 65280 paged={paged} window={window}")
    out, lse = DeviceWorkload(w).prefill(window=window)
    ro, rl = oracle_full(w, window)
    assert np.abs(ro).max() > 1000.0          # the large rows do reach the outputs
    assert_parity(to_host(out), ro, f"prefill vrange paged={paged} W={window}", to_host(lse), rl)


@pytest.mark.parametrize("window", [0, 37])
def test_decode_v_at_the_bound(window):
    rng = np.random.default_rng(50 + window)
    kv_len = np.array([1, 17, 300, 4096, 700, 33])
    w = _with_big_values(wl.make_paged("vrange_dec", kv_len, np.ones_like(kv_len), 64, 8, rng=rng,
                                       decode=True, sink_overrides=wl.outlier_sinks), rng)
    say(f"decode |v| up to 65280 window={window}")
    d = DeviceWorkload(w)
    ro, rl = oracle_full(w, window)
    for s in [1, 3]:
        out, lse = d.decode(s, window=window)
        assert_parity(to_host(out), ro, f"decode vrange W={window} S={s}", to_host(lse), rl)


def test_decode_multi_v_at_the_bound():
    rng = np.random.default_rng(60)
    kv_len = np.array([8, 17, 300, 4096, 700, 33])
    qo_len = np.array([8, 3, 5, 2, 1, 4])
    w = _with_big_values(wl.make_paged("vrange_multi", kv_len, qo_len, 64, 8, rng=rng), rng)
    say("verify decode |v| up to 65280")
    d = DeviceWorkload(w)
    ro, rl = oracle_full(w, 0)
    for s in [1, 3]:
        out, lse = d.decode_multi(s, 8)
        assert_parity(to_host(out), ro, f"multi vrange S={s}", to_host(lse), rl)
