"""sinkattn_decode_paged_noalloc: the split decode with its partials in the
library's own device array, for callers that cannot allocate.  Its results
must be those of sinkattn_decode_paged with caller-owned partials (the same
kernels), on consecutive calls that reuse the array, the second smaller."""

import ctypes

import numpy as np
import pytest

import gqa_attention_sinks_amd as sa
from gqa_attention_sinks_amd import binding
from gqa_attention_sinks_amd import workloads as wl
from tests._gpu import DeviceWorkload, assert_parity, oracle_full, say, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sa.load_library()


def _noalloc(d, s, out, lse):
    """One call through the C ABI."""
    import torch
    w = d.w
    lib = sa.load_library()
    kv = binding.kv_descriptor(d.k, d.v, d.kv_indptr, d.page_indices, d.kv_len)
    P = ctypes.c_void_p
    st = lib.sinkattn_decode_paged_noalloc(P(d.q.data_ptr()), ctypes.byref(kv), P(d.sinks.data_ptr()), s,
                                           P(out.data_ptr()), P(lse.data_ptr()), w.batch, w.num_qo_heads,
                                           w.num_kv_heads, 64, ctypes.c_float(w.scale), 0,
                                           P(torch.cuda.current_stream().cuda_stream))
    assert st == 0, lib.sinkattn_last_error().decode()


def _check(w, s, what):
    import torch
    d = DeviceWorkload(w)
    ref_out, ref_lse = d.decode(s)                       # caller-owned partials, merged
    out = torch.full_like(ref_out, float("nan"))
    lse = torch.full_like(ref_lse, float("nan"))
    _noalloc(d, s, out, lse)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(out), to_host(ref_out)), f"{what}: outputs differ"
    assert np.array_equal(to_host(lse), to_host(ref_lse)), f"{what}: LSE differ"
    ro, rl = oracle_full(w, 0)
    assert_parity(to_host(out), ro, what, to_host(lse), rl)


def test_two_calls_in_a_row_the_second_smaller():
    w1 = wl.paged_decode()                               # 64 requests, 4 splits: 4.3 MB of partials
    s1 = sa.pick_num_splits(w1.kv_len, w1.num_kv_heads)
    say(f"noalloc decode: B=64 S={s1}, then B=10 S=3")
    _check(w1, s1, "noalloc full size")
    w2 = wl.paged_decode(seed=3, batch=10, max_len=700)
    w2.sinks = wl.outlier_sinks(w2.sinks)
    _check(w2, 3, "noalloc small")
    _check(w2, 1, "noalloc unsplit")


def test_many_splits_near_the_limit():
    """128 splits of 3 requests (6.4 MB of partials, most chunks empty)."""
    w = wl.paged_decode(seed=4, batch=3, max_len=3000)
    assert 3 * 64 * 128 * 65 * 4 + 256 <= sa.binding.NOALLOC_SCRATCH_BYTES
    say("noalloc decode: B=3 S=128")
    _check(w, 128, "noalloc 128 splits")
