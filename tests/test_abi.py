"""The C ABI without a GPU: the library loads, exports every entry point that
include/sinkattn.h declares, its host-only split rule equals the oracle's, and
argument errors come back as status codes before anything is launched."""

import ctypes
import os
import re

import numpy as np
import pytest

import gqa_attention_sinks_amd as sa
import oracle
from gqa_attention_sinks_amd import binding

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "sinkattn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sa.library_path()):
        import __graft_entry__
        __graft_entry__.build()
    return sa.load_library()


def _declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sinkattn_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_three_calls():
    names = _declared_symbols()
    for n in ["sinkattn_prefill", "sinkattn_decode_paged", "sinkattn_merge"]:
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    names = _declared_symbols()
    assert names, "no declarations parsed"
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/sinkattn.h but not exported"
    assert set(names) == set(binding.EXPORTED)


def test_abi_version(lib):
    assert sa.abi_version() == 8
    assert lib.sinkattn_status_string(0) == b"ok"
    assert lib.sinkattn_status_string(2) == b"unsupported"


def test_kv_descriptor_layout_matches_the_header(tmp_path):
    """The ctypes mirror of sinkattn_kv has the C struct's size and field
    offsets (a C program built against include/sinkattn.h prints them)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    fields = [f for f, _ in binding._KV._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "sinkattn.h"\nint main(void) {\n'
                   '  printf("%zu", sizeof(sinkattn_kv));\n'
                   + "".join(f'  printf(" %zu", offsetof(sinkattn_kv, {f}));\n' for f in fields)
                   + "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-std=c99", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()]
    want = [ctypes.sizeof(binding._KV)] + [getattr(binding._KV, f).offset for f in fields]
    assert got == want, (got, want)


def test_split_rule_matches_oracle_exactly(lib):
    rng = np.random.default_rng(123)
    all_lens = np.arange(0, 4097, dtype=np.int32)
    for s in range(1, 17):
        np.testing.assert_array_equal(sa.split_bounds(all_lens, s), oracle.split_bounds_ref(all_lens, s))
    lens = rng.integers(0, 300000, size=100000).astype(np.int32)
    for s in [1, 3, 16]:
        np.testing.assert_array_equal(sa.split_bounds(lens, s), oracle.split_bounds_ref(lens, s))
    for s in [37, 256]:
        np.testing.assert_array_equal(sa.split_bounds(lens[:3000], s), oracle.split_bounds_ref(lens[:3000], s))
    # long-context shape: 16 chunks of 8192 keys
    b = sa.split_bounds([131072], 16)
    assert np.all(b[0, :, 1] - b[0, :, 0] == 8192)


def test_pick_num_splits_is_in_range(lib):
    assert 1 <= sa.pick_num_splits(np.full(64, 4096), 8) <= 256
    assert sa.pick_num_splits(np.full(8, 131072), 8) == 16
    assert sa.pick_num_splits(np.full(4, 10), 8) == 1


def test_pick_num_splits_multi(lib):
    lens = np.full(64, 4096)
    # two workgroups per CU (512 at once): about 683 units without a mask and
    # 1024 with one, over 512 (request, KV head) pairs
    assert sa.pick_num_splits_multi(lens, 64, 8, 8) == 2
    assert sa.pick_num_splits_multi(lens, 64, 8, 8, with_mask=True) == 2
    assert sa.pick_num_splits_multi(lens, 64, 8, 2) == 2          # the same kernel for any row count
    assert sa.pick_num_splits_multi(np.full(16, 4096), 64, 8, 8) == 6
    assert sa.pick_num_splits_multi(np.full(4, 10), 64, 8, 8) == 1   # chunks of at least 16 pages
    assert sa.pick_num_splits_multi(np.full(2, 1 << 20), 64, 8, 8) == 16
    assert lib.sinkattn_pick_num_splits_multi(None, 4, 64, 8, 8, 0) == 1


# ---------------------------------------------------------------------------
# argument errors: every call below fails validation on the host, so no
# kernel is launched and the fake device pointers are never touched.
# ---------------------------------------------------------------------------

FAKE = ctypes.c_void_p(0x1000)
INVALID, UNSUPPORTED = 1, 2


def _kv(paged=1, page_size=16, k=FAKE, page_indices=FAKE, kv_len=FAKE):
    return binding._KV(k, FAKE, paged, page_size, FAKE, page_indices if paged else None,
                       kv_len if paged else None, 0)


def _prefill(lib, kv, q=FAKE, qo=FAKE, out=FAKE, batch=2, total_q=4, hq=8, hkv=2, d=64, scale=0.125, window=0,
             host=None):
    hp = None if host is None else np.ascontiguousarray(host, dtype=np.int32).ctypes.data_as(ctypes.c_void_p)
    return lib.sinkattn_prefill(q, qo, ctypes.byref(kv) if kv is not None else None, None, out, None,
                                batch, total_q, hq, hkv, d, ctypes.c_float(scale), window, hp, None)


def _decode(lib, kv, s=1, out=FAKE, o_part=None, lse_part=None, batch=2, hq=8, hkv=2, d=64, scale=0.125,
            window=0, q=FAKE):
    return lib.sinkattn_decode_paged(q, ctypes.byref(kv) if kv is not None else None, None, s, out, o_part,
                                     lse_part, None, batch, hq, hkv, d, ctypes.c_float(scale), window, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(q=None), INVALID),
    (dict(out=None), INVALID),
    (dict(batch=0), INVALID),
    (dict(hq=6, hkv=4), INVALID),
    (dict(d=128), UNSUPPORTED),
    (dict(hq=64, hkv=2), UNSUPPORTED),
    (dict(scale=0.0), INVALID),
    (dict(scale=float("nan")), INVALID),
    (dict(window=-1), INVALID),
    (dict(total_q=1), INVALID),
])
def test_prefill_argument_errors(lib, kwargs, code):
    assert _prefill(lib, _kv(), **kwargs) == code
    assert lib.sinkattn_last_error()


def test_prefill_host_plan_errors(lib):
    # the host copy of qo_indptr must agree with total_q and give every request a row
    assert _prefill(lib, _kv(), host=[0, 2, 3]) == INVALID
    assert _prefill(lib, _kv(), host=[0, 0, 4]) == INVALID
    assert _prefill(lib, _kv(), host=[0, 4, 4]) == INVALID


def test_prefill_kv_errors(lib):
    assert _prefill(lib, None) == INVALID
    assert _prefill(lib, _kv(page_size=32)) == UNSUPPORTED
    assert _prefill(lib, _kv(page_indices=None)) == INVALID
    assert _prefill(lib, _kv(k=None)) == INVALID


@pytest.mark.parametrize("kwargs,code", [
    (dict(q=None), INVALID),
    (dict(s=0), INVALID),
    (dict(s=257), INVALID),
    (dict(s=1, out=None), INVALID),
    (dict(s=4, o_part=None, lse_part=FAKE), INVALID),
    (dict(s=4, o_part=FAKE, lse_part=None), INVALID),
    (dict(d=32), UNSUPPORTED),
    (dict(hq=7, hkv=2), INVALID),
])
def test_decode_argument_errors(lib, kwargs, code):
    assert _decode(lib, _kv(), **kwargs) == code


def test_decode_needs_paged(lib):
    assert _decode(lib, _kv(paged=0)) == INVALID


def _decode_multi(lib, kv, s=1, out=FAKE, o_part=None, lse_part=None, batch=2, total_q=6, max_rows=4,
                  hq=8, hkv=2, d=64, scale=0.125, window=0, q=FAKE, qo=FAKE, mask=None, mask_indptr=None):
    return lib.sinkattn_decode_paged_multi(q, qo, mask, mask_indptr,
                                           ctypes.byref(kv) if kv is not None else None, None, s, out,
                                           o_part, lse_part, None, batch, total_q, max_rows, hq, hkv, d,
                                           ctypes.c_float(scale), window, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(q=None), INVALID),
    (dict(qo=None), INVALID),
    (dict(total_q=1), INVALID),
    (dict(max_rows=0), INVALID),
    (dict(max_rows=9), INVALID),
    (dict(hq=32, hkv=2, max_rows=8), UNSUPPORTED),     # 16 heads x 8 rows > 64 columns
    (dict(s=0), INVALID),
    (dict(s=1, out=None), INVALID),
    (dict(s=4, o_part=None, lse_part=FAKE), INVALID),
    (dict(d=32), UNSUPPORTED),
    (dict(window=-1), INVALID),
    (dict(mask=FAKE, mask_indptr=None), INVALID),
    (dict(mask=FAKE, mask_indptr=FAKE, window=8), INVALID),
])
def test_decode_multi_argument_errors(lib, kwargs, code):
    assert _decode_multi(lib, _kv(), **kwargs) == code
    assert lib.sinkattn_last_error()


def test_decode_multi_needs_paged(lib):
    assert _decode_multi(lib, _kv(paged=0)) == INVALID


def _append(lib, kv, q=None, k=FAKE, v=FAKE, ai=FAKE, cs=FAKE, max_pos=128, inter=0, q_out=None, batch=2,
            total=4, hq=8, hkv=2, d=64):
    return lib.sinkattn_append_paged_kv_rope(q, k, v, ai, ctypes.byref(kv) if kv is not None else None, cs,
                                             max_pos, inter, q_out, batch, total, hq, hkv, d, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(k=None), INVALID),
    (dict(v=None), INVALID),
    (dict(ai=None), INVALID),
    (dict(cs=None), INVALID),
    (dict(q=FAKE), INVALID),                       # q without q_out
    (dict(q_out=FAKE), INVALID),                   # q_out without q
    (dict(max_pos=0), INVALID),
    (dict(inter=2), INVALID),
    (dict(total=-1), INVALID),
    (dict(d=128), UNSUPPORTED),
    (dict(cs=ctypes.c_void_p(0x1004)), INVALID),   # table not 16-byte aligned
    (dict(batch=0), INVALID),
])
def test_append_argument_errors(lib, kwargs, code):
    assert _append(lib, _kv(), **kwargs) == code
    assert lib.sinkattn_last_error()


def test_append_needs_paged(lib):
    assert _append(lib, _kv(paged=0)) == INVALID


def test_zero_sized_calls_accept_null_buffers(lib):
    # nothing to read or write: the token buffers may be NULL and nothing is launched
    assert _append(lib, _kv(), k=None, v=None, total=0) == 0
    assert _append(lib, _kv(), k=None, v=FAKE, total=1) == INVALID
    assert lib.sinkattn_moe_topk_softmax(None, 0, 32, 4, None, None, None) == 0
    assert lib.sinkattn_moe_topk_softmax(None, 1, 32, 4, FAKE, FAKE, None) == INVALID
    assert lib.sinkattn_moe_topk_softmax(None, 0, 32, 33, None, None, None) == INVALID


@pytest.mark.parametrize("args,code", [
    ((None, 4, 32, 4, FAKE, FAKE), INVALID),
    ((FAKE, 4, 32, 4, None, FAKE), INVALID),
    ((FAKE, 4, 32, 4, FAKE, None), INVALID),
    ((FAKE, -1, 32, 4, FAKE, FAKE), INVALID),
    ((FAKE, 4, 0, 1, FAKE, FAKE), UNSUPPORTED),
    ((FAKE, 4, 513, 4, FAKE, FAKE), UNSUPPORTED),
    ((FAKE, 4, 32, 0, FAKE, FAKE), INVALID),
    ((FAKE, 4, 32, 9, FAKE, FAKE), INVALID),
    ((FAKE, 4, 3, 4, FAKE, FAKE), INVALID),
])
def test_moe_argument_errors(lib, args, code):
    assert lib.sinkattn_moe_topk_softmax(*args, None) == code


def test_merge_argument_errors(lib):
    m = lib.sinkattn_merge
    assert m(None, FAKE, 4, 8, 2, 64, FAKE, None, None) == INVALID
    assert m(FAKE, FAKE, 0, 8, 2, 64, FAKE, None, None) == INVALID
    assert m(FAKE, FAKE, 4, 8, 0, 64, FAKE, None, None) == INVALID
    assert m(FAKE, FAKE, 4, 8, 2, 80, FAKE, None, None) == UNSUPPORTED


def test_split_bounds_argument_errors(lib):
    out = np.zeros(8, dtype=np.int32)
    lens = np.array([5], dtype=np.int32)
    f = lib.sinkattn_split_bounds
    assert f(None, 1, 16, 2, out.ctypes.data_as(ctypes.c_void_p)) == INVALID
    assert f(lens.ctypes.data_as(ctypes.c_void_p), 1, 16, 0, out.ctypes.data_as(ctypes.c_void_p)) == INVALID


# ---------------------------------------------------------------------------
# host validation of CPU-built KV metadata (sinkattn_validate_kv_host)
# ---------------------------------------------------------------------------

def _paged_meta():
    from gqa_attention_sinks_amd import workloads as wl
    rng = np.random.default_rng(5)
    kv_len = np.array([1, 16, 17, 300, 4096])
    return wl.make_paged("validate", kv_len, np.ones_like(kv_len), 8, 2, rng=rng)


def test_validate_accepts_the_workload_generators(lib):
    from gqa_attention_sinks_amd import workloads as wl
    w = _paged_meta()
    sa.validate_kv_host(w.kv_indptr, w.num_pages, w.page_indices, w.kv_len)
    c = wl.make_contiguous("validate_c", [5, 9], [5, 1], 4, 1, rng=np.random.default_rng(1))
    sa.validate_kv_host(c.kv_indptr, c.k.shape[0])


def _expect_invalid(fn, needle):
    with pytest.raises(sa.SinkAttnError) as e:
        fn()
    assert e.value.status == INVALID
    assert needle in str(e.value), str(e.value)


def test_validate_rejects_bad_metadata(lib):
    w = _paged_meta()
    ok = (w.kv_indptr, w.num_pages, w.page_indices, w.kv_len)
    # a page id at the pool's end (one past the last page)
    pages = w.page_indices.copy()
    pages[int(w.kv_indptr[3]) + 5] = w.num_pages
    _expect_invalid(lambda: sa.validate_kv_host(ok[0], ok[1], pages, ok[3]), "request 3, page 5")
    pages[int(w.kv_indptr[3]) + 5] = -1
    _expect_invalid(lambda: sa.validate_kv_host(ok[0], ok[1], pages, ok[3]), "outside [0,")
    # a request longer than its page list (17 keys need 2 pages)
    lens = w.kv_len.copy()
    lens[1] = 17
    _expect_invalid(lambda: sa.validate_kv_host(ok[0], ok[1], ok[2], lens), "request 1 holds 17 keys")
    lens[1] = -1
    _expect_invalid(lambda: sa.validate_kv_host(ok[0], ok[1], ok[2], lens), "kv_len[1]")
    # decreasing page-list offsets
    indptr = w.kv_indptr.copy()
    indptr[2] = indptr[1] - 1
    _expect_invalid(lambda: sa.validate_kv_host(indptr, ok[1], ok[2], ok[3]), "decreases at request 1")
    # contiguous rows past the end of k and v
    _expect_invalid(lambda: sa.validate_kv_host(np.array([0, 5, 14]), 13), "exceeds the 13 rows")
    # an empty pool cannot hold pages
    kv = binding._KV(None, None, 1, 16, None, None, None, 0)
    z = np.zeros(2, dtype=np.int32)
    assert lib.sinkattn_validate_kv_host(ctypes.byref(kv), z.ctypes.data_as(ctypes.c_void_p), None,
                                         z.ctypes.data_as(ctypes.c_void_p), 1) == INVALID


def test_validate_ignores_pages_past_the_live_ones(lib):
    # the page list may be longer than the keys need; only live pages are read
    indptr = np.array([0, 3], dtype=np.int32)
    pages = np.array([0, 1, 99], dtype=np.int32)       # the third page is never read
    sa.validate_kv_host(indptr, 2, pages, np.array([20]))
    sa.validate_kv_host(np.array([0, 3, 3]), 2, pages, np.array([20, 0]))   # a request with no key
    _expect_invalid(lambda: sa.validate_kv_host(indptr, 2, pages, np.array([33])), "id 99")


def test_last_hip_error_is_the_last_error(lib):
    assert _decode(lib, _kv(), s=0) == INVALID
    assert lib.sinkattn_last_hip_error() == lib.sinkattn_last_error()
    assert b"num_splits" in lib.sinkattn_last_hip_error()


def test_noalloc_rejects_partials_beyond_its_scratch(lib):
    """The size check comes before any HIP call: 64 requests x 64 heads x 256
    splits need 272 MB of partials, beyond the 8 MiB array."""
    kv = _kv()
    f = lib.sinkattn_decode_paged_noalloc
    assert f(FAKE, ctypes.byref(kv), None, 256, FAKE, None, 64, 64, 8, 64, ctypes.c_float(0.125), 0, None) == INVALID
    msg = lib.sinkattn_last_error()
    assert b"scratch" in msg and b"caller-owned" in msg
    assert f(None, ctypes.byref(kv), None, 2, FAKE, None, 2, 8, 2, 64, ctypes.c_float(0.125), 0, None) == INVALID
    assert f(FAKE, ctypes.byref(kv), None, 2, None, None, 2, 8, 2, 64, ctypes.c_float(0.125), 0, None) == INVALID
    assert f(FAKE, ctypes.byref(kv), None, 0, FAKE, None, 2, 8, 2, 64, ctypes.c_float(0.125), 0, None) == INVALID
    assert f(FAKE, ctypes.byref(_kv(paged=0)), None, 2, FAKE, None, 2, 8, 2, 64, ctypes.c_float(0.125), 0,
             None) == INVALID


# ---------------------------------------------------------------------------
# the balanced decode's host side
# ---------------------------------------------------------------------------

def test_balanced_segment_rule_matches_oracle_exactly(lib):
    rng = np.random.default_rng(77)
    for _ in range(2000):
        batch = int(rng.integers(1, 70))
        lens = rng.integers(0, 5000, size=batch)
        lens[rng.random(batch) < 0.1] = 0
        window = int(rng.choice([0, 0, 1, 16, 100, 3000]))
        n = int(rng.integers(1, 400))
        got = sa.balanced_segments(lens, n, window)
        ref = np.array([[p[0][0], p[-1][0]] for p in oracle.balanced_pieces_ref(lens, n, window)])
        np.testing.assert_array_equal(got, ref)


def test_balanced_workspace_bytes(lib):
    # plan [B+1] and segments [B, 2] int32, lse [slots, Hq] fp32, each padded to 256 bytes, then
    # o [slots, Hq, 64] fp32
    b, hq, n = 64, 64, 192
    slots = n + b
    expect = 1024 + (slots * hq * 4 + 255) // 256 * 256 + slots * hq * 64 * 4
    assert sa.decode_balanced_workspace_bytes(b, hq, n) == expect
    assert lib.sinkattn_decode_balanced_workspace_bytes(0, 64, 4) == -1
    assert 1 <= sa.pick_num_segments(8) <= 65536


def _balanced(lib, kv, n=4, ws=FAKE, ws_bytes=1 << 30, out=FAKE, batch=2, hq=8, hkv=2, d=64, window=0, q=FAKE):
    return lib.sinkattn_decode_paged_balanced(q, ctypes.byref(kv) if kv is not None else None, None, n, ws, ws_bytes,
                                              out, None, batch, hq, hkv, d, ctypes.c_float(0.125), window, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(q=None), INVALID),
    (dict(out=None), INVALID),
    (dict(ws=None), INVALID),
    (dict(ws=ctypes.c_void_p(0x1008)), INVALID),       # workspace not 16-byte aligned
    (dict(ws_bytes=1000), INVALID),                     # too small
    (dict(n=0), INVALID),
    (dict(batch=257), UNSUPPORTED),
    (dict(d=128), UNSUPPORTED),
    (dict(window=-1), INVALID),
])
def test_balanced_argument_errors(lib, kwargs, code):
    assert _balanced(lib, _kv(), **kwargs) == code
    assert lib.sinkattn_last_error()


def test_balanced_needs_paged(lib):
    assert _balanced(lib, _kv(paged=0)) == INVALID
    assert lib.sinkattn_merge_balanced(None, 4, None, 1 << 20, FAKE, None, 2, 8, 64, None) == INVALID
