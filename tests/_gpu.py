"""Helpers for the GPU parity tests: move a workload to the device, run the
HIP library through its binding, run the oracle on the same inputs, and check
the parity bar.

Parity bar (bf16 inputs, fp32 accumulation): per element
|gpu - ref| <= 2e-3 + 1e-2 * |ref| (ref = fp64 oracle, gpu = bf16 output
widened); per row, the L2 norms agree within 1e-2 relative (this keeps teeth
on rows whose values are tiny, e.g. behind a +20 sink); LSE within 2e-3
absolute, infinities matching exactly.  Index work (chunk bounds, gathers) is
checked bit for bit by the probe tests.
"""

import sys

import numpy as np

import gqa_attention_sinks_amd as sa
import oracle

ATOL, RTOL = 2e-3, 1e-2
LSE_ATOL = 2e-3
NORM_RTOL = 1e-2


def say(*msg):
    print("[gpu-test]", *msg, flush=True)
    sys.stdout.flush()


def torch_dev():
    import torch
    return torch, torch.device("cuda:0")


def bits_to_dev(a):
    torch, dev = torch_dev()
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)


def i32_to_dev(a):
    torch, dev = torch_dev()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)


def f32_to_dev(a):
    torch, dev = torch_dev()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def to_host(t):
    """Device tensor -> fp64 numpy (bf16 widened exactly)."""
    return t.float().cpu().numpy().astype(np.float64)


class DeviceWorkload:
    def __init__(self, w):
        self.w = w
        self.q = bits_to_dev(w.q)
        self.qo_indptr = i32_to_dev(w.qo_indptr)
        self.k = bits_to_dev(w.k)
        self.v = bits_to_dev(w.v)
        self.kv_indptr = i32_to_dev(w.kv_indptr)
        self.kv_len = i32_to_dev(w.kv_len)
        self.page_indices = i32_to_dev(w.page_indices) if w.paged else None
        self.sinks = f32_to_dev(w.sinks)

    def prefill(self, window, sinks=True, return_lse=True, host_plan=True, kv_len_host=None):
        w = self.w
        return sa.prefill(self.q, self.qo_indptr, self.k, self.v, self.kv_indptr,
                          self.sinks if sinks else None, w.scale, window=window,
                          page_indices=self.page_indices, kv_len=self.kv_len if w.paged else None,
                          return_lse=return_lse, qo_indptr_host=w.qo_indptr if host_plan else None,
                          kv_len_host=kv_len_host)

    def decode(self, num_splits, window=0, merge=True, return_lse=True, sinks=True, kv_len_host=None):
        w = self.w
        return sa.decode_paged(self.q, self.k, self.v, self.kv_indptr, self.page_indices, self.kv_len,
                               self.sinks if sinks else None, w.scale, num_splits=num_splits, window=window,
                               merge=merge, return_lse=return_lse, kv_len_host=kv_len_host)

    def decode_multi(self, num_splits, max_rows, window=0, merge=True, return_lse=True, masks=None,
                     kv_len_host=None):
        w = self.w
        mask = mask_indptr = None
        if masks is not None:
            from gqa_attention_sinks_amd import workloads as wl
            bits, indptr = wl.pack_masks(masks)
            torch, dev = torch_dev()
            mask = torch.from_numpy(bits).to(dev)
            mask_indptr = i32_to_dev(indptr)
        return sa.decode_paged_multi(self.q, self.qo_indptr, self.k, self.v, self.kv_indptr,
                                     self.page_indices, self.kv_len, self.sinks, w.scale, max_rows,
                                     num_splits=num_splits, window=window, merge=merge,
                                     return_lse=return_lse, custom_mask=mask, mask_indptr=mask_indptr,
                                     kv_len_host=kv_len_host)


def kv_cache(w):
    if w.paged:
        return oracle.KVCache(k=w.k, v=w.v, kv_indptr=w.kv_indptr, paged=True,
                              page_indices=w.page_indices, kv_len=w.kv_len, page_size=w.page_size)
    return oracle.KVCache(k=w.k, v=w.v, kv_indptr=w.kv_indptr)


def host_workers():
    """Oracle worker threads: every core this process may run on."""
    return oracle.sink_attention.default_workers()


def oracle_full(w, window, sinks=True, workers=None):
    return oracle.sink_attention_ref(w.q, w.qo_indptr, kv_cache(w), w.sinks if sinks else None,
                                     w.scale, window, workers=workers or host_workers())


def assert_parity_by_request(w, g, r, what, lse_g, lse_r, requests=None):
    """assert_parity on each request's rows in turn (bounds the temporaries of
    full-size comparisons)."""
    for b in (range(w.batch) if requests is None else requests):
        lo, hi = int(w.qo_indptr[b]), int(w.qo_indptr[b + 1])
        assert_parity(g[lo:hi], r[lo:hi], f"{what} request {b}", lse_g[lo:hi], lse_r[lo:hi])


def assert_parity(g, r, what, lse_g=None, lse_r=None):
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite GPU output"
    err = np.abs(g - r)
    bound = ATOL + RTOL * np.abs(r)
    bad = err > bound
    big = np.abs(r) >= 1e-2
    max_rel = float((err[big] / np.abs(r[big])).max()) if big.any() else 0.0
    say(f"{what}: max_abs={err.max():.3e} max_rel(|r|>=1e-2)={max_rel:.3e} n={g.size}")
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements out of tolerance; worst excess "
                           f"{float((err - bound).max()):.3e} at {np.unravel_index(np.argmax(err - bound), g.shape)}")
    gn = np.linalg.norm(g, axis=-1)
    rn = np.linalg.norm(r, axis=-1)
    nbad = np.abs(gn - rn) > NORM_RTOL * rn + 1e-6
    assert not nbad.any(), f"{what}: {int(nbad.sum())} rows fail the norm guard"
    if lse_g is not None:
        lg = np.asarray(lse_g, dtype=np.float64)
        lr = np.asarray(lse_r, dtype=np.float64)
        inf_r = ~np.isfinite(lr)
        assert np.array_equal(lg[inf_r], lr[inf_r]), f"{what}: infinite LSE entries differ"
        d = np.abs(lg[~inf_r] - lr[~inf_r])
        assert d.size == 0 or d.max() <= LSE_ATOL, f"{what}: LSE off by {d.max():.3e}"
