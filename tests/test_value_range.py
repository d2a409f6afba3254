"""The value range of V that the kernels accept (no GPU needed).

The P.V products run on fp16 matrix instructions, so V is converted from
bf16 to fp16 when it is staged.  These checks pin the boundary that
include/sinkattn.h states as a precondition: every bf16 value with
|v| <= 65280 converts to fp16 exactly (apart from magnitudes below 2^-14,
which land on fp16 subnormals within 2^-25), and the next bf16 magnitude,
65536, overflows fp16.  The conversion rule is IEEE round to nearest even,
which numpy's float32 -> float16 cast implements.
"""

import os
import re

import numpy as np

from gqa_attention_sinks_amd import workloads as wl

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "sinkattn.h")


def _all_bf16():
    bits = np.arange(1 << 16, dtype=np.uint32)
    return (bits << 16).view(np.float32)


def test_largest_bf16_below_fp16_overflow_is_65280():
    x = _all_bf16()
    fin = np.isfinite(x)
    ok = fin & (np.abs(x) < 65520.0)          # fp16's rounding boundary to infinity
    assert np.abs(x[ok]).max() == 65280.0
    assert np.float16(np.float32(65280.0)) == 65280.0
    with np.errstate(over="ignore"):
        assert np.isinf(np.float16(np.float32(65536.0)))
    # 65280 is a bf16 value and 65504 (fp16's largest) is not
    assert wl.bf16_bits(np.float32(65280.0)) == 0x477F
    assert wl.bf16_bits(np.float32(65504.0)) == 0x4780    # rounds up to 65536


def test_every_bf16_in_range_converts_exactly_or_within_subnormal_rounding():
    x = _all_bf16()
    inr = np.isfinite(x) & (np.abs(x) <= 65280.0)
    h = x[inr].astype(np.float16).astype(np.float32)
    normal = np.abs(x[inr]) >= 2.0 ** -14
    assert np.array_equal(h[normal], x[inr][normal])
    assert np.all(np.abs(h[~normal] - x[inr][~normal]) <= 2.0 ** -25)
    # and every finite bf16 above the bound overflows
    out = np.isfinite(x) & (np.abs(x) > 65280.0)
    with np.errstate(over="ignore"):
        assert np.all(np.isinf(x[out].astype(np.float16)))


def test_header_states_the_precondition():
    text = open(HEADER).read()
    assert re.search(r"\|v\| <= 65280", text)
    for call in ("sinkattn_prefill", "sinkattn_decode_paged", "sinkattn_decode_paged_multi"):
        assert call in text[text.index("Value range"):text.index("#ifndef SINKATTN_H_")]
