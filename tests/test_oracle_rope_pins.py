"""Pins of the fp64 append + rotary reference (oracle/rope_append.py)
against things other than itself: a hand-worked rotation, the complex
multiplication form of a 2-D rotation (numpy complex arithmetic), rotation
invariants (norm, inverse, relative position), and a pure-Python placement
of the appended rows into the page pool, plus planted mistakes that must fail.

Sources: "GPT-OSS on day 0", section "GPT-OSS on Hopper" (YaRN rotary
position encoding); "Accelerating Sonar through speculation", section
"Inference with speculative decoding" (per-request KV pages, CPU-built page
tables).
"""

import numpy as np
import pytest

import oracle
import oracle.rope_append as ra


def rotary_table(max_pos, base=10000.0, d=64):
    """A genuine rotary table: pair f turns by pos * base^(-2f/d)."""
    f = np.arange(d // 2)
    ang = np.arange(max_pos)[:, None] * base ** (-2.0 * f / d)[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1)


@pytest.mark.parametrize("interleaved", [False, True])
def test_hand_worked_quarter_turn(interleaved):
    # one vector, unit value on the first element of pair 0; the table turns
    # pair 0 by a quarter turn (cos 0, sin 1) and leaves pair 1 alone
    table = np.zeros((1, 64))
    table[0, :32] = 1.0
    table[0, 0], table[0, 32] = 0.0, 1.0
    x = np.zeros(64)
    x[0] = 1.0
    second = 1 if interleaved else 32          # the partner of element 0
    y = ra.rotate(x, 0, table, interleaved)
    expect = np.zeros(64)
    expect[second] = 1.0                       # (1, 0) -> (0, 1)
    np.testing.assert_array_equal(y, expect)
    # pair 1 untouched by a zero angle: (x2, x3) or (x1, x33) = (2, 3) stays
    x = np.zeros(64)
    i, j = (2, 3) if interleaved else (1, 33)
    x[i], x[j] = 2.0, 3.0
    np.testing.assert_array_equal(ra.rotate(x, 0, table, interleaved), x)


@pytest.mark.parametrize("interleaved", [False, True])
def test_rotation_is_complex_multiplication(interleaved):
    rng = np.random.default_rng(11)
    table = rotary_table(300)
    x = rng.normal(size=(50, 3, 64))
    pos = rng.integers(0, 300, size=(50, 1))
    y = ra.rotate(x, pos, table, interleaved)
    i, j = (np.arange(0, 64, 2), np.arange(1, 64, 2)) if interleaved else (np.arange(32), np.arange(32, 64))
    z = (x[..., i] + 1j * x[..., j]) * (table[pos][..., :32] + 1j * table[pos][..., 32:])
    np.testing.assert_allclose(y[..., i], z.real, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(y[..., j], z.imag, rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("interleaved", [False, True])
def test_rotation_invariants(interleaved):
    rng = np.random.default_rng(12)
    table = rotary_table(4096)
    x = rng.normal(size=(200, 64))
    pos = rng.integers(0, 4096, size=200)
    y = ra.rotate(x, pos, table, interleaved)
    i, j = (np.arange(0, 64, 2), np.arange(1, 64, 2)) if interleaved else (np.arange(32), np.arange(32, 64))
    np.testing.assert_allclose(y[:, i] ** 2 + y[:, j] ** 2, x[:, i] ** 2 + x[:, j] ** 2, rtol=1e-12)
    back = table.copy()
    back[:, 32:] *= -1.0                       # the inverse rotation
    np.testing.assert_allclose(ra.rotate(y, pos, back, interleaved), x, rtol=1e-12, atol=1e-12)
    # relative position: <R(q, p), R(k, p')> depends on p - p' only
    q, k = rng.normal(size=64), rng.normal(size=64)
    for p, pp, dlt in [(5, 3, 100), (1000, 20, 7), (0, 0, 4000)]:
        a = ra.rotate(q, p, table, interleaved) @ ra.rotate(k, pp, table, interleaved)
        b = ra.rotate(q, p + dlt, table, interleaved) @ ra.rotate(k, pp + dlt, table, interleaved)
        assert abs(a - b) < 1e-10


def _tiny_append(rng, hq=4, hkv=2, page_size=16):
    kv_len = np.array([5, 17, 40, 1])
    n_new = np.array([2, 1, 17, 1])
    append_indptr = np.concatenate([[0], np.cumsum(n_new)])
    n_pages = (kv_len + page_size - 1) // page_size
    page_indptr = np.concatenate([[0], np.cumsum(n_pages)])
    pool = int(page_indptr[-1]) + 3
    page_indices = rng.permutation(pool)[: page_indptr[-1]]
    t = int(append_indptr[-1])
    return dict(q=rng.normal(size=(t, hq, 64)), k=rng.normal(size=(t, hkv, 64)), v=rng.normal(size=(t, hkv, 64)),
                append_indptr=append_indptr, kv_len=kv_len, page_indptr=page_indptr, page_indices=page_indices,
                k_pool=np.full((pool, hkv, page_size, 64), np.nan), v_pool=np.full((pool, hkv, page_size, 64), np.nan),
                table=rotary_table(64))


def _run(p, interleaved, **over):
    a = dict(p, **over)
    return oracle.append_rope_ref(a["q"], a["k"], a["v"], a["append_indptr"], a["kv_len"], a["page_indptr"],
                                  a["page_indices"], a["k_pool"], a["v_pool"], a["table"], interleaved)


@pytest.mark.parametrize("interleaved", [False, True])
def test_placement_brute_force(interleaved):
    rng = np.random.default_rng(13)
    p = _tiny_append(rng)
    q_out, kp, vp = _run(p, interleaved)
    # pure-Python placement: walk the requests, count positions by hand
    written = {}
    t = 0
    for b in range(len(p["kv_len"])):
        n = p["append_indptr"][b + 1] - p["append_indptr"][b]
        for i in range(n):
            pos = p["kv_len"][b] - n + i
            page = p["page_indices"][p["page_indptr"][b] + pos // 16]
            written[(int(page), int(pos % 16))] = (t, int(pos))
            t += 1
    assert t == len(p["q"])
    for (page, slot), (tok, pos) in written.items():
        np.testing.assert_array_equal(vp[page, :, slot], p["v"][tok])
        np.testing.assert_allclose(kp[page, :, slot], ra.rotate(p["k"][tok], pos, p["table"], interleaved),
                                   rtol=1e-15)
        np.testing.assert_allclose(q_out[tok], ra.rotate(p["q"][tok], pos, p["table"], interleaved), rtol=1e-15)
    untouched = np.ones(kp.shape[:1] + kp.shape[2:3], dtype=bool)
    for page, slot in written:
        untouched[page, slot] = False
    assert np.isnan(kp.transpose(0, 2, 1, 3)[untouched]).all()
    assert np.isnan(vp.transpose(0, 2, 1, 3)[untouched]).all()


def test_planted_mistakes_are_caught(monkeypatch):
    rng = np.random.default_rng(14)
    table = rotary_table(300)
    x = rng.normal(size=(20, 64))
    pos = rng.integers(1, 300, size=(20,))

    def complex_form(y, interleaved):
        i, j = (np.arange(0, 64, 2), np.arange(1, 64, 2)) if interleaved else (np.arange(32), np.arange(32, 64))
        z = (x[:, i] + 1j * x[:, j]) * (table[pos][:, :32] + 1j * table[pos][:, 32:])
        return np.allclose(y[:, i], z.real) and np.allclose(y[:, j], z.imag)

    good = ra.rotate(x, pos, table, False)
    assert complex_form(good, False)
    assert not complex_form(ra.rotate(x, pos, table, True), False)          # wrong pairing
    assert not complex_form(ra.rotate(x, pos - 1, table, False), False)     # position off by one
    flipped = table.copy()
    flipped[:, 32:] *= -1.0
    assert not complex_form(ra.rotate(x, pos, flipped, False), False)       # sign of sin
    # a placement off by one position is caught by the brute force
    orig = ra.append_positions
    monkeypatch.setattr(ra, "append_positions", lambda ai, kl: (orig(ai, kl)[0], orig(ai, kl)[1] - 1))
    with pytest.raises(AssertionError):
        test_placement_brute_force(False)
