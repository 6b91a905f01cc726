"""Pins for the oracle's OCP E4M3FN codec and bf16 rounding.

The codec is checked against PyTorch's independent float8_e4m3fn
implementation (a library routine), against the anchor values of the OCP
definition, and against brute-force nearest-value search.
"""
import numpy as np
import pytest
import torch

from oracle import vc_oracle as O

ALL = np.arange(256, dtype=np.uint8)


def finite_table():
    vals = O.e4m3_decode(ALL)
    ok = ~np.isnan(vals)
    return ALL[ok], vals[ok]


def test_decode_matches_torch_all_codes():
    ref = torch.from_numpy(ALL.copy()).view(torch.float8_e4m3fn).double().numpy()
    got = O.e4m3_decode(ALL)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    m = ~np.isnan(ref)
    assert np.array_equal(ref[m], got[m])
    assert np.array_equal(np.signbit(ref[m]), np.signbit(got[m]))


def test_decode_anchor_values():
    # the OCP OFP8 specification's named E4M3 points (tests/golden/ocp_e4m3_anchors.txt)
    from golden import rows
    d = O.e4m3_decode
    anchors = rows("ocp_e4m3_anchors.txt")
    assert len(anchors) == 11
    for code, value, *_ in anchors:
        got, want = float(d(int(code, 16))), float(value)
        if np.isnan(want):
            assert np.isnan(got), code
        else:
            assert got == want and np.signbit(got) == np.signbit(want), (code, got, want)
    assert np.sum(~np.isnan(O.e4m3_decode(ALL))) == 254
    # codes 0..126 are strictly increasing in value
    assert np.all(np.diff(O.e4m3_decode(np.arange(127))) > 0)


def test_encode_decode_roundtrip():
    codes, vals = finite_table()
    assert np.array_equal(O.e4m3_encode(vals), codes)


def test_encode_matches_torch_dense_grid_and_midpoints():
    _, vals = finite_table()
    pos = np.unique(np.abs(vals))
    mids = (pos[1:] + pos[:-1]) / 2
    rng = np.random.default_rng(0)
    dense = rng.uniform(-448, 448, 20000)
    small = rng.uniform(-0.05, 0.05, 20000)
    x = np.concatenate([vals, mids, -mids, dense, small, mids * (1 + 1e-9), mids * (1 - 1e-9)])
    x = x[np.abs(x) <= 448]
    x32 = x.astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = O.e4m3_encode(x32.astype(np.float64))
    assert np.array_equal(ref, got)


def test_encode_bruteforce_nearest_ties_to_even():
    codes, vals = finite_table()
    rng = np.random.default_rng(1)
    pos = np.unique(np.abs(vals))
    mids = (pos[1:] + pos[:-1]) / 2
    xs = np.concatenate([rng.uniform(0, 448, 3000), mids, rng.uniform(0, 2 ** -5, 500)])
    nonneg = codes < 0x80
    c0, v0 = codes[nonneg], vals[nonneg]
    for x in xs:
        dist = np.abs(v0 - x)
        best = np.flatnonzero(dist == dist.min())
        if best.size > 1:                       # tie: the even code (mantissa LSB 0)
            best = best[(c0[best] & 1) == 0]
        assert O.e4m3_encode(x) == c0[best[0]], x


def test_encode_saturates_and_signs():
    for x in (448.0, 448.5, 463.9, 464.0, 500.0, 1e6, np.inf):
        assert O.e4m3_encode(x) == 0x7E
        assert O.e4m3_encode(-x) == 0xFE
    assert O.e4m3_encode(0.0) == 0x00
    assert O.e4m3_encode(-0.0) == 0x80
    assert O.e4m3_encode(-1e-30) == 0x80
    assert O.e4m3_encode(2.0 ** -10) == 0x00       # exact half of the smallest subnormal: ties to even (0)
    assert O.e4m3_encode(3 * 2.0 ** -10) == 0x02   # 1.5 quanta -> 2 (even)


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-5, 5, 20000),
                        [0.0, 1.0, -3.0, 1e-30]])
    x32 = x.astype(np.float32).astype(np.float64)   # torch rounds from fp32: compare on fp32 inputs
    ref = torch.from_numpy(x32).to(torch.bfloat16).double().numpy()
    assert np.array_equal(O.bf16_round(x32), ref)
