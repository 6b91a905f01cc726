"""Pins of the oracle's 4-bit residual path (reading R15: OCP MXFP4 -- E2M1
codes with one power-of-two scale per channel and run of 32 consecutive
permuted positions of a 128-key tile).

The 4-bit option is named in "Nunchux AI lanza VC-Attention kernel ..."
(reditua.com), paragraph 2 (NVFP4 beside E4M3); the format details are the
reading stated in the oracle.  Nothing here calls the GPU.
"""
import numpy as np
import pytest

from oracle import vc_oracle as O


# --------------------------------------------------------------- E2M1 codec
def test_e2m1_decode_matches_the_mx_specification_table():
    # every code against the OCP MX specification's E2M1 values
    # (tests/golden/ocp_e2m1_values.txt), signs of zero included
    from golden import rows
    table = rows("ocp_e2m1_values.txt")
    assert len(table) == 16
    d = O.e2m1_decode(np.arange(16))
    for code, value in table:
        got, want = float(d[int(code, 16)]), float(value)
        assert got == want and np.signbit(got) == np.signbit(want), (code, got, want)


def test_e2m1_decode_is_the_2e1m_float_with_bias_1():
    # Properties that fix a 1-sign, 2-exponent, 1-mantissa float with
    # exponent bias 1: code 2 (exponent 1, mantissa 0) is 1.0; each exponent
    # step doubles the value; the two codes of one exponent differ by half an
    # octave step; the subnormal code 1 is half of 1.0; code 0 is zero; bit 3
    # is the sign; the largest value is 2^(3-1) * 1.5 = 6.
    d = O.e2m1_decode(np.arange(16))
    assert d[0] == 0.0 and d[2] == 1.0 and d[1] == 0.5 and d[7] == 6.0
    for c in range(2, 6):
        assert d[c + 2] == 2 * d[c]                       # exponent step
    for c in (2, 4, 6):
        assert d[c + 1] == 1.5 * d[c]                     # mantissa bit
    assert np.all(np.diff(d[:8]) > 0)
    assert np.array_equal(d[8:], -d[:8])


def _nearest_even(x):
    """Brute force: the code whose value is nearest to clamp(|x|, 6); ties to the
    code with mantissa bit 0; sign bit from x."""
    grid = [O.e2m1_decode(c).item() for c in range(8)]
    a = min(abs(x), 6.0)
    best = None
    for c in range(8):
        dist = abs(grid[c] - a)
        if best is None or dist < best[0] or (dist == best[0] and c % 2 == 0):
            best = (dist, c)
    return best[1] | (8 if np.signbit(x) else 0)


def test_e2m1_encode_brute_force_with_ties_and_saturation():
    grid = O.e2m1_decode(np.arange(8))
    mids = (grid[1:] + grid[:-1]) / 2
    xs = np.concatenate([grid, mids, -grid, -mids, [6.5, 7.0, 100.0, -9.0, 1e-30, -1e-30, 0.0, -0.0],
                         np.random.default_rng(0).uniform(-8, 8, 4000)])
    got = O.e2m1_encode(xs)
    want = np.array([_nearest_even(float(x)) for x in xs])
    assert np.array_equal(got, want)


# ---------------------------------------------------------- group scale rule
def test_scale_exponent_is_the_smallest_power_of_two_without_clipping():
    rng = np.random.default_rng(1)
    a = np.concatenate([np.float32(6) * np.float32(2.0) ** np.arange(-20, 20),       # exact boundaries
                        rng.lognormal(0, 6, 5000).astype(np.float32)]).astype(np.float64)
    e = O.mx_scale_exponent(a)
    assert np.all(a / np.ldexp(1.0, e) <= 6.0)
    assert np.all(a / np.ldexp(1.0, e - 1) > 6.0)
    assert O.mx_scale_exponent(np.array([0.0]))[0] == 0


# -------------------------------------------------------------------- groups
def test_groups_are_runs_of_32_positions_of_one_tile_and_channel():
    # Behavioural pin of the grouping: raising one residual value far above
    # the rest moves the scale exponent of exactly one (tile, channel, group)
    # -- the tile of its position, its channel, and the run of 32 consecutive
    # permuted positions (32u .. 32u+31 of the tile) that holds it -- and no
    # other.  A grouping over other key sets (strided keys, 16-key runs,
    # groups crossing tiles or channels) moves other exponents or none.
    rng = np.random.default_rng(7)
    S = 300
    r = (rng.uniform(0.8, 1.0, (S, 128)) * rng.choice([-1, 1], (S, 128))).astype(np.float32)
    _, base = O.quantize_mxfp4(r)
    # max|R| in (0.75, 1.5] -> 2^-2; groups past S=300 (tile 2, groups 2-3) hold no key
    assert np.all(base[:2] == -2) and np.all(base[2, :, :2] == -2) and np.all(base[2, :, 2:] == 0)
    for p, d in ((0, 0), (31, 5), (32, 5), (95, 127), (96, 64), (127, 3), (128, 9), (200, 100), (299, 77)):
        r2 = r.copy()
        r2[p, d] = np.float32(100.0)                 # needs 2^5 (100/32 <= 6 < 100/16)
        _, e2 = O.quantize_mxfp4(r2)
        changed = np.argwhere(e2 != base)
        assert changed.tolist() == [[p // 128, d, (p % 128) // 32]], (p, d, changed.tolist())
        assert e2[p // 128, d, (p % 128) // 32] == 5


# ------------------------------------------------------------ the quantiser
@pytest.mark.parametrize("S", [128, 300, 33])
def test_quantize_mxfp4_per_group_properties(S):
    rng = np.random.default_rng(S)
    r = (rng.standard_normal((S, 128)) * rng.lognormal(0, 3, (1, 128))).astype(np.float32)
    r[:5, 7] = 0.0
    codes, expo = O.quantize_mxfp4(r)
    vals = O.mxfp4_dequant(codes, expo)
    grp = (np.arange(S) % 128) // 32                  # 32 consecutive permuted positions per group
    for b in range((S + 127) // 128):
        for gg in range(4):
            sel = (np.arange(S) // 128 == b) & (grp == gg)
            if not sel.any():
                continue
            amax = np.abs(r[sel].astype(np.float64)).max(axis=0)
            assert np.array_equal(expo[b, :, gg], O.mx_scale_exponent(amax))
            X = np.ldexp(1.0, expo[b, :, gg])
            assert np.array_equal(codes[sel], O.e2m1_encode(r[sel] / X))
            # within one grid step (at most 2 in [4,6]) of the scaled value, i.e. |R - V| <= X
            assert np.all(np.abs(r[sel] - vals[sel]) <= X)
    # values on the grid of one power of two per channel come back exactly
    # (every group's scale divides them into grid values again)
    exact = (O.e2m1_decode(rng.integers(0, 16, (128, 128))) * 2.0 ** rng.integers(-20, 20, (1, 128))).astype(np.float32)
    c2, e2 = O.quantize_mxfp4(exact)
    assert np.array_equal(O.mxfp4_dequant(c2, e2), exact.astype(np.float64))


def test_mxfp4_residual_attention_envelope():
    # the whole oracle path with the 4-bit residual: within a loose envelope of
    # exact attention, and less accurate than the 8-bit residual on the same head
    import synth
    w = synth.workload(2, H=1, S=1024)
    q, k, v = (t[0, :, 0].double().numpy() for t in synth.generate(w, "cpu"))
    rows = np.arange(0, 1024, 7)
    ex = O.attention_exact(q, k, v, rows=rows)
    errs = {}
    for fmt in ("e4m3", "mxfp4"):
        hv = O.prepare_v_head(v, k=w.k, iters=w.iters, v_format=fmt)
        hq = O.prepare_qk_head(q, k, hv.perm)
        errs[fmt] = O.rel_l2(O.attend_head(hq, hv, rows), ex)
    assert errs["mxfp4"] < 0.08
    assert errs["mxfp4"] > errs["e4m3"]
    with pytest.raises(ValueError):
        O.prepare_v_head(v, k=w.k, iters=w.iters, v_format="mxfp4", repair_budget=0.01)
