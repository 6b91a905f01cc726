"""Planted mistakes in the oracle must be caught by its pins.

Each test patches one oracle function with a plausible bug (on the CPU only)
and checks that the pin guarding that step fails.
"""
import numpy as np
import pytest

from oracle import vc_oracle as O
import tests.test_oracle_attention as TA
import tests.test_oracle_codec as TC
import tests.test_oracle_kmeans as TK
import tests.test_oracle_mxfp4 as TM
import tests.test_oracle_quant as TQ


def _fails(fn):
    with pytest.raises(AssertionError):
        fn()


def test_argmax_instead_of_argmin(monkeypatch):
    good = O.kmeans_assign
    monkeypatch.setattr(O, "kmeans_assign", lambda x, c: np.argmax(
        (c.astype(float) ** 2).sum(1)[None] - 2.0 * x.astype(float) @ c.T.astype(float), axis=1))
    _fails(TK.test_assign_equals_bruteforce_distances)
    del good


def test_sign_flip_in_distance(monkeypatch):
    monkeypatch.setattr(O, "kmeans_assign", lambda x, c: np.argmin(
        (c.astype(float) ** 2).sum(1)[None] + 2.0 * x.astype(float) @ c.T.astype(float), axis=1))
    _fails(TK.test_assign_equals_bruteforce_distances)


def test_update_truncates_instead_of_rounding(monkeypatch):
    def bad(x, assign, cent):
        k = cent.shape[0]
        new = cent.copy()
        for c in range(k):
            m = x[assign == c]
            if len(m):
                new[c] = m.sum(0) // len(m)
        return new
    monkeypatch.setattr(O, "kmeans_update", bad)
    _fails(TK.test_update_is_mean_rounded_half_up_exact)


def test_init_phase_from_seed_plus_bh(monkeypatch):
    def bad(S, k, seed, bh):
        stride = max(1, S // k)
        phi = O.splitmix64((seed + bh) & O.MASK64) % stride
        return np.array([(c * S) // k + phi for c in range(k)], dtype=np.int64)
    monkeypatch.setattr(O, "init_positions", bad)
    _fails(TK.test_init_positions_values_from_published_outputs)


def test_init_starts_from_truncated_stride(monkeypatch):
    def bad(S, k, seed, bh):
        stride = max(1, S // k)
        phi = O.splitmix64((seed ^ bh) & O.MASK64) % stride
        return np.array([c * stride + phi for c in range(k)], dtype=np.int64)
    monkeypatch.setattr(O, "init_positions", bad)
    _fails(TK.test_init_positions_values_from_published_outputs)


def test_seven_codes_per_octave(monkeypatch):
    good = O.expcast_codes
    monkeypatch.setattr(O, "expcast_codes", lambda a, s8, m: good(a, np.float32(7 / 8) * s8, m))
    _fails(TA.test_expcast_closed_form_grid)


def test_max_maps_to_wrong_code(monkeypatch):
    good = O.expcast_codes
    monkeypatch.setattr(O, "expcast_codes", lambda a, s8, m: good(a, s8, np.asarray(m) + 0.125))
    _fails(TA.test_expcast_closed_form_grid)


def test_encode_rounds_half_away(monkeypatch):
    def bad(x):
        x = np.asarray(x, np.float64)
        a = np.abs(x)
        _, e = np.frexp(a)
        q = np.ldexp(1.0, np.maximum(e - 1, -6) - 3)
        val = np.minimum(np.floor(a / q + 0.5) * q, 448.0)
        return good(np.copysign(val, x))          # val is exact in E4M3
    good = O.e4m3_encode
    monkeypatch.setattr(O, "e4m3_encode", bad)
    _fails(TC.test_encode_bruteforce_nearest_ties_to_even)


def test_block_mean_off_by_one_count(monkeypatch):
    def bad(vp, block=128):
        S, D = vp.shape
        nb = (S + block - 1) // block
        mu = np.empty((nb, D), np.float32)
        for b in range(nb):
            blk = vp[b * block:min(S, (b + 1) * block)]
            mu[b] = (blk.sum(0) / (blk.shape[0] + 1)).astype(np.float32)
        return mu
    monkeypatch.setattr(O, "block_means", bad)
    _fails(TQ.test_block_means_and_residual_sum_to_zero)


def test_missing_log2e_in_sigma(monkeypatch):
    monkeypatch.setattr(O, "sigma_of", lambda sq, sk, sm: (np.asarray(sq, np.float32) * np.asarray(sk, np.float32)
                                                           * np.float32(sm)).astype(np.float32))
    _fails(TA.test_softmax_temperature_two_keys)


def test_mx_groups_strided_keys(monkeypatch):
    # groups as every fourth run of 4 keys (a strided lane-style set) instead
    # of 32 consecutive positions
    monkeypatch.setattr(O, "mx_group_of_key", lambda j: (np.asarray(j, np.int64) % 16) // 4)
    _fails(TM.test_groups_are_runs_of_32_positions_of_one_tile_and_channel)


def test_mx_groups_of_16(monkeypatch):
    monkeypatch.setattr(O, "mx_group_of_key", lambda j: ((np.asarray(j, np.int64) % 128) // 16) % 4)
    _fails(TM.test_groups_are_runs_of_32_positions_of_one_tile_and_channel)


def _sketch_with(shift_base, lo, hi):
    import math

    def bad(v):
        v = np.asarray(v, dtype=np.float64)
        a = float(np.max(np.abs(v))) if v.size else 0.0
        if a == 0.0:
            return np.zeros(v.shape, dtype=np.int64)
        _, e = math.frexp(a)
        return np.clip(np.rint(np.ldexp(v, shift_base + 1 - e)), lo, hi).astype(np.int64)
    return bad


def test_sketch_eight_bits(monkeypatch):
    # the narrower sketch (max|v| scaled into [64, 128), int8 clamp)
    monkeypatch.setattr(O, "sketch", _sketch_with(6, -128, 127))
    _fails(TK.test_sketch_exact_values)
    _fails(TK.test_sketch_scaling_and_range)


def test_sketch_clamp_asymmetric(monkeypatch):
    monkeypatch.setattr(O, "sketch", _sketch_with(7, -256, 255))
    _fails(TK.test_sketch_exact_values)


def test_e4m3_subnormals_scaled_as_normals(monkeypatch):
    def bad(codes):
        c = np.asarray(codes).astype(np.int64)
        e, m = (c >> 3) & 15, c & 7
        mag = np.where(e == 0, m * 2.0 ** -6, np.ldexp(1.0 + m / 8.0, e - 7))   # subnormal step 2^-6, not 2^-9
        mag = np.where((e == 15) & (m == 7), np.nan, mag)
        return np.where(c >> 7 == 1, -mag, mag)
    monkeypatch.setattr(O, "e4m3_decode", bad)
    _fails(TC.test_decode_matches_torch_all_codes)


def test_amax_scale_from_inverse(monkeypatch):
    # the stored scale taken as 1/inv instead of a/448 (differs in the last fp32 bit for some a)
    def bad(x32):
        x32 = np.asarray(x32, dtype=np.float32)
        a = np.float32(np.max(np.abs(x32)))
        inv = np.float32(448.0) / a if a else np.float32(1.0)
        s = (np.float32(1.0) / inv) if a else np.float32(1.0)
        return O.e4m3_encode((x32 * inv).astype(np.float32)), np.float32(s)
    monkeypatch.setattr(O, "quantize_amax", bad)
    _fails(TQ.test_amax_quant_matches_torch_cast_and_hits_448)


def test_repair_count_rounds_to_nearest(monkeypatch):
    monkeypatch.setattr(O, "repair_count", lambda beta, S: 0 if beta <= 0 else min(S, int(round(float(beta) * S))))
    _fails(TQ.test_repair_count)


def test_cluster_order_unstable(monkeypatch):
    monkeypatch.setattr(O, "cluster_perm", lambda a: np.argsort(-np.asarray(a), kind="stable")[::-1].astype(np.int64))
    _fails(TK.test_perm_is_stable_bijection)


def test_e2m1_ties_away_from_zero(monkeypatch):
    def bad(x):
        x = np.asarray(x, dtype=np.float64)
        grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
        a = np.minimum(np.abs(x), 6.0)
        # nearest grid point, ties to the larger magnitude
        idx = np.searchsorted(grid, a, side="left")
        idx = np.clip(idx, 1, 7)
        lo, hi = grid[idx - 1], grid[idx]
        pick = np.where(a - lo >= hi - a, idx, idx - 1)
        code = pick.astype(np.int64)
        return (code | np.where(np.signbit(x), 8, 0)).astype(np.uint8)
    monkeypatch.setattr(O, "e2m1_encode", bad)
    _fails(TM.test_e2m1_encode_brute_force_with_ties_and_saturation)


def test_mx_scale_always_rounds_up(monkeypatch):
    def bad(amax):
        a = np.asarray(amax, dtype=np.float64)
        e = np.zeros(a.shape, dtype=np.int64)
        nz = a > 0
        _, ex = np.frexp(a[nz] / 6.0)
        e[nz] = ex                                   # one too large for exact powers of two
        return np.clip(e, -127, 127)
    monkeypatch.setattr(O, "mx_scale_exponent", bad)
    _fails(TM.test_scale_exponent_is_the_smallest_power_of_two_without_clipping)
