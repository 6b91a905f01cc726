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
    _fails(TA.test_pipeline_config2_heads_accuracy_and_vsmooth_benefit)
