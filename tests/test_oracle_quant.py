"""Pins for block quantisation, block means and the residual repair set."""
import numpy as np
import torch

from oracle import vc_oracle as O


def test_amax_quant_matches_torch_cast_and_hits_448():
    rng = np.random.default_rng(0)
    for scale in (1e-4, 1.0, 37.0):
        x = (rng.standard_normal((128, 128)) * scale).astype(np.float32)
        codes, s = O.quantize_amax(x)
        inv = np.float32(448.0) / np.float32(np.abs(x).max())
        ref = torch.from_numpy((x * inv).astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(codes, ref)
        assert np.abs(O.e4m3_decode(codes)).max() == 448.0
        assert s == np.float32(np.abs(x).max()) / np.float32(448.0)


def test_amax_quant_error_bound():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((128, 128)) * 3).astype(np.float32)
    codes, s = O.quantize_amax(x)
    deq = O.e4m3_decode(codes) * float(s)
    err = np.abs(deq - x)
    # RNE with 3 mantissa bits: half an ulp = 2^-4 relative for normals, 2^-10*s below 2^-6*s
    bound = np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * float(s)) * (1 + 1e-6)
    assert np.all(err <= bound)


def test_quant_blocks_partial_tail_and_zero_block():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((300, 128)).astype(np.float32)
    x[128:256] = 0.0
    codes, sc = O.quantize_blocks(x)
    assert sc.shape == (3,)
    assert sc[1] == 1.0 and not np.any(codes[128:256])
    c2, s2 = O.quantize_amax(x[256:])
    assert np.array_equal(codes[256:], c2) and sc[2] == s2


def test_block_means_and_residual_sum_to_zero():
    rng = np.random.default_rng(3)
    v = (rng.standard_normal((300, 128)) + 5).astype(np.float32).astype(np.float64)
    mu = O.block_means(v)
    for b, sl in enumerate((slice(0, 128), slice(128, 256), slice(256, 300))):
        assert np.allclose(mu[b], v[sl].mean(axis=0), rtol=2 ** -23, atol=0)
        r = v[sl] - mu[b].astype(np.float64)
        assert np.all(np.abs(r.sum(axis=0)) <= sl.stop * 2 ** -22 * 6)


def test_prepare_v_quantises_residual_per_head():
    rng = np.random.default_rng(4)
    v = rng.standard_normal((400, 128)) + 10 * rng.standard_normal((1, 128))
    v = v.astype(np.float32).astype(np.float64)
    hv = O.prepare_v_head(v, k=4, iters=2)
    assert np.abs(O.e4m3_decode(hv.v8)).max() == 448.0
    assert hv.v_scale == np.float32(np.abs(hv.resid).max()) / np.float32(448)
    # mean restore: mu_b + R reproduces the permuted V to fp32 rounding
    mu_rows = np.repeat(hv.mean.astype(np.float64), 128, axis=0)[:400]
    assert np.allclose(mu_rows + hv.resid, v[hv.perm], rtol=0, atol=2 ** -20 * np.abs(v).max())


def test_repair_set_is_worst_rounded_tokens():
    rng = np.random.default_rng(5)
    v = rng.standard_t(3, (1000, 128))
    hv = O.prepare_v_head(v, k=8, iters=2, repair_budget=0.005)
    n = O.repair_count(0.005, 1000)
    assert n == 5 and hv.rep_pos.size == 5
    deq = O.e4m3_decode(hv.v8) * float(hv.v_scale)
    errn = ((hv.resid - deq) ** 2).sum(axis=1)
    worst = np.argsort(-errn, kind="stable")[:5]
    assert set(worst.tolist()) == set(hv.rep_pos.tolist())
    # e8 quantises the residual error with its own amax scale
    e = (hv.resid - (np.float32(hv.v_scale) * O.e4m3_decode(hv.v8).astype(np.float32))).astype(np.float32)
    c, s = O.quantize_amax(e[hv.rep_pos])
    assert np.array_equal(c, hv.rep_e8) and s == hv.rep_scale


def test_repair_count():
    # ceil(beta * S) with beta as the fp32 the call carries
    assert O.repair_count(0.005, 32768) == 164          # 163.84 -> 164
    assert O.repair_count(0.0, 32768) == 0
    assert O.repair_count(0.5, 3) == 2                  # 1.5 -> 2
    assert O.repair_count(0.0011, 1000) == 2            # fp32 0.0011 * 1000 = 1.09999... -> 2, not 1
    assert O.repair_count(0.25, 8) == 2                 # exact: no rounding up
    assert O.repair_count(0.999, 10) == 10              # capped at S
