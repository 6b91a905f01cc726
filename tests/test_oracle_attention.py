"""Pins for ExpCast and the oracle's online-softmax attention.

Reference points: PyTorch's scaled_dot_product_attention in float64 (a
library routine), closed forms of the ExpCast map, the mean-restore and
joint-permutation identities with quantisation switched off, and the
accuracy envelope against exact attention.
"""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import vc_oracle as O


def _head(seed, S=300, off=0.0, outl=0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((S, 128))
    k = rng.standard_normal((S, 128)) * 1.5
    v = rng.standard_normal((S, 128)) + off * rng.standard_normal((1, 128))
    if outl:
        idx = rng.choice(S, outl, replace=False)
        v[idx] *= 30
    f = lambda a: a.astype(np.float32).astype(np.float64)
    return f(q), f(k), f(v)


# ---------------------------------------------------------------- ExpCast map
def test_expcast_closed_form_grid():
    # t - M = -n + j/8 exactly  ->  code 120 - 8n + j, value 2^(8-n) (1 + j/8)
    for n in range(0, 15):
        for j in range(8):
            if n == 0 and j > 0:
                continue
            t = np.array([[-n + j / 8.0]], dtype=np.float32)
            c = O.expcast_codes(t, np.float32(8.0), np.array([[0.0]]))
            assert c[0, 0] == 120 - 8 * n + j
            assert O.e4m3_decode(c)[0, 0] == 2.0 ** (8 - n) * (1 + j / 8)
    # integer offsets give exact powers of two
    for n in range(15):
        c = O.expcast_codes(np.array([[float(-n)]], np.float32), np.float32(8), np.array([[0.0]]))
        assert O.e4m3_decode(c)[0, 0] == 256.0 * 2.0 ** -n


def test_expcast_ratio_bounds_and_underflow():
    # normal E4M3 codes (>= 8) cover t - M >= -14 - 1/16; below that the
    # subnormal codes m * 2^-9 take over and the octave map no longer holds
    t = np.linspace(-14.0, 0.0, 200001).astype(np.float32)[None, :]
    c = O.expcast_codes(t, np.float32(8), np.array([[0.0]]))
    val = O.e4m3_decode(c)[0]
    ratio = val / (256.0 * np.exp2(t[0].astype(np.float64)))
    # piecewise-linear mantissa: (1+m/8)/2^(m/8) in [1, 1.0607]; rounding to 1/8 octave: 2^(+-1/16)
    lo = 2.0 ** (-1 / 16)
    hi = max((1 + m / 8) / 2 ** (m / 8) for m in range(8)) * 2.0 ** (1 / 16)
    assert ratio.min() >= lo * (1 - 1e-6) and ratio.max() <= hi * (1 + 1e-6)
    assert ratio.min() < lo * 1.001 and ratio.max() > hi * 0.999      # bounds are attained
    assert np.all(np.diff(c[0]) >= 0)                                  # monotone
    far = O.expcast_codes(np.array([[-15.07, -20.0, -1e6]], np.float32), np.float32(8), np.array([[0.0]]))
    assert np.all(far == 0)


# ------------------------------------------------------- exact attention pins
def test_attention_exact_matches_torch_sdpa():
    q, k, v = _head(0)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        scale=float(O.DEFAULT_SM_SCALE))[0].numpy()
    assert O.rel_l2(O.attention_exact(q, k, v), ref) < 1e-13


def _noquant(q, k, v, smooth, pcast="exact", int_max=False, mode="online"):
    hv = O.prepare_v_head(v, smooth=smooth, k=4, iters=2, quant=False)
    hq = O.HeadQK(None, None, None, None)
    return O.attend_head(hq, hv, None, pcast=pcast, quant=False, q_raw=q, k_raw=k[hv.perm],
                         int_max=int_max, mode=mode)


@pytest.mark.parametrize("int_max", [False, True])
def test_unquantised_online_equals_softmax(int_max):
    q, k, v = _head(1)
    ex = O.attention_exact(q, k, v)
    assert O.rel_l2(_noquant(q, k, v, smooth=False, int_max=int_max), ex) < 1e-13


def test_mean_restore_and_joint_permutation_identity():
    # quantisation off: reorder + subtract block means + restore from the row sum
    # reproduces plain attention (residual is stored in fp32, hence 1e-7)
    q, k, v = _head(2, S=517, off=5.0, outl=6)
    ex = O.attention_exact(q, k, v)
    sm = _noquant(q, k, v, smooth=True)
    assert O.rel_l2(sm, ex) < 1e-7
    # with ExpCast probabilities the smoothed and unsmoothed outputs still agree
    # up to the E4M3 underflow edge (codes that hit 0 in one tile order only)
    a = _noquant(q, k, v, smooth=True, pcast="expcast", int_max=True)
    b = _noquant(q, k, v, smooth=False, pcast="expcast", int_max=True)
    assert O.rel_l2(a, b) < 2e-3


def test_online_equals_two_pass_with_integer_max():
    q, k, v = _head(3, S=700)
    a = _noquant(q, k, v, smooth=False, pcast="expcast", int_max=True, mode="online")
    b = _noquant(q, k, v, smooth=False, pcast="expcast", int_max=True, mode="two_pass")
    assert O.rel_l2(a, b) < 2e-3


def test_expcast_accuracy_envelope_unquantised():
    q, k, v = _head(4, S=600)
    ex = O.attention_exact(q, k, v)
    a = _noquant(q, k, v, smooth=False, pcast="expcast", int_max=True)
    assert O.rel_l2(a, ex) < 0.04
    # the "exp then cast to E4M3" path it replaces sits in the same envelope
    b = _noquant(q, k, v, smooth=False, pcast="exp_e4m3", int_max=True)
    assert O.rel_l2(b, ex) < 0.04


def _integer_log_head(qmax, seed=11, S=300, D=128):
    """Integer q, one-hot integer k: every score is an integer in [-2*qmax, 2*qmax]."""
    rng = np.random.default_rng(seed)
    q = rng.integers(-qmax, qmax + 1, size=(S, D)).astype(np.float64)
    k = np.zeros((S, D))
    k[np.arange(S), rng.integers(0, D, size=S)] = rng.integers(0, 3, size=S)   # one non-zero per key
    v = rng.standard_normal((S, D))
    return q, k, v


def _casts(q, k, v, sm, pcasts):
    hv = O.prepare_v_head(v, smooth=False, k=1, iters=0, quant=False)
    hq = O.HeadQK(None, None, None, None)
    return {pc: O.attend_head(hq, hv, None, sm_scale=sm, pcast=pc, quant=False, q_raw=q, k_raw=k[hv.perm],
                              int_max=True) for pc in pcasts}


def test_casts_exact_on_integer_log_scores():
    # Special case with a closed form: when every score times sigma is an
    # integer t and d = t - M is within reach of E4M3, 256 * 2^d is a power of
    # two that E4M3 holds exactly, so the "exp then E4M3 cast" path that
    # ExpCast replaces ("VC-Attention: Value Smoothing and Softmax Casting for
    # Low-bit Attention", Abstract) gives the exact probabilities for d down
    # to -17 (its smallest subnormal 2^-9; without the factor 256 everything
    # below d = -9 would underflow), and ExpCast's byte 120 + 8d -- an E4M3
    # normal number 2^(8+d) -- is exact for d >= -14 and 0 below.
    sm = 1.0 / math.log2(math.e)                     # sigma = sm * log2(e) = 1 exactly in fp64
    assert float(np.float64(sm)) * math.log2(math.e) == 1.0
    q, k, v = _integer_log_head(4)                   # scores in [-8, 8]: d reaches -16
    x = q @ k.T
    assert (x - x.max(axis=1, keepdims=True)).min() == -16.0
    out = _casts(q, k, v, sm, ("exact", "exp_e4m3", "expcast"))
    assert np.array_equal(out["exp_e4m3"], out["exact"])
    assert not np.array_equal(out["expcast"], out["exact"])       # d = -15, -16 cast to 0
    q, k, v = _integer_log_head(3, seed=12)          # scores in [-6, 6]: d >= -12
    out = _casts(q, k, v, sm, ("exact", "exp_e4m3", "expcast"))
    assert np.array_equal(out["expcast"], out["exact"])
    assert np.array_equal(out["exp_e4m3"], out["exact"])
    # off-integer scores: the E4M3 path rounds, so it is not trivially exact
    out = _casts(q, k, v, sm * 1.1, ("exact", "exp_e4m3"))
    assert not np.array_equal(out["exp_e4m3"], out["exact"])


# --------------------------------------------------------- whole pipeline pins
def _cfg(cid, **kw):
    w = synth.workload(cid, **kw)
    q, k, v = synth.generate(w)
    return w, [t.double().numpy() for t in (q, k, v)]


def test_pipeline_config1_accuracy_and_vsmooth_benefit():
    w, (q, k, v) = _cfg(1)
    ex = O.attention_exact(q[0, :, 0], k[0, :, 0], v[0, :, 0])
    P1 = O.prepare(q, k, v, kc=w.k, iters=w.iters)
    P0 = O.prepare(q, k, v, smooth=False)
    e1 = O.rel_l2(O.attention(P1)[(0, 0)], ex)
    e0 = O.rel_l2(O.attention(P0)[(0, 0)], ex)
    assert e1 < 0.04 and e0 < 0.04
    assert e1 <= e0


def test_pipeline_config2_heads_accuracy_and_vsmooth_benefit():
    w, (q, k, v) = _cfg(2, H=2, S=2048)
    rows = np.arange(0, 2048, 7)
    for h in range(2):
        ex = O.attention_exact(q[0, :, h], k[0, :, h], v[0, :, h], rows=rows)
        P1 = O.prepare(q, k, v, kc=32, iters=5, heads=[(0, h)])
        P0 = O.prepare(q, k, v, smooth=False, heads=[(0, h)])
        e1 = O.rel_l2(O.attend_head(P1.heads_qk[(0, h)], P1.heads_v[(0, h)], rows), ex)
        e0 = O.rel_l2(O.attend_head(P0.heads_qk[(0, h)], P0.heads_v[(0, h)], rows), ex)
        assert e1 < 0.04
        assert e1 <= e0, (h, e1, e0)


def test_single_block_and_ragged_tail():
    for S in (1, 5, 128, 129, 255):
        q, k, v = _head(10 + S, S=S, off=2.0)
        ex = O.attention_exact(q, k, v)
        hv = O.prepare_v_head(v, k=min(3, S), iters=2)
        hq = O.prepare_qk_head(q, k, hv.perm)
        assert O.rel_l2(O.attend_head(hq, hv), ex) < 0.04


def test_repair_zero_budget_is_identical_and_repair_helps():
    rng = np.random.default_rng(7)
    S = 1024
    q = rng.standard_normal((S, 128)).astype(np.float16).astype(np.float64)
    k = rng.standard_normal((S, 128)).astype(np.float16).astype(np.float64)
    v = rng.standard_t(3, (S, 128)).astype(np.float16).astype(np.float64)
    hq0 = None
    outs = {}
    for beta in (0.0, 0.005, 0.05):
        hv = O.prepare_v_head(v, k=8, iters=3, repair_budget=beta)
        hq = O.prepare_qk_head(q, k, hv.perm)
        outs[beta] = O.attend_head(hq, hv)
    base = O.prepare_v_head(v, k=8, iters=3)
    hq = O.prepare_qk_head(q, k, base.perm)
    assert np.array_equal(outs[0.0], O.attend_head(hq, base))
    ex = O.attention_exact(q, k, v)
    e = {b: O.rel_l2(o, ex) for b, o in outs.items()}
    assert e[0.05] < e[0.005] < e[0.0]


def test_softmax_temperature_two_keys():
    # Two keys whose exact softmax weights are 9:1 (score gap ln 9 after the
    # 1/sqrt(128) scale), values +e0 and -e0: exact output 0.8 e0.  The
    # quantised path sees the gap as log2(9) = 3.17 octaves, 25 ExpCast steps
    # of 1/8 (ratio 2^(25/8) = 8.72, output 0.794).  A temperature slip (the
    # log2 e factor lost, or natural-log codes) moves the output by ~18%.
    a = float(np.sqrt(np.log(9.0) * np.sqrt(128.0) / 2.0))
    q = np.zeros((2, 128)); q[:, 0] = a          # Q and K have one length; both rows alike
    k = np.zeros((2, 128)); k[0, 0] = a; k[1, 0] = -a
    v = np.zeros((2, 128)); v[0, 0] = 1.0; v[1, 0] = -1.0
    f = lambda x: x.astype(np.float32).astype(np.float64)
    q, k, v = f(q), f(k), f(v)
    ex = O.attention_exact(q, k, v)
    assert abs(ex[0, 0] - 0.8) < 1e-6
    hv = O.prepare_v_head(v, smooth=False)
    hq = O.prepare_qk_head(q, k, hv.perm)
    out = O.attend_head(hq, hv)
    assert abs(out[0, 0] - 0.8) < 0.02, out[0, 0]
    assert np.array_equal(out[0], out[1])
    assert np.all(np.abs(out[0, 1:]) < 1e-12)


def test_rounding_decision_hooks():
    """The parity tests' hooks: without them nothing changes; every reported
    near-boundary decision is within the width and names a real code; moving
    that code by its delta changes exactly that key's probability (the row
    then equals a hand-made recomputation with the one code replaced)."""
    q, k, v = _head(31, S=600)
    hv = O.prepare_v_head(v, k=4, iters=2)
    hq = O.prepare_qk_head(q, k, hv.perm)
    base = O.attend_head(hq, hv)
    assert np.array_equal(base, O.attend_head(hq, hv, code_delta={}, m_delta={}))
    found = None
    for row in range(0, 600, 7):
        ties = []
        out = O.attend_head(hq, hv, np.array([row]), ties=ties, tie_width=0.05)
        assert np.array_equal(out[0], base[row])
        for kind, b, j, d, dist in ties:
            assert dist < 0.05 and d in (-1, 1)
            if kind == "code" and found is None:
                found = (row, b, j, d)
    assert found is not None, "no near-boundary code in 86 rows at width 0.05"
    row, b, j, d = found
    alt = O.attend_head(hq, hv, np.array([row]), code_delta={(b, j): d})[0]
    assert not np.array_equal(alt, base[row])
    # the same row by hand: online softmax over the tiles with that one code moved
    Qd = O.e4m3_decode(hq.q8[[row]])
    Kd = O.e4m3_decode(hq.k8)
    Vd = hv.v_values()
    S = Kd.shape[0]
    M, l, num = -np.inf, 0.0, np.zeros(128)
    for t in range((S + 127) // 128):
        ks = slice(128 * t, min(S, 128 * (t + 1)))
        acc = (Qd @ Kd[ks].T).astype(np.float32)
        sig = O.sigma_of(hq.q_scale[row // 128], hq.k_scale[t], O.DEFAULT_SM_SCALE)
        Mn = max(M, math.ceil(float(np.float32(np.float32(acc.max()) * np.float32(sig)))))
        a = 2.0 ** (M - Mn) if np.isfinite(M) else 0.0
        c = O.expcast_codes(acc, np.float32(8) * np.float32(sig), np.array([[Mn]]))
        if t == b:
            c[0, j] = min(max(c[0, j] + d, 0), 126)
        P = O.e4m3_decode(c)
        r = P.sum()
        l, num, M = a * l + r, a * num + (P @ Vd[ks])[0] + r * hv.mean[t], Mn
    assert np.allclose(alt, num / l, rtol=1e-12, atol=0)
