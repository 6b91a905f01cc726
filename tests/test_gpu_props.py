"""GPU property test: random small shapes through the C ABI against the oracle.

Hypothesis draws every case (derandomized, so each run draws the same ones):
B in {1, 2}, H in 1..4, S in 1..700 (ragged lengths included), k in
1..min(S, 64), T in 0..6, the repair budget in {0, 0.005, 0.05}, fp16 or
bf16 inputs, smoothing on or off, the V residual format (E4M3, or MXFP4
without repair) and the kind of V (plain normal values, or a few channels
scaled up and offset, as outlier channels).  Each case goes through
check_against_oracle: the cluster assignment, the permutation, every code,
scale and block mean bit-exact; the output within the parity tolerances.
A second test draws 8 cases of 1500..9000 tokens (B*H up to 16), where the
attention call takes each of its launch forms.
"""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from test_gpu_parity import check_against_oracle

pytestmark = pytest.mark.gpu


@st.composite
def cases(draw):
    S = draw(st.integers(1, 700))
    c = {
        "B": draw(st.integers(1, 2)),
        "H": draw(st.integers(1, 4)),
        "S": S,
        "kc": draw(st.integers(1, min(S, 64))),
        "iters": draw(st.integers(0, 6)),
        "dtype": draw(st.sampled_from([torch.bfloat16, torch.float16])),
        "smooth": draw(st.booleans()),
        "v_format": draw(st.sampled_from(["e4m3", "mxfp4"])),
        "outliers": draw(st.booleans()),
        "seed": draw(st.integers(0, 2 ** 31 - 1)),
    }
    c["beta"] = 0.0 if c["v_format"] == "mxfp4" else draw(st.sampled_from([0.0, 0.005, 0.05]))
    return c


@settings(max_examples=24, deadline=None, derandomize=True, database=None, print_blob=True,
          suppress_health_check=[HealthCheck.too_slow])
@given(cases())
def test_random_small_shapes(c):
    g = torch.Generator().manual_seed(c["seed"])
    shape = (c["B"], c["S"], c["H"], 128)
    q = torch.randn(shape, generator=g)
    k = torch.randn(shape, generator=g)
    v = torch.randn(shape, generator=g)
    if c["outliers"]:
        ch = torch.randperm(128, generator=g)[:4]
        v[..., ch] = v[..., ch] * 8.0 + 3.0
    q, k, v = (t.to(c["dtype"]).cuda() for t in (q, k, v))
    name = (f"props B={c['B']} H={c['H']} S={c['S']} k={c['kc']} T={c['iters']} beta={c['beta']} "
            f"{c['v_format']} smooth={c['smooth']} outliers={c['outliers']} seed={c['seed']}")
    check_against_oracle(q, k, v, smooth=c["smooth"], kc=c["kc"], iters=c["iters"], seed=c["seed"] % 97,
                         beta=c["beta"], name=name, v_format=c["v_format"])


@st.composite
def mid_cases(draw):
    S = draw(st.integers(1500, 9000))
    c = {
        "B": draw(st.integers(1, 2)),
        "H": draw(st.integers(1, 8)),
        "S": S,
        "kc": draw(st.integers(1, 64)),
        "iters": draw(st.integers(0, 3)),
        "dtype": draw(st.sampled_from([torch.bfloat16, torch.float16])),
        "v_format": draw(st.sampled_from(["e4m3", "mxfp4"])),
        "seed": draw(st.integers(0, 2 ** 31 - 1)),
    }
    c["beta"] = 0.0 if c["v_format"] == "mxfp4" else draw(st.sampled_from([0.0, 0.0, 0.005]))
    return c


@settings(max_examples=8, deadline=None, derandomize=True, database=None, print_blob=True,
          suppress_health_check=[HealthCheck.too_slow])
@given(mid_cases())
def test_random_mid_shapes(c):
    """Lengths of 1500..9000 tokens, where the attention call takes each of
    its launch forms: whole items, the key-axis cut with its merge, and the
    short-launch halves (the form is printed with the case).  The first and
    the last head are compared, on every fourth query row and the last 130."""
    from test_split_plan import plan
    nblk = -(-c["S"] // 128)
    p = plan(c["B"] * c["H"], nblk, 1 if c["beta"] > 0 else 0)
    form = "whole" if p is None else ("halves" if p.get("halves") else f"cut ({p['tail']} items)")
    g = torch.Generator().manual_seed(c["seed"])
    shape = (c["B"], c["S"], c["H"], 128)
    q = torch.randn(shape, generator=g)
    k = torch.randn(shape, generator=g)
    v = torch.randn(shape, generator=g) + 0.5 * torch.randn((1, 1, c["H"], 128), generator=g)
    q, k, v = (t.to(c["dtype"]).cuda() for t in (q, k, v))
    S = c["S"]
    rows = np.unique(np.concatenate([np.arange(0, S, 4), np.arange(max(0, S - 130), S)]))
    name = (f"props-mid B={c['B']} H={c['H']} S={S} k={c['kc']} T={c['iters']} beta={c['beta']} "
            f"{c['v_format']} seed={c['seed']} form={form}")
    heads = sorted({(0, 0), (c["B"] - 1, c["H"] - 1)})
    check_against_oracle(q, k, v, kc=min(c["kc"], S), iters=c["iters"], seed=c["seed"] % 97, beta=c["beta"],
                         rows=rows, heads=heads, name=name, v_format=c["v_format"])
