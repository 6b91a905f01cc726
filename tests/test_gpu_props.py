"""GPU property test: random small shapes through the C ABI against the oracle.

Hypothesis draws every case (derandomized, so each run draws the same ones):
B in {1, 2}, H in 1..4, S in 1..700 (ragged lengths included), k in
1..min(S, 64), T in 0..6, the repair budget in {0, 0.005, 0.05}, fp16 or
bf16 inputs, smoothing on or off, the V residual format (E4M3, or MXFP4
without repair) and the kind of V (plain normal values, or a few channels
scaled up and offset, as outlier channels).  Each case goes through
check_against_oracle: the cluster assignment, the permutation, every code,
scale and block mean bit-exact; the output within the parity tolerances.
"""
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
