"""Accuracy report per workload: what V-Smooth and the repair buy, measured.

For two heads of each workload, on a fixed sample of query rows, the GPU
output is compared with exact fp64 attention (softmax(Q K^T * sm_scale) V on
the original bf16/fp16 inputs) for three settings of the same call:

* V-Smooth on (the method),
* V-Smooth off (plain per-head E4M3 V, identity order, no block means),
* for the repair workload, V-Smooth on without the repair.

Each run is also checked against the oracle as in the parity tests, and the
oracle's own rel-L2 against exact attention on the same rows is reported
beside the GPU's: the GPU may exceed it by at most 2% (plus 1e-3), so any
error above the 4% accuracy target is shown to be the method's, not the
kernel's.  The 4% target is gated where the method meets it; the workloads
whose names say "accuracy_4pct_not_met" are those where the oracle itself
is above it (zero-mean V), and there the test checks that it is.  Beside the
errors the report gives the residual-energy ratio of the clustering, sum R^2
over sum (V - mean of its unsorted 128-token block)^2, from the oracle's own
prepare: below 1 when the reorder groups similar tokens (a reported figure,
not a gate).
"""
import numpy as np
import pytest
import torch

import bit_attention_video_vc_amd as vc
import synth
from oracle import vc_oracle as O
from test_gpu_parity import EXACT_RATIO, EXACT_SLACK, TOL_EXACT, TOL_ORACLE, GpuRun, say

pytestmark = pytest.mark.gpu

ROWS = 48


def _residual_energy_ratio(vn, hv):
    """sum R^2 (clustered blocks) / sum (V - unsorted block mean)^2, fp64."""
    S = vn.shape[0]
    r2 = float(np.sum(hv.resid.astype(np.float64) ** 2))
    plain = 0.0
    for b in range(0, S, 128):
        blk = vn[b:b + 128]
        plain += float(np.sum((blk - blk.mean(axis=0)) ** 2))
    return r2 / plain if plain > 0 else 1.0


def _errors(q, k, v, w, heads, rows, beta, smooth):
    opts = vc.v_opts(smooth, w.k, w.iters, 0, beta)
    run = GpuRun(q, k, v, opts)
    H = run.H
    out = []
    for (b, h) in heads:
        qn, kn, vn = (t[b, :, h].double().cpu().numpy() for t in (q, k, v))
        hv = O.prepare_v_head(vn, smooth=smooth, k=w.k, iters=w.iters, seed=0, bh=b * H + h, repair_budget=beta)
        hq = O.prepare_qk_head(qn, kn, hv.perm)
        ref = O.bf16_round(O.attend_head(hq, hv, rows))
        got = run.out[b, :, h].float().cpu().numpy()[rows].astype(np.float64)
        ex = O.attention_exact(qn, kn, vn, rows=rows)
        e_or = O.rel_l2(got, ref)
        tag = f"{w.name} (b={b},h={h}) smooth={smooth} beta={beta}"
        assert e_or <= TOL_ORACLE, f"{tag}: rel-L2 vs oracle {e_or:.3e}"
        e_ex, e_or_ex = O.rel_l2(got, ex), O.rel_l2(ref, ex)
        assert e_ex <= EXACT_RATIO * e_or_ex + EXACT_SLACK, f"{tag}: vs exact {e_ex:.3e}, oracle's own {e_or_ex:.3e}"
        out.append((e_ex, _residual_energy_ratio(vn, hv) if smooth else None, e_or_ex))
    del run
    torch.cuda.empty_cache()
    return out


CASES = [
    # (config, overrides, heads, repair workload, the 4% target met by the method on these rows)
    (1, {}, [(0, 0)], False, True),
    (2, {}, [(0, 0), (0, 7)], False, True),
    (4, {"H": 7}, [(0, 0), (0, 6)], False, True),
    (3, {}, [(0, 0), (0, 39)], False, False),
    (5, {}, [(0, 0), (1, 23)], True, False),
]


def _case_id(c):
    return f"config{c[0]}" + ("" if c[4] else "_accuracy_4pct_not_met_method_on_zero_mean_v")


@pytest.mark.parametrize("cid,kw,heads,repair,meets", CASES, ids=[_case_id(c) for c in CASES])
def test_accuracy_report(cid, kw, heads, repair, meets):
    w = synth.workload(cid, **kw)
    q, k, v = (t.cuda() for t in synth.generate(w, "cpu"))
    rows = synth.sample_rows(w.S, min(ROWS, w.S)).numpy()
    smooth = _errors(q, k, v, w, heads, rows, w.repair_budget, True)
    plain = _errors(q, k, v, w, heads, rows, w.repair_budget, False)
    norep = _errors(q, k, v, w, heads, rows, 0.0, True) if repair else None
    for i, (b, h) in enumerate(heads):
        e_s, ratio, e_s_or = smooth[i]
        e_p, _, e_p_or = plain[i]
        line = (f"{w.name} B={w.B} H={w.H} S={w.S} (b={b},h={h}): rel-L2 vs exact: V-Smooth {e_s:.3e} "
                f"(oracle {e_s_or:.3e}), plain E4M3 V {e_p:.3e} (oracle {e_p_or:.3e})")
        if norep is not None:
            line += f", V-Smooth without repair {norep[i][0]:.3e} (oracle {norep[i][2]:.3e})"
        line += f"; residual energy ratio {ratio:.3f}"
        say(line)
        assert ratio > 0.0, line
        if meets:
            assert e_s <= TOL_EXACT, line
        else:
            # the miss is the method's: the oracle itself is above the target
            assert e_s_or > TOL_EXACT, "labelled not met, but the oracle meets 4%: " + line
            say(f"4% accuracy target: not met ({w.name}, b={b}, h={h}): method {e_s_or:.3e}, GPU {e_s:.3e}")
        if norep is not None:
            # the repair adds back part of the residual's quantisation error;
            # it must not make the output measurably worse
            assert e_s <= norep[i][0] * 1.05 + 1e-6, line
