"""The ExpCast ablation build (libvc_ablation_exp.so) against the oracle.

That build replaces ExpCast by the FP32 exponential it was designed to
remove ("VC-Attention: Value Smoothing and Softmax Casting for Low-bit
Attention", Abstract): p = 256 * 2^(acc*sigma - M), cast to E4M3 with round
to nearest even.  It exists to measure ExpCast's saving on this GPU; the
oracle's pcast="exp_e4m3" path is its reference (pinned in
test_oracle_attention.py: exact on integer log-domain scores).  Everything
else -- prepared inputs, integer running maximum, row sums, restore, repair
-- is shared with the method, so the same parity bar applies: rel-L2 <= 5e-3
of the oracle, whose probabilities differ from the kernel's only where the
fp32 exponential lands within rounding of an E4M3 rounding boundary.
"""
import numpy as np
import pytest
import torch

import bit_attention_video_vc_amd as vc
import synth
from oracle import vc_oracle as O
from test_gpu_parity import TOL_ORACLE, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ablation_lib():
    main = vc.lib_path
    vc.use_library(vc.ablation_exp_lib_path)
    assert vc.lib().vc_version().decode().endswith("+ablation-exp-cast")
    yield
    vc.use_library(main)


CASES = [
    # (config, overrides, extra options)
    (1, {}, {}),
    (2, {}, {}),
    (2, {"S": 1000}, {"beta": 0.01}),      # ragged tail and repair tiles
]


@pytest.mark.parametrize("cid,kw,extra", CASES, ids=["config1", "config2", "config2_S1000_repair"])
def test_ablation_matches_oracle_exp_cast(ablation_lib, cid, kw, extra):
    w = synth.workload(cid, **kw)
    q, k, v = (t.cuda() for t in synth.generate(w, "cpu"))
    beta = extra.get("beta", w.repair_budget)
    opts = vc.v_opts(True, w.k, w.iters, 0, beta)
    ws = vc.alloc_workspace(v, opts)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    vc.vc_prepare_v(v, opts, ws)
    vc.vc_prepare_qk(q, k, opts, ws)
    vc.vc_attention_fwd(out, opts, ws)
    torch.cuda.synchronize()
    rows = synth.sample_rows(w.S, min(64, w.S)).numpy()
    errs = []
    for (b, h) in [(0, 0), (0, w.H - 1)]:
        qn, kn, vn = (t[b, :, h].double().cpu().numpy() for t in (q, k, v))
        hv = O.prepare_v_head(vn, smooth=True, k=w.k, iters=w.iters, seed=0, bh=b * w.H + h, repair_budget=beta)
        hq = O.prepare_qk_head(qn, kn, hv.perm)
        ref = O.bf16_round(O.attend_head(hq, hv, rows, pcast="exp_e4m3"))
        got = out[b, :, h].float().cpu().numpy()[rows].astype(np.float64)
        assert np.all(np.isfinite(got))
        e = O.rel_l2(got, ref)
        # and it is a different cast from ExpCast's: the oracle's ExpCast output is further away
        e_expcast = O.rel_l2(got, O.bf16_round(O.attend_head(hq, hv, rows, pcast="expcast")))
        errs.append((e, e_expcast))
        assert e <= TOL_ORACLE, f"config {cid} (b={b},h={h}): rel-L2 vs oracle exp-cast {e:.3e}"
        assert e_expcast > e, f"config {cid} (b={b},h={h}): closer to ExpCast than to the exp cast"
    say(f"ablation build, {w.name} S={w.S}: rel-L2 vs oracle exp-cast "
        f"{max(x[0] for x in errs):.3e} (vs oracle ExpCast {min(x[1] for x in errs):.3e})")
