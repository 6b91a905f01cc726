"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (one prepare_v + prepare_qk + attention call over all heads).

For a few heads per workload every prepared product is compared bit-exactly
with the oracle and a fixed sample of query rows (always including the first
and the ragged last row) is compared with the oracle's output; for every head
the properties that hold at any size are checked on the GPU: the permutation
is a permutation, cluster ids ascend along it, and the output is finite.
"""
import numpy as np
import pytest
import torch

import bit_attention_video_vc_amd as vc
import synth
from test_gpu_parity import check_against_oracle, say

pytestmark = pytest.mark.gpu

ROWS_PER_HEAD = 48


def _whole_call_properties(run, name):
    BH, S = run.B * run.H, run.S
    off = run.lay.perm
    perm = run.ws[off:off + 4 * BH * S].view(torch.int32).reshape(BH, S).long()
    off = run.lay.assign
    assign = run.ws[off:off + 4 * BH * S].view(torch.int32).reshape(BH, S).long()
    ar = torch.arange(S, device=perm.device).expand(BH, S)
    assert torch.equal(torch.sort(perm, dim=1).values, ar), name + ": perm is not a permutation in some head"
    along = torch.gather(assign, 1, perm)
    assert bool((along[:, 1:] >= along[:, :-1]).all()), name + ": cluster ids do not ascend along perm"
    assert bool(torch.isfinite(run.out.float()).all()), name + ": non-finite output"
    say(f"{name}: all {BH} heads: perm/assign properties and finite output ok")


def _run(cid, heads, target_met, v_format="e4m3", **kw):
    w = synth.workload(cid, **kw)
    q, k, v = (t.cuda() for t in synth.generate(w, "cpu"))
    rows = synth.sample_rows(w.S, ROWS_PER_HEAD).numpy()
    run = check_against_oracle(q, k, v, kc=w.k, iters=w.iters, beta=w.repair_budget, rows=rows, heads=heads,
                               name=f"{w.name} B={w.B} H={w.H} S={w.S} {v_format}", target_met=target_met,
                               v_format=v_format)
    _whole_call_properties(run, w.name)


def test_full_minimax_h56():
    # the benchmark's workload: B=1, S=73397, H=56
    _run(4, heads=[(0, 0), (0, 29), (0, 55)], target_met=True)


@pytest.mark.parametrize("H", [7, 14])
def test_full_minimax_other_heads(H):
    _run(4, heads=[(0, 0), (0, H - 1)], target_met=True, H=H)


def test_full_wan_720p_accuracy_4pct_not_met_method_on_zero_mean_v():
    # zero-mean V with 0.2% outlier tokens at 50x: the per-head V scale is set
    # by the outliers and the oracle itself sits 5-6% from exact attention;
    # the GPU is gated at 1.02x the oracle's error (plus 1e-3) instead
    _run(3, heads=[(0, 0), (0, 39)], target_met=False)


def test_full_batched_repair_accuracy_4pct_not_met_method_on_zero_mean_v():
    # Student-t V (zero mean): the oracle itself sits ~5.7% from exact
    _run(5, heads=[(0, 0), (1, 23)], target_met=False)


def test_full_minimax_h14_mxfp4():
    # the 4-bit residual at the benchmark's sequence length (its own kernel
    # instance: FP4 P.V operands and the anchor maximum)
    _run(4, heads=[(0, 0), (0, 13)], target_met=True, v_format="mxfp4", H=14)
