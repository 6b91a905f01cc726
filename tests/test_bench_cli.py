"""bench.py's command-line contract, checked without a GPU."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, capture_output=True,
                          text=True, timeout=300)


def test_more_than_one_gpu_exits_with_a_message():
    r = _bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""                       # no JSON line


def test_no_gpu_fails_loudly():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    r = _bench("--steps", "1", "--warmup", "0", "--no-cpu-baseline")
    assert r.returncode == 2
    assert "needs a GPU" in r.stderr
    assert r.stdout == ""


def test_prepare_byte_model():
    sys.path.insert(0, ROOT)
    import bench
    import synth
    w = synth.workload(4)                       # B=1 S=73397 H=56, T=5
    n = 56 * 73397 * 128
    rep = bench.prepare_report(w, 1.0, 1.0)     # 1 ms each
    # V: (T+1) assignment passes + block means + quantise at 2 B, one 1-byte write
    assert rep["prepare_v_algorithmic_GBps"] == round(17 * n / 1e-3 / 1e9, 1)
    # Q and K: read 2 B, write 1 B each
    assert rep["prepare_qk_algorithmic_GBps"] == round(6 * n / 1e-3 / 1e9, 1)


def test_roofline_kernel_label_follows_the_launch_plan():
    """bench.py names the short-launch kernel exactly for the workloads the
    library's work split runs in that form (the rule of attn_split, restated
    by tests/test_split_plan.py)."""
    sys.path.insert(0, ROOT)
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import bench
    import synth
    from test_split_plan import plan
    for cid, kw in [(1, {}), (2, {}), (2, {"S": 2049, "H": 14}), (2, {"S": 4500, "H": 3}), (2, {"S": 4096, "H": 9}),
                    (3, {}), (4, {}), (4, {"H": 7}), (5, {})]:
        w = synth.workload(cid, **kw)
        p = plan(w.B * w.H, -(-w.S // 128), 1 if w.repair_budget > 0 else 0)
        halves = bool(p and p.get("halves"))
        assert ("k_vc_attn_halves" in bench.attention_kernels(w)) == halves, (cid, kw)
