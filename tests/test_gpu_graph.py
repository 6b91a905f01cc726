"""The three calls recorded into one HIP graph and replayed.

The library launches kernels on the caller's stream and nothing else -- it
allocates nothing, clears memory with kernels (no memset nodes), never
synchronises and never reads device data on the host -- so a caller whose
shapes are fixed can record a whole forward once and replay it, which removes
the launch gaps that dominate short sequences.  A graph reads and writes the
buffers it was recorded with: each replay here gets fresh inputs copied into
them, eager calls of the same library run between replays, and every replay
is compared bit for bit with an eager call on the same inputs (the whole path
is deterministic).
"""
import pytest
import torch

import bit_attention_video_vc_amd as vc
import synth
from test_gpu_parity import say

pytestmark = pytest.mark.gpu

CASES = [
    # (config, overrides, repair budget, unbatched [S,H,128] view)
    (1, {}, 0.0, True),
    (2, {}, 0.0, False),
    (2, {"S": 1000}, 0.01, False),   # ragged tail and repair tiles
    (2, {"S": 4500, "H": 3}, 0.0, False),   # the attention call cut along the key axis, then merged
]


def _fresh(t: torch.Tensor, seed: int) -> torch.Tensor:
    g = torch.Generator(device=t.device).manual_seed(seed)
    noise = torch.randn(t.shape, generator=g, device=t.device, dtype=torch.float32)
    return (t.float() * 0.9 + noise * 0.5).to(t.dtype)


@pytest.mark.parametrize("cid,kw,beta,unbatched", CASES, ids=["config1_SH128", "config2", "config2_S1000_repair", "config2_S4500_cut"])
def test_graph_replays_match_eager(cid, kw, beta, unbatched):
    w = synth.workload(cid, **kw)
    q, k, v = (t.cuda() for t in synth.generate(w, "cpu"))
    if unbatched:
        q, k, v = q[0], k[0], v[0]
    opts = vc.v_opts(True, w.k, w.iters, 0, beta)
    qs, ks, vs = q.clone(), k.clone(), v.clone()     # the graph's input buffers
    ws = vc.alloc_workspace(vs, opts)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")

    def full_call(s):
        vc.vc_prepare_v(vs, opts, ws, s)
        vc.vc_prepare_qk(qs, ks, opts, ws, s)
        vc.vc_attention_fwd(out, opts, ws, 0.0, s)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        full_call(side)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        full_call(torch.cuda.current_stream())

    for rep in range(4):
        if rep:
            for src, dst, sd in ((q, qs, 11), (k, ks, 12), (v, vs, 13)):
                dst.copy_(_fresh(src, 100 * rep + sd))
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        # eager call of the same library on the same inputs, own buffers
        ref = vc.attention(qs.clone(), ks.clone(), vs.clone(), clusters=w.k, iters=w.iters, repair_budget=beta)
        torch.cuda.synchronize()
        assert torch.isfinite(got.float()).all()
        assert torch.equal(got, ref), f"replay {rep}: max diff {(got.float() - ref.float()).abs().max().item():.3e}"
    say(f"graph replay, {w.name} S={w.S} H={w.H}{' [S,H,128]' if unbatched else ''}: 4 replays bit-identical to eager")
