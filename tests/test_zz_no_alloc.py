"""The allocation-free V prepare, vc_prepare_v_noalloc, against vc_prepare_v.

vc_prepare_v_noalloc serves callers that cannot allocate device memory: its
k-means, sort and repair scratch lives in a static device array of the
library, so the caller's workspace holds only the prepared products
(layout.scratch bytes).  Both entry points run the same kernels, so every
prepared product and the attention output must be bit-identical.  Two calls
in a row on the shared static array, the second on a smaller input, show that
a call does not depend on what the previous call left there.
"""
import ctypes
import sys

import pytest
import torch

import bit_attention_video_vc_amd as vc
import synth

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[no-alloc] {msg}", flush=True)
    sys.stdout.flush()


def _full_call(q, k, v, opts, ws, noalloc):
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    (vc.vc_prepare_v_noalloc if noalloc else vc.vc_prepare_v)(v, opts, ws)
    vc.vc_prepare_qk(q, k, opts, ws)
    vc.vc_attention_fwd(out, opts, ws)
    return out


@pytest.mark.parametrize("cases", [[
    # (config model, B, H, S, k, T, repair budget)
    (2, 1, 4, 3000, 16, 3, 0.01),
    (5, 2, 1, 1000, 8, 2, 0.02),
]], ids=["two_calls_second_smaller"])
def test_noalloc_matches_prepare_v(cases):
    for (cid, B, H, S, kc, T, beta) in cases:
        w = synth.workload(cid, B=B, H=H, S=S)
        q, k, v = synth.generate(w, "cuda")
        opts = vc.v_opts(True, kc, T, 0, beta)
        lay = vc.vc_workspace_layout(v, opts)
        say(f"B={B} H={H} S={S} {v.dtype} k={kc} T={T} beta={beta}: scratch {lay.total - lay.scratch} bytes "
            f"(static array {vc.NOALLOC_SCRATCH_BYTES})")
        assert lay.total - lay.scratch <= vc.NOALLOC_SCRATCH_BYTES
        # same poison in both workspaces: bytes no kernel writes stay equal
        ws_a = torch.full((lay.total,), 0x7F, dtype=torch.uint8, device="cuda")
        ws_b = torch.full((lay.scratch,), 0x7F, dtype=torch.uint8, device="cuda")
        out_a = _full_call(q, k, v, opts, ws_a, noalloc=False)
        out_b = _full_call(q, k, v, opts, ws_b, noalloc=True)
        torch.cuda.synchronize()
        assert torch.equal(ws_a[:lay.scratch], ws_b), "prepared products differ"
        assert torch.equal(out_a, out_b), "attention output differs"
        assert bool(torch.isfinite(out_a.float()).all())
        say(f"B={B} H={H} S={S}: prepared products and output bit-identical")


def test_noalloc_rejects_a_shape_past_the_static_array():
    # repair scores alone need B*H*S*8 bytes: 8*2^20*8 = 64 MiB > 32 MiB.
    # Rejected on the host before any device call, so the pointers are
    # aligned stand-ins that are never dereferenced.
    S, H = 1 << 20, 8
    d = vc.VcDesc(1, S, H, 128, vc.VC_BF16, 0, S * H * 128, H * 128, 128)
    opts = vc.v_opts(True, 8, 1, 0, 0.01)
    lay = vc.vc_workspace_layout(d, opts)
    assert lay.total - lay.scratch > vc.NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(0x100000)
    st = vc.lib().vc_prepare_v_noalloc(ctypes.byref(d), fake, ctypes.byref(opts), fake, lay.scratch, None)
    assert st == vc.VC_ERR_UNSUPPORTED
    assert "scratch" in vc.lib().vc_last_error().decode()
    # a workspace below the prepared products' size is refused as for vc_prepare_v
    st = vc.lib().vc_prepare_v_noalloc(ctypes.byref(d), fake, ctypes.byref(opts), fake, lay.scratch - 1, None)
    assert st == vc.VC_ERR_WORKSPACE
