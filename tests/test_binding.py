"""Host-side checks of the Python binding that need no GPU: tensors that are
not on a GPU are refused before the library is called (the kernels would
otherwise dereference host pointers)."""
import pytest
import torch

import bit_attention_video_vc_amd as vc


def _cpu(shape=(1, 256, 2, 128)):
    return torch.zeros(shape, dtype=torch.bfloat16)


def test_prepare_v_refuses_host_tensors():
    with pytest.raises(ValueError, match="GPU tensor"):
        vc.vc_prepare_v(_cpu(), vc.v_opts(True, 4, 1), torch.empty(16, dtype=torch.uint8))


def test_prepare_qk_refuses_host_tensors():
    with pytest.raises(ValueError, match="q must be a GPU tensor"):
        vc.vc_prepare_qk(_cpu(), _cpu(), vc.v_opts(True, 4, 1), torch.empty(16, dtype=torch.uint8))


def test_attention_fwd_refuses_host_tensors():
    with pytest.raises(ValueError, match="out must be a GPU tensor"):
        vc.vc_attention_fwd(_cpu(), vc.v_opts(True, 4, 1), torch.empty(16, dtype=torch.uint8))


def test_attention_refuses_host_tensors_and_non_tensors():
    with pytest.raises(ValueError, match="GPU tensor"):
        vc.attention(_cpu(), _cpu(), _cpu())
    with pytest.raises(ValueError, match="GPU tensor"):
        vc.vc_prepare_v(_cpu(), vc.v_opts(True, 4, 1), None)


def test_workspace_must_be_contiguous():
    ws = torch.empty(64, dtype=torch.uint8)
    assert vc._ws_bytes(ws) == 64
    assert vc._ws_bytes(ws.view(torch.int32)) == 64
    with pytest.raises(ValueError, match="contiguous"):
        vc._ws_bytes(ws[::2])


def test_descriptor_of_unbatched_and_strided_views():
    t = _cpu((300, 3, 128))
    d = vc.desc_of(t)
    assert (d.B, d.S, d.H, d.D, d.dtype) == (1, 300, 3, 128, vc.VC_BF16)
    assert (d.sS, d.sH) == (3 * 128, 128)
    # a head-major tensor viewed as [B,S,H,D]
    hm = torch.zeros((2, 3, 300, 128), dtype=torch.float16).permute(0, 2, 1, 3)
    d = vc.desc_of(hm)
    assert (d.B, d.S, d.H, d.dtype) == (2, 300, 3, vc.VC_F16)
    assert (d.sB, d.sS, d.sH) == (3 * 300 * 128, 128, 300 * 128)
    with pytest.raises(ValueError):
        vc.desc_of(torch.zeros((4, 128, 2), dtype=torch.bfloat16).permute(0, 2, 1))   # D not contiguous


def test_attention_refuses_mismatched_shapes():
    # the workspace is laid out for v's shape; q, k or out of another shape
    # are refused before any library call (the check needs no GPU)
    v = _cpu((1, 256, 2, 128))
    for bad in ((1, 128, 2, 128), (1, 256, 3, 128), (2, 256, 2, 128)):
        with pytest.raises(ValueError, match="all must match"):
            vc.attention(_cpu(bad), _cpu(), v)
        with pytest.raises(ValueError, match="all must match"):
            vc.attention(_cpu(), _cpu(bad), v)
        with pytest.raises(ValueError, match="all must match"):
            vc.attention(_cpu(), _cpu(), v, out=_cpu(bad))
