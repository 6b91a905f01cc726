"""Python binding of libvc.so, the gfx950 VC-Attention forward library.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/vc.h``.  PyTorch supplies
device memory and the current stream.  Importing this module does not load
the library; the first call does, and raises if it has not been built.

Entry points (same names as the C ABI):
  vc_workspace_layout(v_like, opts)                 -> VcWsLayout
  vc_prepare_v(v, opts, ws)
  vc_prepare_v_noalloc(v, opts, ws)                 (scratch in a static device array)
  vc_prepare_qk(q, k, opts, ws)
  vc_attention_fwd(out, opts, ws, sm_scale=0.0)
plus the convenience ``attention(q, k, v, ...)`` that runs all three.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

__all__ = [
    "VcDesc", "VcVOpts", "VcAttnOpts", "VcWsLayout", "VcHeadHdr", "VCError", "lib", "lib_path",
    "ablation_exp_lib_path", "use_library",
    "v_opts", "VC_V_E4M3", "VC_V_MXFP4", "desc_of", "vc_workspace_layout", "vc_prepare_v", "vc_prepare_v_noalloc",
    "vc_prepare_qk", "vc_attention_fwd", "NOALLOC_SCRATCH_BYTES",
    "alloc_workspace", "attention", "EXPORTS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libvc.so")
# Measurement build: FP32 exponential + E4M3 cast in place of ExpCast.
ablation_exp_lib_path = os.path.join(_HERE, "libvc_ablation_exp.so")

VC_OK, VC_ERR_ARG, VC_ERR_UNSUPPORTED, VC_ERR_WORKSPACE, VC_ERR_DEVICE = range(5)
VC_F16, VC_BF16 = 0, 1

# symbols the header declares (checked by the ABI tests)
EXPORTS = ("vc_workspace_layout", "vc_prepare_v", "vc_prepare_v_noalloc", "vc_prepare_qk", "vc_attention_fwd",
           "vc_status_string", "vc_last_error", "vc_version")
# bytes of the static scratch array behind vc_prepare_v_noalloc (vc.h)
NOALLOC_SCRATCH_BYTES = 32 << 20


class VcDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("S", ctypes.c_int32), ("H", ctypes.c_int32), ("D", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("sB", ctypes.c_int64), ("sS", ctypes.c_int64), ("sH", ctypes.c_int64)]


class VcVOpts(ctypes.Structure):
    _fields_ = [("smooth", ctypes.c_int32), ("k", ctypes.c_int32), ("iters", ctypes.c_int32),
                ("v_format", ctypes.c_int32), ("seed", ctypes.c_uint64), ("repair_budget", ctypes.c_float),
                ("reserved2", ctypes.c_float)]


class VcAttnOpts(ctypes.Structure):
    _fields_ = [("sm_scale", ctypes.c_float), ("reserved", ctypes.c_int32)]


class VcWsLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in (
        "total", "q8", "q_scale", "k8", "k_scale", "v8", "v_mean", "v_muop", "hdr",
        "assign", "perm", "rep_pos", "rep_k8", "rep_ks", "rep_e8", "attn_part", "scratch")] + \
        [("nblk", ctypes.c_int32), ("nrep", ctypes.c_int32), ("nrep_pad", ctypes.c_int32),
         ("reserved", ctypes.c_int32)]


class VcHeadHdr(ctypes.Structure):
    _fields_ = [("v_scale", ctypes.c_float), ("v_inv", ctypes.c_float), ("v_amax_bits", ctypes.c_uint32),
                ("r_amax_bits", ctypes.c_uint32), ("shift", ctypes.c_int32), ("nrep", ctypes.c_int32),
                ("rep_scale", ctypes.c_float), ("e_amax_bits", ctypes.c_uint32)]


class VCError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libvc.so (in-tree build) and declare its signatures."""
    global _lib
    if _lib is None:
        if not os.path.exists(lib_path):
            raise RuntimeError(f"{lib_path} is not built; run `python -m bit_attention_video_vc_amd.build`")
        L = ctypes.CDLL(lib_path)
        P = ctypes.POINTER
        L.vc_workspace_layout.argtypes = [P(VcDesc), P(VcVOpts), P(VcWsLayout)]
        L.vc_prepare_v.argtypes = [P(VcDesc), ctypes.c_void_p, P(VcVOpts), ctypes.c_void_p, ctypes.c_size_t,
                                   ctypes.c_void_p]
        L.vc_prepare_v_noalloc.argtypes = L.vc_prepare_v.argtypes
        L.vc_prepare_qk.argtypes = [P(VcDesc), ctypes.c_void_p, P(VcDesc), ctypes.c_void_p, P(VcVOpts),
                                    ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.vc_attention_fwd.argtypes = [P(VcDesc), ctypes.c_void_p, P(VcVOpts), P(VcAttnOpts), ctypes.c_void_p,
                                       ctypes.c_size_t, ctypes.c_void_p]
        for f in ("vc_workspace_layout", "vc_prepare_v", "vc_prepare_v_noalloc", "vc_prepare_qk", "vc_attention_fwd"):
            getattr(L, f).restype = ctypes.c_int
        L.vc_status_string.argtypes = [ctypes.c_int]
        for f in ("vc_status_string", "vc_last_error", "vc_version"):
            getattr(L, f).restype = ctypes.c_char_p
        _lib = L
    return _lib


def use_library(path: str) -> None:
    """Make the binding call the library at `path` from now on (e.g. the
    ExpCast ablation build); it is loaded on the next call."""
    global _lib, lib_path
    lib_path = path
    _lib = None


def _check(status: int) -> None:
    if status != VC_OK:
        L = lib()
        raise VCError(status, f"{L.vc_status_string(status).decode()}: {L.vc_last_error().decode()}")


VC_V_E4M3, VC_V_MXFP4 = 0, 1


def v_opts(smooth: bool = True, k: int = 32, iters: int = 5, seed: int = 0, repair_budget: float = 0.0,
           v_format: int = VC_V_E4M3) -> VcVOpts:
    return VcVOpts(int(bool(smooth)), int(k), int(iters), int(v_format), int(seed), float(repair_budget), 0.0)


def desc_of(t: torch.Tensor) -> VcDesc:
    """Descriptor of a [B,S,H,128] or [S,H,128] fp16/bf16 tensor (D contiguous)."""
    if t.dim() == 3:
        t = t.unsqueeze(0)
    if t.dim() != 4:
        raise ValueError("expected a [B,S,H,D] or [S,H,D] tensor")
    if t.stride(3) != 1:
        raise ValueError("the head dimension must be contiguous")
    dt = {torch.float16: VC_F16, torch.bfloat16: VC_BF16}.get(t.dtype, -1)
    B, S, H, D = t.shape
    return VcDesc(B, S, H, D, dt, 0, t.stride(0), t.stride(1), t.stride(2))


def _device_of(**tensors: torch.Tensor) -> torch.device:
    """The one GPU that every tensor is on; raises before any library call
    otherwise (the kernels dereference these pointers on the current device)."""
    dev = None
    for name, t in tensors.items():
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            where = t.device if isinstance(t, torch.Tensor) else type(t).__name__
            raise ValueError(f"{name} must be a GPU tensor (got {where})")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other tensors on {dev}")
    return dev


def _ws_bytes(ws: torch.Tensor) -> int:
    if not ws.is_contiguous():
        raise ValueError("the workspace must be a contiguous tensor")
    return ws.numel() * ws.element_size()


def _stream(stream, dev: torch.device) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    elif isinstance(stream, torch.cuda.Stream) and stream.device != dev:
        raise ValueError(f"stream is on {stream.device}, the tensors on {dev}")
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def vc_workspace_layout(v_like: torch.Tensor | VcDesc, opts: VcVOpts) -> VcWsLayout:
    d = v_like if isinstance(v_like, VcDesc) else desc_of(v_like)
    out = VcWsLayout()
    _check(lib().vc_workspace_layout(ctypes.byref(d), ctypes.byref(opts), ctypes.byref(out)))
    return out


def alloc_workspace(v_like: torch.Tensor, opts: VcVOpts) -> torch.Tensor:
    lay = vc_workspace_layout(v_like, opts)
    return torch.empty(lay.total, dtype=torch.uint8, device=v_like.device)


def vc_prepare_v(v: torch.Tensor, opts: VcVOpts, ws: torch.Tensor, stream=None) -> None:
    dev = _device_of(v=v, ws=ws)
    d, nbytes = desc_of(v), _ws_bytes(ws)
    with torch.cuda.device(dev):
        _check(lib().vc_prepare_v(ctypes.byref(d), ctypes.c_void_p(v.data_ptr()), ctypes.byref(opts),
                                  ctypes.c_void_p(ws.data_ptr()), nbytes, _stream(stream, dev)))


def vc_prepare_v_noalloc(v: torch.Tensor, opts: VcVOpts, ws: torch.Tensor, stream=None) -> None:
    """vc_prepare_v with its scratch in the library's static device array;
    `ws` needs only layout.scratch bytes."""
    dev = _device_of(v=v, ws=ws)
    d, nbytes = desc_of(v), _ws_bytes(ws)
    with torch.cuda.device(dev):
        _check(lib().vc_prepare_v_noalloc(ctypes.byref(d), ctypes.c_void_p(v.data_ptr()), ctypes.byref(opts),
                                          ctypes.c_void_p(ws.data_ptr()), nbytes, _stream(stream, dev)))


def vc_prepare_qk(q: torch.Tensor, k: torch.Tensor, opts: VcVOpts, ws: torch.Tensor, stream=None) -> None:
    dev = _device_of(q=q, k=k, ws=ws)
    dq, dk, nbytes = desc_of(q), desc_of(k), _ws_bytes(ws)
    with torch.cuda.device(dev):
        _check(lib().vc_prepare_qk(ctypes.byref(dq), ctypes.c_void_p(q.data_ptr()), ctypes.byref(dk),
                                   ctypes.c_void_p(k.data_ptr()), ctypes.byref(opts), ctypes.c_void_p(ws.data_ptr()),
                                   nbytes, _stream(stream, dev)))


def vc_attention_fwd(out: torch.Tensor, opts: VcVOpts, ws: torch.Tensor, sm_scale: float = 0.0,
                     stream=None) -> None:
    dev = _device_of(out=out, ws=ws)
    d, nbytes = desc_of(out), _ws_bytes(ws)
    a = VcAttnOpts(float(sm_scale), 0)
    with torch.cuda.device(dev):
        _check(lib().vc_attention_fwd(ctypes.byref(d), ctypes.c_void_p(out.data_ptr()), ctypes.byref(opts),
                                      ctypes.byref(a), ctypes.c_void_p(ws.data_ptr()), nbytes,
                                      _stream(stream, dev)))


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, smooth: bool = True, clusters: int = 32,
              iters: int = 5, seed: int = 0, repair_budget: float = 0.0, sm_scale: float = 0.0,
              v_format: int = VC_V_E4M3, ws: torch.Tensor | None = None, out: torch.Tensor | None = None,
              stream=None) -> torch.Tensor:
    """Full call: prepare_v, prepare_qk and the fused forward; returns bf16 [B,S,H,128] (or [S,H,128])."""
    o = v_opts(smooth, clusters, iters, seed, repair_budget, v_format)
    # the three calls share one workspace laid out for v's shape: refuse any
    # other shape before the first call
    for name, t in (("q", q), ("k", k)) + ((("out", out),) if out is not None else ()):
        if isinstance(t, torch.Tensor) and isinstance(v, torch.Tensor) and t.shape != v.shape:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, v has {tuple(v.shape)}; all must match")
    _device_of(q=q, k=k, v=v, **({} if out is None else {"out": out}))
    if ws is None:
        ws = alloc_workspace(v, o)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    vc_prepare_v(v, o, ws, stream)
    vc_prepare_qk(q, k, o, ws, stream)
    vc_attention_fwd(out, o, ws, sm_scale, stream)
    return out


@dataclass
class WorkspaceView:
    """Host-side views of a prepared workspace (copies), for tests and diagnostics."""

    layout: VcWsLayout
    B: int
    S: int
    H: int

    def region(self, ws: torch.Tensor, name: str, dtype: torch.dtype, count: int) -> torch.Tensor:
        off = getattr(self.layout, name)
        nbytes = count * torch.tensor([], dtype=dtype).element_size()
        return ws[off:off + nbytes].view(dtype).cpu()
