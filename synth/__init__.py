"""Seeded synthetic workloads for the VC-Attention forward pass.

This module only draws random tensors.  It holds none of the method's
arithmetic (no quantisation, clustering or attention), so both the CPU oracle
and the GPU path can take their inputs from it without sharing any of the
computation they are compared on.

The shapes and value structure follow the video-DiT workloads the pages
describe; no captured tensors, datasets or model weights are used.

* "VC-Attention: Value Smoothing and Softmax Casting for Low-bit Attention",
  Abstract: the large values of V are not tied to particular channels or to
  particular places in space or time, so the generator draws their token
  positions at random per head.
* "Nunchux AI lanza VC-Attention kernel ..." (reditua.com), paragraph 1: a
  5 s 720p clip from a 14B model is about 70k tokens; paragraph 2: value
  outliers sit in a few tokens and move between layers, heads and steps.
* "Open VC Attention", section "Описание": Q/K/V of shape [B,S,H,128] in
  FP16/BF16, S=73397 with 7, 14 or 56 heads.

Recipe (all draws from one ``torch.Generator`` seeded with
``20260914 + config_id``; the draw order is fixed as written below):

====  =====================  ==========================================  =====
cfg   B x H x S  (dtype)      Q, K                       V                        k,T
====  =====================  ==========================================  =====
1     1 x 1 x 256 (bf16)     N(0,1)                       N(0,1); 4 outlier tokens x20 2,3
                                                          at random positions; per-
                                                          channel offset N(0,2)
2     1 x 8 x 4096 (bf16)    N(0,1) x per-(tensor,head)   N(0,1) + per-(head,channel)  32,5
                             scale U(0.5,2)               offset N(0,3); 20 outlier
                                                          tokens (0.5%) x30 per head
3     1 x 40 x 75600 (bf16)  AR(1) along tokens, rho=0.9, N(0,1); 151 outlier tokens 32,5
                             unit variance, per (h,d)     (0.2%) x50 per head
4     1 x H x 73397 (bf16),  as config 2                  as config 2 at 0.2%        32,5
      H in {7,14,56}                                      (147 tokens) x30
5     2 x 24 x 32768 (fp16)  N(0,1)                       Student-t (nu=3) per       32,5
                                                          element; repair 0.005
====  =====================  ==========================================  =====

An outlier token j has its noise part scaled: v_j = m * z_j + offset.
Outlier positions are drawn independently for every (batch, head).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

SEED_BASE = 20260914


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, dtype and the V-Smooth options."""

    name: str
    config_id: int
    B: int
    H: int
    S: int
    D: int = 128
    dtype: torch.dtype = torch.bfloat16
    k: int = 32
    iters: int = 5
    repair_budget: float = 0.0
    extra: dict = field(default_factory=dict)

    @property
    def flops(self) -> float:
        """Attention FLOP per forward call, 4*B*H*S^2*D."""
        return 4.0 * self.B * self.H * float(self.S) ** 2 * self.D


def workload(config_id: int, H: int | None = None, S: int | None = None,
             B: int | None = None) -> Workload:
    """Return the workload descriptor for config 1..5 (optionally resized)."""
    table = {
        1: Workload("tiny", 1, 1, 1, 256, k=2, iters=3),
        2: Workload("small_multihead", 2, 1, 8, 4096),
        3: Workload("wan_720p_5s", 3, 1, 40, 75600),
        4: Workload("minimax_h3", 4, 1, 56, 73397),
        5: Workload("batched_repair", 5, 2, 24, 32768, dtype=torch.float16,
                    repair_budget=0.005),
    }
    w = table[config_id]
    kw = {}
    if H is not None:
        kw["H"] = H
    if S is not None:
        kw["S"] = S
    if B is not None:
        kw["B"] = B
    if kw:
        w = Workload(**{**w.__dict__, **kw})
    return w


def _outlier_mask(g: torch.Generator, B: int, H: int, S: int, n_out: int) -> torch.Tensor:
    """Boolean [B,S,H] mask with n_out distinct positions per (b,h)."""
    mask = torch.zeros(B, H, S, dtype=torch.bool)
    n_out = min(n_out, S)
    if n_out > 0:
        keys = torch.rand(B, H, S, generator=g)
        idx = torch.topk(keys, n_out, dim=-1).indices
        mask.scatter_(-1, idx, True)
    return mask.permute(0, 2, 1).contiguous()


def _ar1(g: torch.Generator, B: int, S: int, H: int, D: int, rho: float) -> torch.Tensor:
    """Unit-variance AR(1) process along the token axis, independent per (b,h,d).

    x_0 = eps_0 and x_t = rho * x_{t-1} + sqrt(1 - rho^2) * eps_t.
    """
    import numpy as np
    from scipy.signal import lfilter

    eps = torch.randn(B, S, H, D, generator=g)
    # filter along a contiguous last axis ([B,H,D,S]); the recurrence per
    # series is the same whatever the memory layout (torch does the copies:
    # they run on all cores)
    e = eps.permute(0, 2, 3, 1).contiguous().double().numpy()
    c = math.sqrt(1.0 - rho * rho)
    out = np.empty_like(e)
    out[..., 0] = e[..., 0]
    if S > 1:
        zi = (rho * e[..., 0])[..., None]                   # filter state [B,H,D,1]
        out[..., 1:], _ = lfilter([c], [1.0, -rho], e[..., 1:], axis=-1, zi=zi)
    return torch.from_numpy(out).float().permute(0, 3, 1, 2).contiguous()


def generate(w: Workload, device: str | torch.device = "cpu"):
    """Draw (q, k, v) as [B,S,H,D] tensors of ``w.dtype`` on ``device``.

    The draws happen on the CPU with a seeded generator, so the values do not
    depend on the device they are later moved to.
    """
    g = torch.Generator().manual_seed(SEED_BASE + w.config_id)
    B, H, S, D = w.B, w.H, w.S, w.D
    cid = w.config_id
    if cid == 1:
        q = torch.randn(B, S, H, D, generator=g)
        k = torch.randn(B, S, H, D, generator=g)
        z = torch.randn(B, S, H, D, generator=g)
        off = 2.0 * torch.randn(B, 1, H, D, generator=g)
        mask = _outlier_mask(g, B, H, S, 4)
        v = torch.where(mask.unsqueeze(-1), 20.0 * z, z) + off
    elif cid in (2, 4):
        q = torch.randn(B, S, H, D, generator=g)
        k = torch.randn(B, S, H, D, generator=g)
        qs = 0.5 + 1.5 * torch.rand(B, 1, H, 1, generator=g)
        ks = 0.5 + 1.5 * torch.rand(B, 1, H, 1, generator=g)
        q = q * qs
        k = k * ks
        z = torch.randn(B, S, H, D, generator=g)
        off = 3.0 * torch.randn(B, 1, H, D, generator=g)
        n_out = max(1, round((0.005 if cid == 2 else 0.002) * S))
        mask = _outlier_mask(g, B, H, S, n_out)
        v = torch.where(mask.unsqueeze(-1), 30.0 * z, z) + off
    elif cid == 3:
        q = _ar1(g, B, S, H, D, 0.9)
        k = _ar1(g, B, S, H, D, 0.9)
        z = torch.randn(B, S, H, D, generator=g)
        mask = _outlier_mask(g, B, H, S, max(1, round(0.002 * S)))
        v = torch.where(mask.unsqueeze(-1), 50.0 * z, z)
    elif cid == 5:
        q = torch.randn(B, S, H, D, generator=g)
        k = torch.randn(B, S, H, D, generator=g)
        # Student-t with nu=3: z / sqrt(chi2_3 / 3), chi2_3 = sum of 3 squared normals
        z = torch.randn(B, S, H, D, generator=g)
        chi = torch.zeros(B, S, H, D)
        for _ in range(3):
            chi += torch.randn(B, S, H, D, generator=g) ** 2
        v = z / torch.sqrt(chi / 3.0)
    else:
        raise ValueError(f"unknown config {cid}")
    cast = lambda t: t.to(w.dtype).to(device)
    return cast(q), cast(k), cast(v)


def sample_rows(S: int, n: int, seed: int = 7) -> torch.Tensor:
    """A fixed, sorted sample of n query rows in [0, S), always including the ragged tail."""
    g = torch.Generator().manual_seed(seed)
    n = min(n, S)
    rows = set(torch.randperm(S, generator=g)[: max(0, n - 2)].tolist())
    rows.update({0, S - 1})
    return torch.tensor(sorted(rows), dtype=torch.int64)
