"""Plain CPU oracle for the VC-Attention forward pass.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  It shares no code with the HIP library (no kernels, headers,
helpers, tables or constant generators) and imports nothing from it.

What it computes, step by step, in NumPy float64 except where a step itself
defines a rounding (then the rounding is written out).  Sources, cited by page
title and section:

[ABS]  "VC-Attention: Value Smoothing and Softmax Casting for Low-bit
       Attention", section "Abstract (arXiv)" -- the method statement.
[HF]   "Hugging Face Introduces VC-Attention: Breakthrough Optimization for
       Low-bit Attention Mechanisms", section "Technical Breakthroughs and Core
       Innovations" -- one-line definitions of V-Smooth and ExpCast-FP8.
[OVC]  "Open VC Attention", section "Описание" (Description) -- per-block Q/K
       scales, per-head V scale, BF16 output, [B,S,H,128] FP16/BF16 inputs,
       non-causal, V residual repair with a budget such as 0.005.
[NUN]  "Nunchux AI lanza VC-Attention kernel para acelerar generacion de
       video" (reditua.com), paragraph 2 -- k-means per batch and head, the
       mean of each 128-token block subtracted, E4M3 residual.

Where the pages leave a step open, the reading taken is stated at the step
(they are also listed together in the design notes of the repository):

 R1  K is permuted together with V (non-causal attention is invariant to a
     joint key/value permutation); Q and the output keep the original order.
 R2  k-means runs on an integer sketch of V (exact arithmetic), squared-L2
     Lloyd iterations, seeded strided initialisation, ties to the lowest
     cluster, empty clusters keep their centroid.
 R3  Tokens are ordered by ascending cluster id, stable within a cluster.
 R4  Blocks are 128 permuted positions; the last block may be partial and its
     mean is over its real tokens only.
 R5  Q/K scales: one per 128-token block per (b,h), amax/448; V scale: one per
     (b,h) over the residual.
 R6  ExpCast: 8 codes per octave, the running row maximum maps to code 120
     (value 256), round half to even, clamp to [0, 126].
 R7  The running maximum is kept as an integer in the log2 domain, so every
     rescale is an exact power of two.
 R8  The row sum is the sum of the decoded E4M3 probabilities that the PV
     product consumes.
 R9  Mean restore adds r_b * mu_b per tile (r_b = that tile's row sum).
 R10 Repair: the ceil(beta*S) permuted positions with the largest residual
     error norm (ties to the smaller position) add back their E4M3-quantised
     error with its own per-(b,h) scale; their probabilities are not added to
     the row sum a second time.
 R11 Softmax scale defaults to fp32(1/sqrt(128)); output is bf16 (RNE).
 R15 4-bit residual ([NUN] paragraph 2 names NVFP4 beside E4M3), taken as
     OCP MXFP4: E2M1 codes, one power-of-two (E8M0) scale per channel and
     group of 32 consecutive permuted positions within a 128-key tile
     (positions 32u .. 32u+31 of the tile form group u), the scale being the
     smallest power of two X with max|R|/X <= 6, so nothing is clipped;
     values round half to even; no per-head scale (s_v = 1, mu' = mu).

Parity pins: every function here is pinned by tests under ``tests/`` that use
closed forms, brute force, library routines or invariants -- none is "parity
unpinned" except the end-to-end agreement with the authors' own kernels, for
which the pages give no code, no captured tensors and no worked example.
"""
from __future__ import annotations

from dataclasses import dataclass, field
import math

import numpy as np

F32 = np.float32
E4M3_MAX = 448.0
LOG2E_F32 = F32(math.log2(math.e))          # fp32 nearest to log2(e)
DEFAULT_SM_SCALE = F32(1.0 / math.sqrt(128.0))
BLOCK = 128
MASK64 = (1 << 64) - 1


# --------------------------------------------------------------------------
# OCP E4M3FN codec (the FP8 format the abstract [ABS] names: E4M3)
# --------------------------------------------------------------------------
def e4m3_decode(codes) -> np.ndarray:
    """Decode OCP E4M3FN bytes to float64.

    Layout s.eeee.mmm, exponent bias 7.  Exponent field 0 is subnormal
    (m * 2^-9); otherwise 2^(e-7) * (1 + m/8).  0x7F / 0xFF are NaN; there are
    no infinities.  Largest finite value 0x7E = 448.
    """
    c = np.asarray(codes).astype(np.int64)
    s = c >> 7
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def e4m3_encode(x) -> np.ndarray:
    """Encode to OCP E4M3FN with round-half-to-even, saturating at +-448.

    The sign bit is the sign of the input, also when the magnitude rounds to
    zero (so -0.0 and tiny negatives give 0x80).  NaN input is undefined.
    """
    x = np.asarray(x, dtype=np.float64)
    neg = np.signbit(x)
    a = np.abs(x)
    _, e = np.frexp(a)                 # a = f * 2^e with f in [0.5, 1)
    ex = np.maximum(e - 1, -6)         # floor(log2 a), clamped at the subnormal exponent
    quantum = np.ldexp(1.0, ex - 3)    # 3 mantissa bits
    val = np.rint(a / quantum) * quantum          # a/quantum is exact (power-of-two)
    val = np.minimum(val, E4M3_MAX)               # saturate (also +-inf)
    # value -> code
    sub = val < 2.0 ** -6
    _, ev = np.frexp(np.where(sub, 1.0, val))
    mant = np.where(sub, 0.0, (np.ldexp(np.where(sub, 1.0, val), 1 - ev) - 1.0) * 8.0)
    code = np.where(sub, val * 2.0 ** 9, (ev + 6) * 8 + mant)
    code = code.astype(np.int64) | np.where(neg, 0x80, 0)
    return code.astype(np.uint8)


# --------------------------------------------------------------------------
# OCP E2M1 (FP4) codec and MX groups (R15)
# --------------------------------------------------------------------------
E2M1_MAX = 6.0


def e2m1_decode(codes) -> np.ndarray:
    """E2M1 code (bit 3 sign, bits 2..1 exponent with bias 1, bit 0 mantissa) -> value."""
    c = np.asarray(codes, dtype=np.int64)
    e = (c >> 1) & 3
    m = (c & 1).astype(np.float64)
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, (e - 1).astype(np.int64)))
    return np.where(c & 8, -mag, mag)


def e2m1_encode(x) -> np.ndarray:
    """Nearest E2M1 code, ties to the even mantissa, saturating at +-6; the sign
    bit follows the input's sign (also when the magnitude rounds to 0)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E2M1_MAX)
    grid = e2m1_decode(np.arange(8))                    # 0, 0.5, 1, 1.5, 2, 3, 4, 6 (ascending)
    i = np.searchsorted(grid, a, side="left")           # first grid value >= a
    lo = np.clip(i - 1, 0, 7)
    hi = np.clip(i, 0, 7)
    dlo, dhi = a - grid[lo], grid[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((hi & 1) == 0))
    code = np.where(pick_hi, hi, lo)
    return (code | np.where(np.signbit(x), 8, 0)).astype(np.int64)


MX_GROUP = 32     # permuted positions per MXFP4 scale group (R15)


def mx_group_of_key(j) -> np.ndarray:
    """Group (0..3) of permuted position j within its 128-key tile: the runs
    of 32 consecutive positions 32u .. 32u+31 form group u (R15)."""
    return (np.asarray(j, dtype=np.int64) % BLOCK) // MX_GROUP


def mx_scale_exponent(amax) -> np.ndarray:
    """Smallest e with amax / 2^e <= 6 (exact), clamped to [-127, 127]; 0 if amax == 0."""
    a = np.asarray(amax, dtype=np.float64)
    e = np.zeros(a.shape, dtype=np.int64)
    nz = a > 0
    m, ex = np.frexp(a[nz] / E2M1_MAX)                  # a/6 = m * 2^ex, m in [0.5, 1)
    e[nz] = np.where(m == 0.5, ex - 1, ex)              # exact powers of two need no rounding up
    return np.clip(e, -127, 127)


def quantize_mxfp4(resid: np.ndarray):
    """R15: resid [S, D] fp32 (permuted order) -> codes [S, D] (E2M1) and
    exponents [nblk, D, 4] (scale of (tile, channel, group) = 2^e)."""
    S, D = resid.shape
    nblk = (S + BLOCK - 1) // BLOCK
    codes = np.zeros((S, D), dtype=np.int64)
    expo = np.zeros((nblk, D, 4), dtype=np.int64)
    grp = mx_group_of_key(np.arange(BLOCK))
    for b in range(nblk):
        rows = resid[b * BLOCK: min(S, (b + 1) * BLOCK)].astype(np.float64)
        gk = grp[:rows.shape[0]]
        for g in range(4):
            sel = gk == g
            if not np.any(sel):
                continue
            e = mx_scale_exponent(np.max(np.abs(rows[sel]), axis=0))          # [D]
            expo[b, :, g] = e
            codes[b * BLOCK + np.nonzero(sel)[0]] = e2m1_encode(rows[sel] / np.ldexp(1.0, e)[None, :])
    return codes, expo


def mxfp4_dequant(codes: np.ndarray, expo: np.ndarray) -> np.ndarray:
    """Values of quantize_mxfp4's output, [S, D] float64."""
    S, D = codes.shape
    grp = mx_group_of_key(np.arange(S) % BLOCK)
    e = expo[np.arange(S) // BLOCK][np.arange(S), :, grp]                     # [S, D]
    return e2m1_decode(codes) * np.ldexp(1.0, e)


def bf16_round(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), as float64."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    q = np.ldexp(1.0, np.maximum(e, -125) - 8)    # 8 significant bits
    with np.errstate(invalid="ignore"):
        r = np.rint(x / q) * q
    return np.where(np.isfinite(x), r, x)


# --------------------------------------------------------------------------
# Per-block amax quantisation (Q and K)  [OVC: per-block Q/K scales]
# --------------------------------------------------------------------------
def quantize_amax(x32: np.ndarray):
    """Quantise one block (any shape, float32 values) with one amax scale.

    a = max|x|.  a == 0: scale 1 and x*1 is encoded (all codes are +-0).
    Otherwise inv = fp32(448/a), scale = fp32(a/448), code = e4m3(fp32(x*inv)).
    Returns (codes uint8, scale float32).
    """
    x32 = np.asarray(x32, dtype=F32)
    a = F32(np.max(np.abs(x32))) if x32.size else F32(0)
    if a == 0:
        inv = F32(1.0)
        s = F32(1.0)
    else:
        inv = F32(448.0) / a
        s = a / F32(448.0)
    y = (x32 * inv).astype(F32)
    return e4m3_encode(y), F32(s)


def quantize_blocks(x32: np.ndarray, block: int = BLOCK):
    """Per 128-row block amax quantisation of an [S, D] float32 matrix.

    Returns (codes [S, D] uint8, scales [nblk] float32).
    """
    S = x32.shape[0]
    nblk = (S + block - 1) // block
    codes = np.empty(x32.shape, dtype=np.uint8)
    scales = np.empty(nblk, dtype=F32)
    for b in range(nblk):
        sl = slice(b * block, min(S, (b + 1) * block))
        codes[sl], scales[b] = quantize_amax(x32[sl])
    return codes, scales


# --------------------------------------------------------------------------
# V-Smooth clustering  [ABS: lightweight online clustering reorders value
# tokens; NUN: k-means per batch and head]; readings R2, R3
# --------------------------------------------------------------------------
def splitmix64(z: int) -> int:
    """One output of Vigna's SplitMix64 for the state value z (public definition)."""
    z = (z + 0x9E3779B97F4A7C15) & MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def sketch(v: np.ndarray) -> np.ndarray:
    """Integer sketch of one head's V [S, D]: exact power-of-two scaling.

    a = max|v|; shift = 7 - floor(log2 a); x = clamp(rne(v * 2^shift), -255, 255).
    All-zero V gives an all-zero sketch.
    """
    v = np.asarray(v, dtype=np.float64)
    a = float(np.max(np.abs(v))) if v.size else 0.0
    if a == 0.0:
        return np.zeros(v.shape, dtype=np.int64)
    _, e = math.frexp(a)               # a in [2^(e-1), 2^e)
    shift = 8 - e                      # = 7 - floor(log2 a)
    x = np.rint(np.ldexp(v, shift))
    return np.clip(x, -255, 255).astype(np.int64)


def init_positions(S: int, k: int, seed: int, bh: int) -> np.ndarray:
    """Seeded strided initial centroid positions t_c = floor(c*S/k) + phi."""
    stride = max(1, S // k)
    phi = splitmix64((seed ^ bh) & MASK64) % stride
    return np.array([(c * S) // k + phi for c in range(k)], dtype=np.int64)


def kmeans_assign(x: np.ndarray, cent: np.ndarray) -> np.ndarray:
    """argmin_c (|c|^2 - 2 x.c), ties to the lowest c.

    Every product and partial sum is an integer below 2^24 in magnitude, so
    the float64 matrix product is exact in any summation order.
    """
    xf = x.astype(np.float64)
    cf = cent.astype(np.float64)
    score = (cf * cf).sum(axis=1)[None, :] - 2.0 * (xf @ cf.T)
    return np.argmin(score, axis=1).astype(np.int64)      # first minimum


def kmeans_update(x: np.ndarray, assign: np.ndarray, cent: np.ndarray) -> np.ndarray:
    """New centroid = floor((2*sum + n) / (2n)) per coordinate (the mean rounded
    half up); a cluster with n == 0 keeps its centroid."""
    k = cent.shape[0]
    n = np.bincount(assign, minlength=k).astype(np.int64)
    onehot = np.zeros((x.shape[0], k), dtype=np.float64)
    onehot[np.arange(x.shape[0]), assign] = 1.0
    # integer sums of at most S terms of magnitude <= 255 (below 2^32 for
    # S <= 2^24): exact in float64 in any order
    sums = np.rint(onehot.T @ x.astype(np.float64)).astype(np.int64)
    new = cent.copy()
    nz = n > 0
    new[nz] = (2 * sums[nz] + n[nz, None]) // (2 * n[nz, None])
    return new


def kmeans(x: np.ndarray, k: int, iters: int, seed: int, bh: int):
    """Lloyd's k-means on the integer sketch; returns (assign, centroids, history).

    history holds the centroid array after init and after each update.
    """
    S = x.shape[0]
    if not 1 <= k <= S:
        raise ValueError("need 1 <= k <= S")
    cent = x[init_positions(S, k, seed, bh)].copy()
    hist = [cent.copy()]
    for _ in range(iters):
        a = kmeans_assign(x, cent)
        cent = kmeans_update(x, a, cent)
        hist.append(cent.copy())
    return kmeans_assign(x, cent), cent, hist


def cluster_perm(assign: np.ndarray) -> np.ndarray:
    """perm[p] = original token at permuted position p: ascending cluster, stable."""
    return np.argsort(assign, kind="stable").astype(np.int64)


# --------------------------------------------------------------------------
# Block means, residual quantisation, repair  [ABS, NUN, OVC]; R4, R5, R10
# --------------------------------------------------------------------------
@dataclass
class HeadV:
    """Everything prepare_v produces for one (b, h); positions are permuted."""

    assign: np.ndarray          # [S] cluster id per ORIGINAL token
    perm: np.ndarray            # [S] original token at permuted position p
    mean: np.ndarray            # [nblk, D] block means (fp32 values)
    resid: np.ndarray           # [S, D] residual R (fp32 values, permuted order)
    v8: np.ndarray              # [S, D] E4M3 codes of the residual
    v_scale: np.float32
    rep_pos: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int64))  # sorted permuted positions
    rep_e8: np.ndarray = field(default_factory=lambda: np.zeros((0, 128), np.uint8))
    rep_scale: np.float32 = F32(1.0)
    rep_norm2: np.ndarray | None = None     # [S] squared error norm (fp64)
    centroids: np.ndarray | None = None
    v_format: str = "e4m3"                  # "e4m3" (per-head scale) or "mxfp4" (R15)
    v4: np.ndarray | None = None            # [S, D] E2M1 codes (mxfp4)
    v4_exp: np.ndarray | None = None        # [nblk, D, 4] scale exponents (mxfp4)

    def v_values(self) -> np.ndarray:
        """Dequantised residual the P.V product consumes, [S, D] float64."""
        if self.v_format == "mxfp4":
            return mxfp4_dequant(self.v4, self.v4_exp)
        return float(self.v_scale) * e4m3_decode(self.v8)


def block_means(vp: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """mu_b = fp32(fp64(sum of the block's real tokens) / n_b), per channel."""
    S, D = vp.shape
    nblk = (S + block - 1) // block
    mu = np.empty((nblk, D), dtype=F32)
    for b in range(nblk):
        blk = vp[b * block: min(S, (b + 1) * block)]
        mu[b] = (blk.sum(axis=0, dtype=np.float64) / np.float64(blk.shape[0])).astype(F32)
    return mu


def repair_count(beta: float, S: int) -> int:
    """Number of repaired tokens: ceil(beta * S) with beta taken as given (fp32 -> fp64)."""
    if beta <= 0:
        return 0
    return min(S, int(math.ceil(float(np.float64(F32(beta))) * S)))


def prepare_v_head(v: np.ndarray, *, smooth: bool = True, k: int = 32, iters: int = 5,
                   seed: int = 0, bh: int = 0, repair_budget: float = 0.0,
                   quant: bool = True, v_format: str = "e4m3") -> HeadV:
    """V-Smooth for one head, V given as [S, D] float64 (exact bf16/fp16 values).

    1. cluster (integer k-means on the sketch) and order tokens by cluster;
    2. subtract each 128-position block's mean: R = fp32(v - mu);
    3. quantise R with one per-head amax scale to E4M3 (v_format="e4m3"), or
       to MXFP4 with one power-of-two scale per 32-key group (R15; no repair);
    4. optional repair set (R10).
    quant=False keeps R unquantised (v8 then holds no codes; used by the
    identity tests through attend_head's quant switch).
    """
    S, D = v.shape
    if smooth:
        x = sketch(v)
        if not np.any(x):
            assign = np.zeros(S, dtype=np.int64)
            cent = None
        else:
            assign, cent, _ = kmeans(x, k, iters, seed, bh)
        perm = cluster_perm(assign)
    else:
        assign = np.zeros(S, dtype=np.int64)
        perm = np.arange(S, dtype=np.int64)
        cent = None
    vp = v[perm]
    nblk = (S + BLOCK - 1) // BLOCK
    if smooth:
        mu = block_means(vp)
    else:
        mu = np.zeros((nblk, D), dtype=F32)
    mu_rows = np.repeat(mu.astype(np.float64), BLOCK, axis=0)[:S]
    resid = (vp - mu_rows).astype(F32)               # single rounding of the exact difference
    if not quant:
        return HeadV(assign, perm, mu, resid, np.zeros((S, D), np.uint8), F32(1.0), centroids=cent)
    if v_format == "mxfp4":
        if repair_count(repair_budget, S) > 0:
            raise ValueError("the MXFP4 residual has no repair")
        v4, v4e = quantize_mxfp4(resid)
        return HeadV(assign, perm, mu, resid, np.zeros((S, D), np.uint8), F32(1.0), centroids=cent,
                     v_format="mxfp4", v4=v4, v4_exp=v4e)
    v8, s_v = quantize_amax(resid)
    hv = HeadV(assign, perm, mu, resid, v8, s_v, centroids=cent)
    n_rep = repair_count(repair_budget, S)
    if n_rep > 0:
        deq = (F32(s_v) * e4m3_decode(v8).astype(F32)).astype(F32)
        err = (resid - deq).astype(F32)
        e64 = err.astype(np.float64)
        norm2 = np.zeros(S, dtype=np.float64)
        for d in range(D):                             # sequential fp64 sum over d
            norm2 = norm2 + e64[:, d] * e64[:, d]
        order = np.lexsort((np.arange(S), -norm2))     # largest first, ties -> smaller p
        pos = np.sort(order[:n_rep])
        e8, s_e = quantize_amax(err[pos])
        hv.rep_pos, hv.rep_e8, hv.rep_scale, hv.rep_norm2 = pos, e8, s_e, norm2
    return hv


@dataclass
class HeadQK:
    """prepare_qk's products for one (b, h)."""

    q8: np.ndarray          # [S, D] codes, original order
    q_scale: np.ndarray     # [nblk] per 128-token block of Q (original order)
    k8: np.ndarray          # [S, D] codes, PERMUTED order (row p = token perm[p])
    k_scale: np.ndarray     # [nblk] per permuted 128-position block


def prepare_qk_head(q: np.ndarray, k: np.ndarray, perm: np.ndarray) -> HeadQK:
    """Per-block amax E4M3 quantisation of Q (original order) and K (gathered by perm)."""
    q8, qs = quantize_blocks(q.astype(F32))
    k8, ks = quantize_blocks(k[perm].astype(F32))
    return HeadQK(q8, qs, k8, ks)


# --------------------------------------------------------------------------
# ExpCast  [ABS: log-domain scores -> E4M3 probability codes with one FMA;
# HF: no FP32 exponential and no format conversion]; R6, R7
# --------------------------------------------------------------------------
def expcast_codes(acc32: np.ndarray, sigma8, m_int) -> np.ndarray:
    """code = clamp(rne(fp32(acc*8*sigma + (120 - 8*M))), 0, 126).

    acc32: fp32 scores [R, n]; sigma8: fp32 8*sigma (per row [R,1] or scalar);
    m_int: integer running max per row [R,1].  The E4M3 value of the code is a
    piecewise-linear stand-in for 256 * 2^(acc*sigma - M).
    """
    x = acc32.astype(np.float64) * np.asarray(sigma8, np.float64) + (120.0 - 8.0 * np.asarray(m_int, np.float64))
    x = x.astype(F32)
    return np.clip(np.rint(x.astype(np.float64)), 0, 126).astype(np.int64)


# --------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------
def sigma_of(s_q, s_k, sm_scale) -> np.ndarray:
    """sigma = fp32(fp32(fp32(s_q * s_k) * sm_scale) * log2 e)."""
    return ((np.asarray(s_q, F32) * np.asarray(s_k, F32)).astype(F32) * F32(sm_scale)).astype(F32) * LOG2E_F32


def attend_head(hq: HeadQK, hv: HeadV, rows=None, *, sm_scale=DEFAULT_SM_SCALE,
                pcast: str = "expcast", quant: bool = True, q_raw=None, k_raw=None,
                mode: str = "online", int_max: bool = True, repair: bool = True,
                code_delta=None, m_delta=None, ties=None, tie_width: float = 2e-3) -> np.ndarray:
    """Online-softmax attention for the given query rows of one head; returns float64 [R, D].

    Tiles of 128 permuted keys are visited in ascending order [ABS: the online
    softmax row sum].  Per tile b, for every query row:
      acc   = Q8 . K8^T (exact, rounded to fp32)
      sigma = fp32(fp32(fp32(s_q*s_k)*sm_scale)*log2 e)
      M_new = max(M, ceil(fp32(max_j acc*sigma)))          (R7, integer)
      alpha = 2^(M - M_new)
      code  = ExpCast(acc, 8*sigma, M_new);  P = dec(code)  (R6)
      r_b   = sum_j P                                        (R8)
      l     = alpha*l + r_b
      num   = alpha*num + P . (s_v*dec(V8)) + r_b*mu_b      (R9)
    Repair (R10): num += s_e * sum_{p in W} dec(code_ip) * dec(e8_p), with the
    codes taken against the final M and not added to l.
    out = num / l.

    Switches (self-tests and ablations only):
      pcast="expcast" | "exp_e4m3" (exact exp2 then an E4M3 cast) | "exact"
      (exact exp2, no probability quantisation);
      quant=False uses q_raw/k_raw (float64, K in permuted order) and the
      unquantised residual, all scales 1;
      mode="two_pass" takes every code against the final maximum;
      int_max=False keeps a real-valued running maximum (pcast != "expcast").

    Rounding-decision hooks (parity tests only; they change no result unless
    given): the matrix core sums a score's 128 products in its own order, so
    its fp32 score can differ from this one (exact, rounded once) by a few
    ulps, and an ExpCast argument or a tile maximum that lies that close to a
    rounding boundary can round the other way on the GPU.
      ties: a list that receives, for the first requested row, every such
        near-boundary decision as (kind, b, j, delta, distance): kind "code"
        for key j of tile b whose fp32 ExpCast argument is within tie_width
        of a half-integer (delta = +1 if it rounded down, -1 if up), kind
        "max" for tile b whose fp32 max*sigma is within tie_width of an
        integer (delta = the other possible ceiling minus this one; j = -1);
      code_delta {(b, j): delta}: key j of tile b takes code + delta;
      m_delta {b: delta}: tile b's ceil(max*sigma) is taken + delta.
    """
    S, D = hv.resid.shape
    nblk = (S + BLOCK - 1) // BLOCK
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rows.size
    if quant:
        Qd = e4m3_decode(hq.q8[rows])
        Kd = e4m3_decode(hq.k8)
        Vd = hv.v_values()
        s_q = hq.q_scale[rows // BLOCK][:, None]
        s_k = hq.k_scale
    else:
        Qd = np.asarray(q_raw, np.float64)[rows]
        Kd = np.asarray(k_raw, np.float64)
        Vd = hv.resid.astype(np.float64)
        s_q = np.ones((R, 1), F32)
        s_k = np.ones(nblk, F32)
    mu = hv.mean.astype(np.float64)

    def scores(b):
        ks = slice(b * BLOCK, min(S, (b + 1) * BLOCK))
        acc = Qd @ Kd[ks].T
        if quant:
            acc = acc.astype(F32)          # exact value rounded once to fp32
        sig = sigma_of(s_q, s_k[b], sm_scale) if quant else \
            np.full((R, 1), float(np.float64(sm_scale)) * math.log2(math.e))
        return ks, acc, sig

    def probs(acc, sig, M, b=None):
        if pcast == "expcast":
            s8 = (F32(8) * sig).astype(F32)
            c = expcast_codes(acc, s8, M)
            if ties is not None and b is not None:
                x = (acc[:1].astype(np.float64) * np.asarray(s8, np.float64)[:1] +
                     (120.0 - 8.0 * np.asarray(M, np.float64)[:1])).astype(F32).astype(np.float64)[0]
                fr = x - np.floor(x)
                for j in np.nonzero((x >= 0) & (np.abs(fr - 0.5) < tie_width))[0]:
                    ties.append(("code", b, int(j), 1 if fr[j] < 0.5 else -1, float(abs(fr[j] - 0.5))))
            if code_delta and b is not None:
                c = c.copy()
                for (tb, j), dlt in code_delta.items():
                    if tb == b:
                        c[:, j] = np.clip(c[:, j] + dlt, 0, 126)
            return e4m3_decode(c)
        t = acc.astype(np.float64) * np.asarray(sig, np.float64)
        p = 256.0 * np.exp2(t - M)
        return e4m3_decode(e4m3_encode(p)) if pcast == "exp_e4m3" else p

    def tile_max(acc, sig, b=None):
        m = (np.max(acc, axis=1, keepdims=True).astype(F32) * sig).astype(F32) if quant else \
            np.max(acc * np.asarray(sig, np.float64), axis=1, keepdims=True)
        if not int_max:
            return m.astype(np.float64)
        c = np.ceil(m.astype(np.float64))
        if ties is not None and b is not None:
            f = float(m[0, 0]) - math.floor(float(m[0, 0]))
            if 0 < f < tie_width or f == 0.0:
                ties.append(("max", b, -1, 1 if f == 0.0 else -1, f))
            elif f > 1.0 - tie_width:
                ties.append(("max", b, -1, 1, 1.0 - f))
        if m_delta and b in m_delta:
            c = c + m_delta[b]
        return c

    M = np.full((R, 1), -np.inf)
    if mode == "two_pass":
        for b in range(nblk):
            _, acc, sig = scores(b)
            M = np.maximum(M, tile_max(acc, sig))
    l = np.zeros((R, 1))
    num = np.zeros((R, D))
    for b in range(nblk):
        ks, acc, sig = scores(b)
        if mode == "online":
            Mn = np.maximum(M, tile_max(acc, sig, b))
            alpha = np.where(np.isfinite(M), np.exp2(M - Mn), 0.0)
            l *= alpha
            num *= alpha
            M = Mn
        P = probs(acc, sig, M, b)
        r = P.sum(axis=1, keepdims=True)
        l += r
        num += P @ Vd[ks] + r * mu[b][None, :]
    if repair and quant and hv.rep_pos.size:
        W = hv.rep_pos
        accW = (Qd @ Kd[W].T).astype(F32)
        sigW = sigma_of(s_q, s_k[W // BLOCK][None, :], sm_scale)
        if pcast == "expcast":
            PW = e4m3_decode(expcast_codes(accW, (F32(8) * sigW).astype(F32), M))
        else:
            PW = probs(accW, sigW, M)
        num += float(hv.rep_scale) * (PW @ e4m3_decode(hv.rep_e8))
    return num / l


def attention_exact(q: np.ndarray, k: np.ndarray, v: np.ndarray, sm_scale=DEFAULT_SM_SCALE,
                    rows=None) -> np.ndarray:
    """Exact fp64 softmax attention softmax(q k^T * sm_scale) v for one head [S, D]."""
    q = np.asarray(q, np.float64)
    if rows is not None:
        q = q[np.asarray(rows)]
    s = (q @ np.asarray(k, np.float64).T) * float(np.float64(sm_scale))
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return (p @ np.asarray(v, np.float64)) / p.sum(axis=1, keepdims=True)


# --------------------------------------------------------------------------
# Whole tensors [B, S, H, D]
# --------------------------------------------------------------------------
@dataclass
class Prepared:
    B: int
    S: int
    H: int
    heads_v: dict
    heads_qk: dict


def prepare(q, k, v, *, smooth=True, kc=32, iters=5, seed=0, repair_budget=0.0,
            heads=None) -> Prepared:
    """prepare_v then prepare_qk for every (b, h) (or only the listed (b, h) pairs)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, S, H, D = q.shape
    assert D == 128
    hv, hq = {}, {}
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    for (b, h) in todo:
        hv[(b, h)] = prepare_v_head(v[b, :, h], smooth=smooth, k=kc, iters=iters, seed=seed,
                                    bh=b * H + h, repair_budget=repair_budget)
        hq[(b, h)] = prepare_qk_head(q[b, :, h], k[b, :, h], hv[(b, h)].perm)
    return Prepared(B, S, H, hv, hq)


def attention(prep: Prepared, rows=None, sm_scale=DEFAULT_SM_SCALE, heads=None) -> dict:
    """bf16-rounded output rows per (b, h): {(b,h): float64 [R, D]}."""
    out = {}
    for key in (heads if heads is not None else prep.heads_v.keys()):
        o = attend_head(prep.heads_qk[key], prep.heads_v[key], rows, sm_scale=sm_scale)
        out[key] = bf16_round(o)
    return out


def rel_l2(a, b) -> float:
    """||a - b||_2 / ||b||_2 in float64."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))
