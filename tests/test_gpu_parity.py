"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bit-exact: cluster assignments, the permutation, Q/K/V E4M3 codes and their
scales, block means, the repair set and its codes.  Floating point: the bf16
output within relative L2 <= 5e-3 of the oracle's (the two differ only by
the FP8 MFMA's fp32 accumulation order and the rare probability codes that
this flips), and within 4% of exact fp64 attention.
"""
import itertools
import sys

import numpy as np
import pytest
import torch

import bit_attention_video_vc_amd as vc
import synth
from oracle import vc_oracle as O

pytestmark = pytest.mark.gpu

TOL_ORACLE = 5e-3
# every query row on its own, relative L2 against the oracle's row: a head can
# meet the per-head bound with one 16-query sub-tile far off (at S=4096 a
# 5% error in 16 rows adds only ~0.3% to the head's norm)
TOL_ROW = 2e-2
# A row above TOL_ROW passes only as the oracle's own row with one or two
# near-boundary rounding decisions taken the other way (explain_row): the
# matrix core sums a score's 128 FP8 products in its own order, so an ExpCast
# argument within ~1e-4 of a half-integer (or a tile maximum that close to an
# integer) can round the other way; one flipped code of a dominant key moves
# its row by a few percent.  The GPU row must then match that alternative
# within TOL_FLIP.
TOL_FLIP = 5e-3
# the accuracy target against exact fp64 attention
TOL_EXACT = 0.04
# The kernel must add nothing to the method's own error: its rel-L2 against
# exact attention is at most 1.02x the oracle's on the same rows plus 1e-3.
# Where the oracle itself (the method) is above 4% on a case's rows -- zero-
# mean V makes the output a small average of noise (|out| ~ 2% of |v|) and
# E4M3 Q, K, V and ExpCast then cost ~2.5-3% each -- the 4% target is
# reported as not met for that case instead of being gated.
EXACT_RATIO, EXACT_SLACK = 1.02, 1e-3


def say(msg):
    print(f"[gpu-parity] {msg}", flush=True)
    sys.stdout.flush()


# ---- unpacking of the documented tile formats ---------------------------------
def _row_tile_index():
    r = np.arange(128)[:, None]
    d = np.arange(128)[None, :]
    return ((((r // 16) * 2 + (d % 32) // 16) * 64 + (r % 16) + 16 * (d // 32)) * 16) + d % 16


def _tr_tile_index():
    j = np.arange(128)[:, None]
    d = np.arange(128)[None, :]
    g = (j % 16) // 4
    i = 4 * (j // 16) + j % 4
    return ((((d // 16) * 2 + i // 16) * 64 + (d % 16) + 16 * g) * 16) + i % 16


ROW_IDX = _row_tile_index()
TR_IDX = _tr_tile_index()


def _mxfp4_tile_index():
    """Byte, nibble shift and scale byte of (position j, channel d) in an MXFP4
    tile slot, from the layout documented with the C ABI: positions 32u..32u+31
    form group u, position 32u + n is nibble n of lane group u."""
    j = np.arange(128)[:, None]
    d = np.arange(128)[None, :]
    u, n = j // 32, j % 32
    lane = u * 16 + d % 16
    byte = ((d // 16) * 64 + lane) * 16 + n // 2
    shift = 4 * (n % 2)
    uu = np.arange(4)[None, :, None]
    dd = np.arange(128)[:, None, None]
    sbyte = (8192 + (uu * 16 + dd % 16) * 8 + dd // 16)[:, :, 0]        # [d, u]
    return byte, shift, sbyte


def _mx_row_of_position():
    """Row of a k8 tile that holds permuted position p in an MXFP4 workspace:
    the inverse of the documented mx(r) = 64(t/4) + 16g + 4(t%4) + i for row
    r = 16t + 4g + i."""
    r = np.arange(128)
    t, g, i = r // 16, (r % 16) // 4, r % 4
    pos = 64 * (t // 4) + 16 * g + 4 * (t % 4) + i
    assert np.array_equal(np.sort(pos), np.arange(128))
    row = np.empty(128, np.int64)
    row[pos] = r
    return row


MX_ROW_OF_POS = _mx_row_of_position()


MX_BYTE, MX_SHIFT, MX_SBYTE = _mxfp4_tile_index()


def unpack_mxfp4(raw: np.ndarray, nblk: int):
    """nblk MXFP4 tile slots -> E2M1 codes [nblk*128, 128] and exponents [nblk, 128, 4]."""
    t = raw.reshape(nblk, 16384)
    codes = (t[:, MX_BYTE] >> MX_SHIFT) & 15                             # [nblk, 128, 128]
    expo = t[:, MX_SBYTE].astype(np.int64) - 127                        # [nblk, d, u]
    return codes.reshape(-1, 128).astype(np.int64), expo


def muop_rows(nblk):
    return 16 * ((nblk + 3 + 15) // 16)


def decode_muop(raw: np.ndarray, nblk: int):
    """Restore-operand rows -> (hi, lo) bf16 parts as float32 [nblk_pad, 128].

    Row 16G + 2*dt + h, lane l (8 bytes at 8*l): 4 bf16 values for channel
    16*dt + l%16 and blocks 16G + 4*(l//16) + j."""
    u16 = raw.view(np.uint16).reshape(-1, 8, 2, 4, 16, 4)      # [G, dt, h, lane//16, lane%16, j]
    f = (u16.astype(np.uint32) << 16).view(np.float32)
    out = f.transpose(2, 0, 3, 5, 1, 4).reshape(2, -1, 128)   # [h, 16G + 4*(lane//16) + j, 16*dt + lane%16]
    return out[0], out[1]


def expected_muop(mean: np.ndarray, v_scale: float):
    """mu/s_v in fp32, split into bf16 high part (round to nearest even) and bf16 low part."""
    mp = torch.from_numpy(mean.astype(np.float32)) / torch.tensor(np.float32(v_scale))
    hi = mp.to(torch.bfloat16).float()
    lo = (mp - hi).to(torch.bfloat16).float()
    return hi.numpy(), lo.numpy()


def unpack_tiles(raw: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """[..., ntiles*16384] bytes -> [..., ntiles*128, 128] codes (row r / key j, channel d)."""
    lead = raw.shape[:-1]
    t = raw.reshape(*lead, -1, 16384)
    out = t[..., idx]                                  # [..., ntiles, 128, 128]
    return out.reshape(*lead, -1, 128)


class GpuRun:
    def __init__(self, q, k, v, opts, sm_scale=0.0, out=None):
        self.q, self.k, self.v, self.opts = q, k, v, opts
        self.lay = vc.vc_workspace_layout(v, opts)
        self.ws = torch.full((self.lay.total,), 0x7F, dtype=torch.uint8, device=v.device)  # E4M3 NaN poison
        self.out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device) if out is None else out
        vc.vc_prepare_v(v, opts, self.ws)
        vc.vc_prepare_qk(q, k, opts, self.ws)
        vc.vc_attention_fwd(self.out, opts, self.ws, sm_scale)
        torch.cuda.synchronize()
        B, S, H = (q.shape[0], q.shape[1], q.shape[2]) if q.dim() == 4 else (1, q.shape[0], q.shape[1])
        self.B, self.S, self.H = B, S, H

    def region(self, name, dtype, count):
        off = getattr(self.lay, name)
        n = count * torch.tensor([], dtype=dtype).element_size()
        return self.ws[off:off + n].view(dtype).cpu().numpy()

    def head_region(self, name, dtype, per_head, bh):
        """One head's slice of a per-head workspace region (per_head elements each)."""
        es = torch.tensor([], dtype=dtype).element_size()
        off = getattr(self.lay, name) + bh * per_head * es
        return self.ws[off:off + per_head * es].view(dtype).cpu().numpy()

    def head_view(self, bh):
        """Every prepared product of head bh, unpacked from the documented formats."""
        S, L = self.S, self.lay
        nb, npad = L.nblk, L.nrep_pad
        v = {
            "perm": self.head_region("perm", torch.int32, S, bh),
            "assign": self.head_region("assign", torch.int32, S, bh),
            "q8": unpack_tiles(self.head_region("q8", torch.uint8, nb * 16384, bh), ROW_IDX),
            "k8": unpack_tiles(self.head_region("k8", torch.uint8, nb * 16384, bh), ROW_IDX),
            "v8": unpack_tiles(self.head_region("v8", torch.uint8, nb * 16384, bh), TR_IDX),
            "q_scale": self.head_region("q_scale", torch.float32, nb, bh),
            "k_scale": self.head_region("k_scale", torch.float32, nb, bh),
            "v_mean": self.head_region("v_mean", torch.float32, nb * 128, bh).reshape(nb, 128),
            "hdr": self.head_region("hdr", torch.float32, 8, bh),
            "v_muop": self.head_region("v_muop", torch.uint8, muop_rows(nb) * 512, bh),
        }
        if npad:
            v["rep_pos"] = self.head_region("rep_pos", torch.int32, npad, bh)
            v["rep_e8"] = unpack_tiles(self.head_region("rep_e8", torch.uint8, npad * 128, bh), TR_IDX)
            v["rep_k8"] = unpack_tiles(self.head_region("rep_k8", torch.uint8, npad * 128, bh), ROW_IDX)
        return v


def _np(t):
    return t.detach().double().cpu().numpy()


def explain_row(hq, hv, row, got, sm):
    """The near-boundary rounding decisions of the oracle's row `row` (at most
    two, among the eight nearest) that, taken the other way, give `got`
    within TOL_FLIP; None if none do."""
    ties = []
    O.attend_head(hq, hv, np.array([row]), sm_scale=sm, ties=ties)
    cands = sorted(ties, key=lambda t: t[4])[:8]
    for n in (1, 2):
        for sel in itertools.combinations(cands, n):
            cd = {(b, j): d for (kind, b, j, d, _) in sel if kind == "code"}
            md = {b: d for (kind, b, j, d, _) in sel if kind == "max"}
            alt = O.bf16_round(O.attend_head(hq, hv, np.array([row]), sm_scale=sm, code_delta=cd, m_delta=md))[0]
            e = O.rel_l2(got, alt)
            if e <= TOL_FLIP:
                return sel, e
    return None


def check_against_oracle(q, k, v, *, smooth=True, kc=32, iters=5, seed=0, beta=0.0, rows=None, heads=None,
                         sm_scale=0.0, name="", target_met=None, v_format="e4m3", out=None):
    """Run the GPU path and compare every prepared product and the output with the oracle.

    Output gates per head: rel-L2 vs the oracle <= TOL_ORACLE, every row's
    rel-L2 vs the oracle's row <= TOL_ROW (or the row explained by
    explain_row within TOL_FLIP), and rel-L2 vs exact fp64 attention
    <= EXACT_RATIO x the oracle's own + EXACT_SLACK.  The 4% target vs exact
    is gated on every head where the oracle meets it; a head where the oracle
    itself is above it is a miss of the method, listed in run.target_misses.
    target_met=True asserts there is no such miss, False that the case
    does miss (so a case labelled "not met" is one where the method is above
    4%), None reports only."""
    say(f"{name}: shape={tuple(q.shape)} dtype={q.dtype} smooth={smooth} k={kc} T={iters} beta={beta} "
        f"v_format={v_format}")
    fmt = vc.VC_V_MXFP4 if v_format == "mxfp4" else vc.VC_V_E4M3
    opts = vc.v_opts(smooth, kc, iters, seed, beta, fmt)
    run = GpuRun(q, k, v, opts, sm_scale, out=out)
    B, S, H = run.B, run.S, run.H
    q4, k4, v4, o4 = (t if t.dim() == 4 else t[None] for t in (q, k, v, run.out))
    sm = O.DEFAULT_SM_SCALE if sm_scale == 0.0 else np.float32(sm_scale)
    heads = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    errs, errs_ex, errs_or_ex, row_errs, misses = [], [], [], [], []
    for (b, h) in heads:
        bh = b * H + h
        qn, kn, vn = (_np(t[b, :, h]) for t in (q4, k4, v4))     # this head only, as float64
        hv = O.prepare_v_head(vn, smooth=smooth, k=kc, iters=iters, seed=seed, bh=bh, repair_budget=beta,
                              v_format=v_format)
        hq = O.prepare_qk_head(qn, kn, hv.perm)
        tag = f"{name} (b={b},h={h})"
        gv = run.head_view(bh)
        nb = run.lay.nblk
        assert np.array_equal(gv["assign"], hv.assign), tag + " assign"
        assert np.array_equal(gv["perm"], hv.perm), tag + " perm"
        assert np.array_equal(gv["q8"][:S], hq.q8), tag + " q8"
        assert not gv["q8"][S:].any(), tag + " q8 padding"
        assert np.array_equal(gv["q_scale"], hq.q_scale), tag + " q_scale"
        k8 = gv["k8"]
        if v_format == "mxfp4":
            # rows relabelled so every FP4 lane group holds one 32-position group
            k8 = k8.reshape(nb, 128, 128)[:, MX_ROW_OF_POS].reshape(nb * 128, 128)
        assert np.array_equal(k8[:S], hq.k8), tag + " k8"
        assert not k8[S:].any(), tag + " k8 padding"
        assert np.array_equal(gv["k_scale"], hq.k_scale), tag + " k_scale"
        if v_format == "mxfp4":
            codes, expo = unpack_mxfp4(run.head_region("v8", torch.uint8, nb * 16384, bh), nb)
            assert np.array_equal(codes[:S], hv.v4), tag + " E2M1 codes"
            assert not codes[S:].any(), tag + " E2M1 padding"
            # groups with no real key (past S in the last tile) carry no defined scale
            last_real = S - 128 * (nb - 1)
            live = np.ones((nb, 128, 4), bool)
            for u in range(4):
                live[nb - 1, :, u] = 32 * u < last_real
            assert np.array_equal(expo[live], hv.v4_exp[live]), tag + " E8M0 scales"
        else:
            assert np.array_equal(gv["v8"][:S], hv.v8), tag + " v8"
            assert not gv["v8"][S:].any(), tag + " v8 padding"
        assert np.array_equal(gv["v_mean"], hv.mean), tag + " block means"
        assert gv["hdr"][0] == hv.v_scale, tag + " v_scale"
        mhi, mlo = decode_muop(gv["v_muop"], nb)
        ehi, elo = expected_muop(hv.mean, hv.v_scale)
        assert np.array_equal(mhi[:nb], ehi) and np.array_equal(mlo[:nb], elo), tag + " restore operands"
        assert not mhi[nb:].any() and not mlo[nb:].any(), tag + " restore operand padding"
        if beta > 0:
            n = hv.rep_pos.size
            assert np.array_equal(gv["rep_pos"][:n], hv.rep_pos), tag + " repair set"
            assert np.all(gv["rep_pos"][n:] == -1)
            assert np.array_equal(gv["rep_e8"][:n], hv.rep_e8), tag + " repair codes"
            assert np.array_equal(gv["rep_k8"][:n], hq.k8[hv.rep_pos]), tag + " repair K rows"
            assert gv["hdr"][6] == hv.rep_scale, tag + " repair scale"
        r = np.arange(S) if rows is None else np.asarray(rows)
        ref = O.bf16_round(O.attend_head(hq, hv, r, sm_scale=sm))
        got = o4[b, :, h].float().cpu().numpy()[r].astype(np.float64)
        assert np.all(np.isfinite(got)), tag + " non-finite output"
        e = O.rel_l2(got, ref)
        row_e = np.linalg.norm(got - ref, axis=1) / np.maximum(np.linalg.norm(ref, axis=1), 1e-300)
        ex = O.attention_exact(qn, kn, vn, sm_scale=sm, rows=r)
        e_ex = O.rel_l2(got, ex)
        e_or_ex = O.rel_l2(ref, ex)
        errs.append(e)
        errs_ex.append(e_ex)
        errs_or_ex.append(e_or_ex)
        row_errs.append(float(row_e.max()))
        assert e <= TOL_ORACLE, f"{tag}: rel-L2 vs oracle {e:.3e}"
        for i in np.nonzero(row_e > TOL_ROW)[0]:
            expl = explain_row(hq, hv, int(r[i]), got[i], sm)
            assert expl is not None, \
                f"{tag}: row {int(r[i])} rel-L2 vs oracle {row_e[i]:.3e}, not a near-boundary rounding flip"
            say(f"{tag}: row {int(r[i])} rel-L2 vs oracle {row_e[i]:.3e} is the oracle with "
                f"{[t[:4] for t in expl[0]]} rounded the other way (then {expl[1]:.1e})")
        assert e_ex <= EXACT_RATIO * e_or_ex + EXACT_SLACK, \
            f"{tag}: rel-L2 vs exact {e_ex:.3e}, the oracle's own {e_or_ex:.3e}"
        if e_or_ex <= TOL_EXACT:
            assert e_ex <= TOL_EXACT, f"{tag}: rel-L2 vs exact {e_ex:.3e} (oracle {e_or_ex:.3e})"
        else:
            misses.append((tag, e_ex, e_or_ex))
    say(f"{name}: max rel-L2 vs oracle {max(errs):.3e} (worst row {max(row_errs):.3e}), vs exact fp64 "
        f"{max(errs_ex):.3e} (oracle's own {max(errs_or_ex):.3e})")
    for tag, e_ex, e_or_ex in misses:
        say(f"{tag}: 4% target vs exact not met by the method: GPU {e_ex:.3e}, oracle {e_or_ex:.3e}")
    if target_met is True:
        assert not misses, f"{name}: the 4% target is missed: {misses}"
    elif target_met is False:
        assert misses, f"{name}: labelled 4% not met, but every head meets it"
    run.err_exact = errs_ex
    run.err_oracle_exact = errs_or_ex
    run.target_misses = misses
    return run


def _cfg(cid, device="cuda", **kw):
    w = synth.workload(cid, **kw)
    q, k, v = synth.generate(w, device)
    return w, q, k, v


def test_config1_tiny():
    w, q, k, v = _cfg(1)
    check_against_oracle(q, k, v, kc=w.k, iters=w.iters, name="config1")


def test_config2_small_multihead():
    w, q, k, v = _cfg(2)
    check_against_oracle(q, k, v, kc=w.k, iters=w.iters, name="config2")


@pytest.mark.parametrize("S", [1, 5, 127, 129, 300, 1000])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_ragged_shapes(S, dtype):
    g = torch.Generator().manual_seed(100 + S)
    B, H = 2, 3
    q = torch.randn(B, S, H, 128, generator=g).to(dtype).cuda()
    k = (1.5 * torch.randn(B, S, H, 128, generator=g)).to(dtype).cuda()
    v = (torch.randn(B, S, H, 128, generator=g) + 3 * torch.randn(B, 1, H, 128, generator=g)).to(dtype).cuda()
    check_against_oracle(q, k, v, kc=min(5, S), iters=3, name=f"ragged S={S} {dtype}")


@pytest.mark.parametrize("kc,iters,seed", [(33, 2, 0), (48, 0, 2**64 - 1), (64, 3, 12345), (1, 2, 0)],
                         ids=["k33", "k48_T0_seed_max", "k64_seed", "k1"])
def test_kmeans_options(kc, iters, seed):
    # cluster counts that need 3 and 4 tiles of 16 centroids in the assignment
    # pass, the largest k, no Lloyd iteration at all (initial centroids, then
    # the final assignment), one cluster, and seeds other than 0 (the initial
    # centroids' offset), on two batches of two heads
    w, q, k, v = _cfg(2, B=2, H=2, S=1000)
    check_against_oracle(q, k, v, kc=kc, iters=iters, seed=seed, name=f"k={kc} T={iters} seed={seed}")


@pytest.mark.parametrize("B,H,S", [(1, 65535, 130), (16, 65535, 1)], ids=["H65535_S130", "BH_max_S1"])
def test_largest_head_count(B, H, S):
    """The most heads one launch takes: H = 65535 (the grid's second
    dimension) with B = 1 and S = 130 (a full tile and a ragged one of 2
    keys); and B = 16 (the third dimension) for B*H = 1048560, next to the
    2^20 limit, at the degenerate length S = 1 (one key per head).  Inputs
    are drawn on the GPU from a seeded generator; five heads (both ends,
    the middle, the neighbours of the ends) are checked against the oracle
    in full, and the output, filled with NaN before the call, must come out
    finite everywhere: every head's every row is written."""
    g = torch.Generator(device="cuda").manual_seed(65535 + B)
    q, k, v = (torch.randn((B, S, H, 128), generator=g, device="cuda").to(torch.bfloat16) for _ in range(3))
    out = torch.full((B, S, H, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    heads = [(0, 0), (0, 1), (B // 2, H // 2), (B - 1, H - 2), (B - 1, H - 1)]
    check_against_oracle(q, k, v, kc=min(4, S), iters=2, seed=3, heads=heads, name=f"heads B={B} H={H} S={S}",
                         out=out)
    assert bool(torch.isfinite(out).all()), "output rows left unwritten"
    del q, k, v, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("S", [8422400, 1 << 24], ids=["S8422400", "S_max_2^24"])
def test_kmeans_sums_past_int32(S):
    """k-means at a length where a cluster's sketch sum passes 2^31.

    S tokens (8422400, and the largest supported length 2^24) with channel
    0 = 1.9921875 (sketch +255) except a run of 200 tokens at -1.9921875
    (sketch -255) around cluster 1's initial position; every other channel
    is 0.  With k=2 and one iteration the centroids must come out
    (255, 0, ...) and (-255, 0, ...): cluster 0's sum is 255 * (S - 200) >
    2^31 - 1, so a 32-bit accumulation would wrap and pull both centroids
    to -255.  The answer is known by construction: A tokens in cluster 0,
    the run in cluster 1, the permutation A then the run, each ascending."""
    seed = 5
    init = O.init_positions(S, 2, seed, 0)
    lo, hi = max(S // 2, int(init[1]) - 100), min(S, max(S // 2, int(init[1]) - 100) + 200)
    assert int(init[0]) < S // 2 and lo <= int(init[1]) < hi and hi - lo == 200
    assert 255 * (S - 200) > 2 ** 31 - 1
    say(f"k-means sums past int32: S={S} run [{lo}, {hi})")
    v = torch.zeros((1, S, 1, 128), dtype=torch.bfloat16, device="cuda")
    v[0, :, 0, 0] = 1.9921875
    v[0, lo:hi, 0, 0] = -1.9921875
    opts = vc.v_opts(True, 2, 1, seed, 0.0)
    lay = vc.vc_workspace_layout(v, opts)
    ws = torch.zeros((lay.total,), dtype=torch.uint8, device="cuda")
    vc.vc_prepare_v(v, opts, ws)
    torch.cuda.synchronize()
    assign = ws[lay.assign:lay.assign + 4 * S].view(torch.int32).cpu().numpy()
    perm = ws[lay.perm:lay.perm + 4 * S].view(torch.int32).cpu().numpy()
    want = np.zeros(S, np.int32)
    want[lo:hi] = 1
    assert np.array_equal(assign, want), f"{int((assign != want).sum())} tokens in the wrong cluster"
    want_perm = np.concatenate([np.arange(0, lo), np.arange(hi, S), np.arange(lo, hi)]).astype(np.int32)
    assert np.array_equal(perm, want_perm)
    del v, ws
    torch.cuda.empty_cache()


def test_sketch_rounding_extremes():
    """The two edges of the k-means sketch x = clamp(rne(v * 2^shift), +-255).

    fp16 V clipped at +-(1 - 2^-11): shift = 8, and the top fp16 values
    1 - j * 2^-11 (j = 1..4) scale to 255.5 .. 255.875, which round to 256
    and must clamp to 255 (j = 4 is a tie, to even).  Compared in full."""
    g = torch.Generator().manual_seed(41)
    S, H = 700, 2
    q = torch.randn(1, S, H, 128, generator=g).to(torch.float16)
    k = torch.randn(1, S, H, 128, generator=g).to(torch.float16)
    top = 1.0 - 2.0 ** -11
    v = (torch.randn(1, S, H, 128, generator=g) * 0.6).clamp(-top, top).to(torch.float16)
    vs = v.float() * 256
    assert int(((vs.abs() >= 255.5) & (vs.abs() < 256)).sum()) > 1000
    check_against_oracle(q.cuda(), k.cuda(), v.cuda(), kc=8, iters=3, name="sketch clamp (fp16)")


def test_sketch_tiny_bf16_head():
    """A bf16 head with max|v| < 2^-120 (shift > 127, so 2^shift is no fp32
    value): the sketch takes its two-step scaling.  Assignments and the
    permutation are bit-exact against the oracle.  The rest of such a head
    is not compared: its residual scale 448 / max|v| overflows fp32 on both
    sides."""
    g = torch.Generator().manual_seed(43)
    S = 900
    v = (torch.randn(1, S, 1, 128, generator=g, dtype=torch.float64) * 2.0 ** -124).to(torch.bfloat16)
    a = float(v.double().abs().max())
    assert 0 < a < 2.0 ** -120 and 7 - int(np.floor(np.log2(a))) > 127
    kc, iters, seed = 12, 3, 4
    opts = vc.v_opts(True, kc, iters, seed, 0.0)
    lay = vc.vc_workspace_layout(v, opts)
    ws = torch.zeros((lay.total,), dtype=torch.uint8, device="cuda")
    vc.vc_prepare_v(v.cuda(), opts, ws)
    torch.cuda.synchronize()
    with np.errstate(over="ignore", invalid="ignore"):
        hv = O.prepare_v_head(_np(v[0, :, 0]), smooth=True, k=kc, iters=iters, seed=seed, bh=0)
    assign = ws[lay.assign:lay.assign + 4 * S].view(torch.int32).cpu().numpy()
    perm = ws[lay.perm:lay.perm + 4 * S].view(torch.int32).cpu().numpy()
    assert len(np.unique(hv.assign)) > 1
    assert np.array_equal(assign, hv.assign)
    assert np.array_equal(perm, hv.perm)


@pytest.mark.parametrize("smooth", [0, 1])
def test_plain_and_smooth_on_outliers(smooth):
    w, q, k, v = _cfg(2, H=2, S=2048)
    check_against_oracle(q, k, v, smooth=bool(smooth), kc=16, iters=4, name=f"smooth={smooth}")


@pytest.mark.parametrize("beta", [0.005, 0.05])
def test_repair(beta):
    w, q, k, v = _cfg(5, B=2, H=2, S=2048)
    run = check_against_oracle(q, k, v, kc=8, iters=3, beta=beta, name=f"repair beta={beta}")
    base = check_against_oracle(q, k, v, kc=8, iters=3, beta=0.0, name="repair baseline beta=0")
    # re-adding the worst-rounded tokens' residual lowers the error vs exact attention
    assert np.mean(run.err_exact) < np.mean(base.err_exact)


@pytest.mark.parametrize("S,beta,dups", [(9000, 0.3, True), (9000, 1e-4, False), (300, 0.9, True)],
                         ids=["S9000_beta0.3_ties", "S9000_one_token", "S300_beta0.9_ties"])
def test_repair_select_edges(S, beta, dups):
    # the top-k select over a key count that leaves its 8 x 1024-key chunks
    # ragged, a repair set of one token, a budget of 90%, and many equal error
    # norms: with every token a copy of one of 50 rows, copies in one block
    # have the same error, so the set among ties goes by position
    g = torch.Generator().manual_seed(31 + S)
    B, H = 1, 2
    q = torch.randn(B, S, H, 128, generator=g).to(torch.bfloat16)
    k = torch.randn(B, S, H, 128, generator=g).to(torch.bfloat16)
    v = torch.randn(B, S, H, 128, generator=g)
    if dups:
        v = v[:, torch.randint(0, 50, (S,), generator=g)]
    v = v.to(torch.bfloat16)
    check_against_oracle(q.cuda(), k.cuda(), v.cuda(), kc=4, iters=2, beta=beta, name=f"repair edges S={S} beta={beta}",
                         rows=np.arange(0, S, max(1, S // 64)))


def test_strided_views_and_3d_input():
    g = torch.Generator().manual_seed(5)
    S, H = 700, 2
    big = torch.randn(S, H, 3, 128, generator=g).to(torch.bfloat16).cuda()   # packed qkv
    q, k, v = big[:, :, 0], big[:, :, 1], big[:, :, 2]                        # [S,H,128] strided views
    assert not q.is_contiguous()
    run = check_against_oracle(q, k, v, kc=4, iters=2, name="strided 3d")
    # output into a strided buffer gives the same bytes
    out2 = torch.zeros(S, H, 2, 128, dtype=torch.bfloat16, device="cuda")[:, :, 1]
    opts = vc.v_opts(True, 4, 2)
    vc.vc_attention_fwd(out2, opts, run.ws)
    torch.cuda.synchronize()
    assert torch.equal(out2, run.out)


def test_sm_scale_option():
    w, q, k, v = _cfg(1)
    check_against_oracle(q, k, v, kc=2, iters=3, sm_scale=0.05, name="sm_scale=0.05")


def test_deterministic_and_reusable_workspace():
    w, q, k, v = _cfg(2, H=3, S=1500)
    opts = vc.v_opts(True, 8, 3)
    a = GpuRun(q, k, v, opts)
    b = GpuRun(q, k, v, opts)
    assert torch.equal(a.out, b.out)
    used = [("assign", a.lay.perm - a.lay.assign), ("q8", a.lay.v_mean - a.lay.q8)]
    for name, n in used:
        off = getattr(a.lay, name)
        assert torch.equal(a.ws[off:off + n], b.ws[off:off + n]), name
    # the forward alone can be re-run on a prepared workspace
    out2 = torch.empty_like(a.out)
    vc.vc_attention_fwd(out2, opts, a.ws)
    torch.cuda.synchronize()
    assert torch.equal(out2, a.out)


def test_zero_value_head_and_zero_blocks():
    S, H = 400, 2
    g = torch.Generator().manual_seed(9)
    q = torch.randn(1, S, H, 128, generator=g).to(torch.bfloat16)
    k = torch.randn(1, S, H, 128, generator=g).to(torch.bfloat16)
    v = torch.randn(1, S, H, 128, generator=g).to(torch.bfloat16)
    v[:, :, 0] = 0                      # all-zero V head
    q[:, 128:256] = 0                   # all-zero Q block
    k[:, 0:128, 1] = 0                  # zero K rows (join whichever permuted block they land in)
    check_against_oracle(q.cuda(), k.cuda(), v.cuda(), kc=3, iters=2, name="zero head/blocks")


@pytest.mark.parametrize("v_format", ["e4m3", "mxfp4"])
@pytest.mark.parametrize("smooth", [False, True])
def test_steep_maximum_rises(v_format, smooth):
    """Spike keys along one direction c: even queries (+4c) see their running
    maximum rise by ~30, ~100 and ~104 octaves at three tiles (the last one
    ragged), odd queries (-4c) see the spikes far below their maximum.  So
    within one wave some lanes rescale and others do not; the 100-octave rise
    moves the MXFP4 anchor (rises past 64 octaves) and takes the E4M3 rescale
    to 2^-100.  With smooth=False the key order is the original one, so the
    rises land at the tiles chosen here."""
    S, H = 1000, 2
    g = torch.Generator().manual_seed(77)
    c = torch.randn(128, generator=g)
    c = c / c.norm()
    sign = torch.where(torch.arange(S) % 2 == 0, 1.0, -1.0)
    q = torch.randn(1, S, H, 128, generator=g) + 4.0 * sign[None, :, None, None] * c
    k = torch.randn(1, S, H, 128, generator=g)
    v = torch.randn(1, S, H, 128, generator=g) + 2 * torch.randn(1, 1, H, 128, generator=g)
    octave = 4.0 * float(O.DEFAULT_SM_SCALE) * float(np.log2(np.e))     # log2 units per unit of lam
    for pos, octaves in ((130, 30.0), (400, 100.0), (990, 104.0)):
        k[0, pos] = (octaves / octave) * c
    # The even rows' attention collapses onto the two last spikes (weights
    # 16:1), so their output is essentially one token's V and carries that
    # token's full quantisation error, with no averaging: up to ~9% for the
    # 4-bit residual.  The oracle parity (5e-3) is the gate here; the exact
    # envelope only catches gross errors.
    check_against_oracle(q.to(torch.bfloat16).cuda(), k.to(torch.bfloat16).cuda(), v.to(torch.bfloat16).cuda(),
                         smooth=smooth, kc=4, iters=2, name=f"steep rises {v_format} smooth={smooth}", v_format=v_format)


# ---- 4-bit residual (MXFP4) ---------------------------------------------------
# The 4-bit residual is coarser than E4M3 (the oracle itself sits up to ~4% from
# exact attention on config 2), so its runs get the gross-error envelope.
def test_mxfp4_config2():
    w, q, k, v = _cfg(2)
    check_against_oracle(q, k, v, kc=w.k, iters=w.iters, name="config2 mxfp4", v_format="mxfp4")


@pytest.mark.parametrize("S", [1, 129, 1000])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_mxfp4_ragged(S, dtype):
    g = torch.Generator().manual_seed(200 + S)
    B, H = 2, 3
    q = torch.randn(B, S, H, 128, generator=g).to(dtype).cuda()
    k = (1.5 * torch.randn(B, S, H, 128, generator=g)).to(dtype).cuda()
    v = (torch.randn(B, S, H, 128, generator=g) + 3 * torch.randn(B, 1, H, 128, generator=g)).to(dtype).cuda()
    check_against_oracle(q, k, v, kc=min(5, S), iters=3, name=f"mxfp4 ragged S={S} {dtype}", v_format="mxfp4")


def test_mxfp4_smooth_off_and_zero_head():
    w, q, k, v = _cfg(2, H=2, S=700)
    v[:, :, 1] = 0                      # an all-zero head: scales 2^0, codes 0
    check_against_oracle(q, k, v, smooth=False, kc=4, iters=2, name="mxfp4 smooth=0", v_format="mxfp4")


def test_mxfp4_rejects_repair():
    w, q, k, v = _cfg(1)
    opts = vc.v_opts(True, 2, 1, 0, 0.01, vc.VC_V_MXFP4)
    with pytest.raises(vc.VCError) as e:
        vc.alloc_workspace(v, opts)
    assert e.value.status == vc.VC_ERR_UNSUPPORTED


# ---- work items cut along the key axis (the partial last round of
# workgroups, and launches with fewer items than compute units): pieces of
# 16-tile groups whose partial results a merge kernel combines -------------
SPLIT_CASES = [
    # (B, H, S, v_format, heads checked): what the cut does there
    (1, 3, 4500, "e4m3", None),                     # 54 items cut into three 1-group pieces, the last ragged
    (1, 6, 8492, "e4m3", None),                     # 204 items of 5 groups, runs of 4 crossing item boundaries
    (1, 20, 4196, "e4m3", [(0, 0), (0, 15), (0, 19)]),  # 256 items whole, then 84 cut (heads 15-19)
    (1, 6, 8492, "mxfp4", None),                    # the 4-bit residual's anchor exponent in the partials
]


@pytest.mark.parametrize("B,H,S,v_format,heads", SPLIT_CASES,
                         ids=["S4500_three_pieces", "S8492_runs_cross_items", "H20_whole_then_cut",
                              "S8492_mxfp4"])
def test_key_axis_split(B, H, S, v_format, heads):
    from test_split_plan import plan
    p = plan(B * H, -(-S // 128))
    assert p is not None and not p.get("halves"), "the shape must be cut"
    w, q, k, v = _cfg(2, B=B, H=H, S=S)
    rows = np.unique(np.concatenate([np.arange(0, S, 3), np.arange(max(0, S - 130), S)]))
    run = check_against_oracle(q, k, v, kc=8, iters=2, rows=rows, heads=heads,
                               name=f"split B={B} H={H} S={S} {v_format}", v_format=v_format)
    # repeated calls on one prepared workspace rewrite the partial slots and
    # merge them in the same order: the same bytes every time
    for rep in range(3):
        again = torch.empty_like(run.out)
        vc.vc_attention_fwd(again, run.opts, run.ws)
        torch.cuda.synchronize()
        assert torch.equal(again, run.out), f"call {rep + 2} differs from the first"


HALVES_CASES = [
    # (B, H, S, v_format): the short-launch form, one workgroup per query block, keys in two halves
    (2, 4, 4096, "e4m3"),      # config 2's class: two halves of 16 tiles
    (1, 8, 4046, "e4m3"),      # the second half's last tile ragged (78 keys)
    (1, 14, 2049, "e4m3"),     # second half one tile with one key: 15 masked steps after it
    (1, 6, 3000, "e4m3"),      # halves of 16 and 8 tiles, the second ragged: 8 masked steps
    (1, 6, 3000, "mxfp4"),     # the 4-bit residual's anchor exponents meet in the merge
    (1, 8, 4096, "mxfp4"),     # config 2 with the 4-bit residual
]


@pytest.mark.parametrize("B,H,S,v_format", HALVES_CASES,
                         ids=["B2_S4096", "S4046_ragged", "S2049_one_key_half", "S3000_unequal",
                              "S3000_mxfp4", "S4096_mxfp4"])
def test_short_launch_halves(B, H, S, v_format):
    from test_split_plan import plan
    p = plan(B * H, -(-S // 128))
    assert p is not None and p.get("halves"), "the shape must take the short-launch form"
    w, q, k, v = _cfg(2, B=B, H=H, S=S)
    run = check_against_oracle(q, k, v, kc=8, iters=2, name=f"halves B={B} H={H} S={S} {v_format}",
                               v_format=v_format)
    assert not run.target_misses or v_format == "mxfp4"
    for rep in range(3):
        again = torch.empty_like(run.out)
        vc.vc_attention_fwd(again, run.opts, run.ws)
        torch.cuda.synchronize()
        assert torch.equal(again, run.out), f"call {rep + 2} differs from the first"
