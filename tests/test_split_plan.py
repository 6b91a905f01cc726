"""Host-side checks of the attention work split (no GPU).

A short launch (at most 256 query blocks, two 16-tile groups per item)
runs instead one workgroup per query block with its keys in two halves
merged inside the workgroup; it needs no partial slots.

A work item is one (b,h) and pair of 128-query blocks.  The first
items - R run whole (R = items mod 256, the partial last round of the 256
compute units); the last R are cut along the key axis into runs of `per`
16-tile groups over tail_wg workgroups, each run holding one or two pieces,
and a merge kernel combines the pieces of every cut item.  Nothing is cut
when there is a repair set, when R is 0, or when cutting saves no group.

These tests restate the documented rule and check (a) that the library's
workspace layout reserves exactly two partial slots per tail workgroup, and
(b) that the run / piece / merge-slot arithmetic the tail and merge kernels
use covers every (item, group) exactly once, never gives a workgroup more
than two pieces, and lets the merge find exactly the slots that were
written -- for every shape tried, before any of it runs on a GPU.
"""
import ctypes
import os

import pytest

import bit_attention_video_vc_amd as vc

SLOTS, GROUP = 256, 16
PART_BYTES = 4 * (256 * 128 + 2 * 256)       # O [256][128], l [256], exponents [256], fp32

pytestmark = pytest.mark.skipif(not os.path.exists(vc.lib_path), reason="libvc.so not built")


def plan(BH, nblk, nrep=0):
    items = BH * ((nblk + 1) // 2)
    ngrp = -(-nblk // GROUP)
    R = items % SLOTS
    if nrep > 0 or R == 0 or ngrp < 2:
        return None
    per = -(-R * ngrp // SLOTS)
    if ngrp == 2 and BH * nblk <= SLOTS:
        # the short-launch form: one workgroup per query block, key halves at 16 tiles
        return dict(halves=True, wg=BH * nblk, ka=GROUP, ngrp=ngrp)
    if per >= ngrp:
        return None
    return dict(items=items, whole=items - R, tail=R, per=per, ngrp=ngrp, tail_wg=-(-R * ngrp // per))


def pieces(p, nblk):
    """The tail kernel's pieces: {workgroup: [(item, kv0, kv1, slot or None)]}."""
    ngrp, per, R = p["ngrp"], p["per"], p["tail"]
    out = {}
    for t in range(p["tail_wg"]):
        g, gend, j = t * per, min(t * per + per, R * ngrp), 0
        while j < 2 and g < gend:
            i = g // ngrp
            g0 = g - i * ngrp
            g1 = min(ngrp, g0 + (gend - g))
            whole = g0 == 0 and g1 == ngrp
            out.setdefault(t, []).append((i, GROUP * g0, min(nblk, GROUP * g1), None if whole else 2 * t + j))
            g += g1 - g0
            j += 1
        assert g == gend, "a run left groups for a third piece"
    return out


def merge_slots(p, i):
    """The merge kernel's slots of cut item i (None: it ran whole in one workgroup)."""
    ngrp, per = p["ngrp"], p["per"]
    wf, wl = (i * ngrp) // per, ((i + 1) * ngrp - 1) // per
    if wf == wl:
        return None
    return {2 * w + (0 if w * per >= i * ngrp else 1) for w in range(wf, wl + 1)}


SHAPES = [(BH, S) for BH in (1, 2, 3, 6, 7, 8, 14, 20, 40, 48, 56, 100, 224) for S in
          (129, 1000, 2049, 4096, 4500, 8492, 20000, 32768, 73397, 75600)]


@pytest.mark.parametrize("BH,S", SHAPES)
def test_runs_cover_every_group_once_and_merge_finds_the_slots(BH, S):
    nblk = -(-S // 128)
    p = plan(BH, nblk)
    if p is None:
        return
    if p.get("halves"):
        # two halves of whole 16-tile groups, the second one non-empty and no
        # longer than the first (which sets the step count), one round
        ka = p["ka"]
        assert ka % GROUP == 0 and 0 < nblk - ka <= ka and p["wg"] <= SLOTS
        return
    cover, written = {}, {}
    for t, ps in pieces(p, nblk).items():
        assert 1 <= len(ps) <= 2
        for (i, kv0, kv1, slot) in ps:
            assert kv0 % GROUP == 0 and 0 <= kv0 < kv1 <= nblk
            for kv in range(kv0, kv1):
                assert (i, kv) not in cover
                cover[(i, kv)] = t
            if slot is not None:
                assert 0 <= slot < 2 * p["tail_wg"]
                written.setdefault(i, set()).add(slot)
    assert len(cover) == p["tail"] * nblk                  # every tile of every cut item, once
    for i in range(p["tail"]):
        assert merge_slots(p, i) == written.get(i)
    # the cut tail takes at most per/ngrp of a whole item's time (< one round)
    assert p["per"] < p["ngrp"] and p["tail_wg"] <= SLOTS


@pytest.mark.parametrize("B,H,S,beta", [(1, 8, 4096, 0.0), (1, 14, 73397, 0.0), (1, 40, 75600, 0.0),
                                        (1, 56, 73397, 0.0), (2, 24, 32768, 0.0), (1, 8, 4096, 0.01),
                                        (1, 1, 256, 0.0), (1, 3, 4500, 0.0)])
def test_layout_reserves_two_partial_slots_per_tail_workgroup(B, H, S, beta):
    d = vc.VcDesc(B, S, H, 128, vc.VC_BF16, 0, S * H * 128, H * 128, 128)
    lay = vc.vc_workspace_layout(d, vc.v_opts(True, 8, 1, 0, beta))
    nrep = lay.nrep
    p = plan(B * H, -(-S // 128), nrep)
    want = 0 if p is None or p.get("halves") else 2 * p["tail_wg"] * PART_BYTES
    assert lay.scratch - lay.attn_part >= want
    assert lay.scratch - lay.attn_part < want + 256            # the region's size, 256-byte aligned
    assert lay.attn_part % 256 == 0
    if beta > 0:
        assert p is None                                        # never cut with a repair set
