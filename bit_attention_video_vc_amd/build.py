"""Build libvc.so (HIP, gfx950) in-tree with hipcc.

    python -m bit_attention_video_vc_amd.build

The library is written next to this file so that it travels with the source
tree; nothing is installed.  A second library, libvc_ablation_exp.so, is
built from the same sources with VC_ABLATION_EXP_CAST: the attention kernel
with an FP32 exponential and an E4M3 cast in place of ExpCast, for measuring
what ExpCast saves (it is not the method; the benchmark times it beside
libvc.so on request).
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libvc.so")
ABLATION_EXP_LIB = os.path.join(HERE, "libvc_ablation_exp.so")

HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # fp32 arithmetic exactly as written: no fused multiply-add contraction
    # (explicit fmaf calls still fuse); quantisation codes depend on it.
    "-ffp-contract=off",
    # packed-FP32 VALU instructions are not generated
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


# Extra flags per source.  The attention kernel is NaN-free by construction
# (finite inputs, no infinities used as sentinels), so fmaxf needs no
# IEEE-mode canonicalisation of MFMA results.
PER_FILE_FLAGS = {"vc_attn.hip": ["-fno-honor-nans"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _build_lib(out: str, defines: list[str], tag: str, verbose: bool) -> str:
    srcs = sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    compile_flags = [f for f in HIP_FLAGS if f != "-shared"]
    objs = []
    for src in srcs:
        obj = os.path.join(objdir, os.path.basename(src) + tag + ".o")
        cmd = [hipcc(), *compile_flags, *PER_FILE_FLAGS.get(os.path.basename(src), []), *defines, *inc, "-c", src,
               "-o", obj]
        _run(cmd, verbose)
        objs.append(obj)
    tmp = out + ".tmp"
    _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Build libvc.so; returns its path."""
    return _build_lib(LIB, [], "", verbose)


def build_ablation_exp(verbose: bool = False) -> str:
    """Build libvc_ablation_exp.so (FP32 exp + E4M3 cast instead of ExpCast)."""
    return _build_lib(ABLATION_EXP_LIB, ["-DVC_ABLATION_EXP_CAST"], ".ablation_exp", verbose)


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd))
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libvc.so")


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_ablation_exp(verbose=True))
