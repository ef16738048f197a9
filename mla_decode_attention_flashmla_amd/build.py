"""Ahead-of-time build of libmla_decode.so for gfx950 (hipcc, no JIT cache).

Run ``python -m mla_decode_attention_flashmla_amd.build`` (or __graft_entry__.build()).
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmla_decode.so")
SOURCES = ["mla_abi.hip", "mla_sched.hip", "mla_main_bf16.hip", "mla_main_f32.hip",
           "mla_combine.hip", "mla_sparse.hip", "mla_append.hip"]
ARCH = "gfx950"
# read-bandwidth probes for the roofline measurement (bench.py --hbm-ceiling), a library of
# their own: nothing on the decode path links them
PROBE_SOURCES = ["hbm_probe.hip"]
PROBE_LIB = os.path.join(PKG, "libmla_probe.so")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    return "hipcc"


# Per-file extra flags.  The bf16 main kernel owns all AGPRs through inline asm (the O
# accumulator), so the compiler must never park spilled VGPRs there.
EXTRA = {"mla_main_bf16.hip": ["-mllvm", "-amdgpu-spill-vgpr-to-agpr=0"]}


def compile_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # packed fp32 VALU forms are kept out of generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    ]


def build(verbose: bool = False) -> str:
    """Compile every HIP source (in parallel) and link libmla_decode.so in the package
    directory."""
    from concurrent.futures import ThreadPoolExecutor

    build_dir = os.path.join(ROOT, "_build")
    os.makedirs(build_dir, exist_ok=True)
    cmds, objs = [], []
    for src in SOURCES + PROBE_SOURCES:
        obj = os.path.join(build_dir, src.replace(".hip", ".o"))
        cmds.append([hipcc(), *compile_flags(), *EXTRA.get(src, []), "-c",
                     os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)

    def compile_one(cmd):
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True, stdout=subprocess.PIPE, stderr=subprocess.PIPE)

    workers = max(1, min(len(cmds), os.cpu_count() or 1, 8))
    with ThreadPoolExecutor(workers) as pool:
        for f in [pool.submit(compile_one, c) for c in cmds]:
            f.result()
    nmain = len(SOURCES)
    for lib, lib_objs in ((LIB, objs[:nmain]), (PROBE_LIB, objs[nmain:])):
        tmp = lib + ".tmp"
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *lib_objs, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True, stdout=subprocess.PIPE, stderr=subprocess.PIPE)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    try:
        print(build(verbose="-v" in sys.argv))
    except subprocess.CalledProcessError as e:
        sys.stderr.write(e.stderr.decode(errors="replace"))
        raise SystemExit(1)
