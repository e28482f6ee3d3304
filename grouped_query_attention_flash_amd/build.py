"""Build libgqa_attn.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m grouped_query_attention_flash_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgqa_attn.so")
SOURCES = ["api.hip", "attn_fwd.hip", "attn_bwd.hip"]
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU ops.
HIPFLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def build(verbose: bool = False) -> str:
    # the runtime tuning table, generated from tuning/mi355x.json
    from grouped_query_attention_flash_amd.tuning import gen_table
    gen_table.generate()
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objs = []
    procs = []
    for src in SOURCES:
        obj = os.path.join(CSRC, src.replace(".hip", ".o"))
        cmd = [hipcc, *HIPFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        objs.append(obj)
    failed = False
    for cmd, p in procs:
        out, _ = p.communicate()
        # hipcc's host pass does not know the packed-fp32 feature; that warning is harmless
        lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
        if lines:
            print("\n".join(lines), file=sys.stderr)
        if p.returncode != 0:
            failed = True
            print("FAILED: " + " ".join(cmd), file=sys.stderr)
    if failed:
        raise RuntimeError("HIP build failed")
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc, "-shared", "-fPIC", "--offload-arch=" + ARCH, *objs, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
