"""Build libtq.so (the HIP library behind include/tq.h) in-tree with hipcc for gfx950.

Usage: python -m rotation_lloyd_max_amd.build  (or call build()).
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libtq.so")

SOURCES = ["tq_api.cpp", "rotate.hip", "encode.hip", "encode_p2.hip", "encode_m.hip", "qmv.hip", "qmv_16.hip", "qmv_8.hip",
           "qmv_4.hip", "qmv_3.hip", "rot16.hip", "multi_gather.hip", "gather_qmm.hip",
           "dequant.hip", "slot_ids.hip", "kv_fetch.hip", "dense.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.isabs(cand) and os.path.exists(cand) or not os.path.isabs(cand)):
            return cand
    return "hipcc"


def build(verbose=False, jobs=None):
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    hipcc = _hipcc()
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [hipcc] + HIPCC_FLAGS + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # the host pass does not know the packed-fp32 target feature; that warning is noise
        lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l and l.strip()]
        if p.returncode != 0:
            failed.append(src)
            print("\n".join(lines), file=sys.stderr)
        elif verbose and lines:
            print("\n".join(lines))
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = LIB + ".tmp"
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
