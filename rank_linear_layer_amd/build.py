"""Build the gfx950 HIP library liblr_linear.so in-tree with hipcc.

    python -m rank_linear_layer_amd.build

Every HIP source is compiled with packed-FP32 instructions disabled
(-target-feature -packed-fp32-ops): the compiler would otherwise form
v_pk_* FP32 operations on its own, and no kernel here needs them.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_NAME = "liblr_linear.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = ["lr_linear.cpp", "lr_decode.hip", "lr_decode_res.hip", "lr_prefill.hip", "lr_prefill_w4.hip", "lr_dense.hip",
           "lr_decode_split.hip", "lr_decode_xcd.hip",
           "lr_gac.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def common_flags():
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", "-I", CSRC]


def build(verbose: bool = False, jobs: int = 4) -> str:
    cc = hipcc()
    tmp = tempfile.mkdtemp(prefix="lrl_build_")
    try:
        objs = []
        procs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            cmd = [cc] + common_flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
            if src.endswith(".cpp"):
                cmd = [cc] + common_flags() + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
            objs.append(obj)
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
            if len(procs) >= jobs:
                _wait(procs.pop(0))
        for p in procs:
            _wait(p)
        out_tmp = LIB_PATH + ".tmp%d" % os.getpid()
        cmd = [cc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", out_tmp] + objs
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(out_tmp, LIB_PATH)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB_PATH


def _wait(item):
    src, proc = item
    out, _ = proc.communicate()
    text = out.decode(errors="replace")
    lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln]
    if proc.returncode != 0:
        sys.stderr.write("\n".join(lines) + "\n")
        raise RuntimeError("hipcc failed on %s" % src)
    if lines:
        sys.stderr.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
