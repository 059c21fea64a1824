"""Build libmq.so (gfx950) in-tree with hipcc.

    python -m weight_activation_quantized_amd._build [-D NAME=VALUE ...] [--out PATH]

Compiles every source under csrc/ with hipcc for gfx950 and links one shared
library next to this file. Always recompiles (a few seconds per file); runs
without a GPU.
"""

import argparse
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libmq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["mq_api.cpp", "quant_int8.hip", "w8a8_gemm.hip", "w8a8_gemv.hip", "w4a16_gemv.hip",
           "w4a16_gemv_blocked.hip", "w4a16_gemv_blocked_prescaled.hip", "w4a16_gemm.hip", "kv_quant.hip",
           "int4_layout.hip", "w8a8_noalloc.hip"]

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # keep the compiler from forming packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]

# Per-source extra flags: MFMA results in ordinary VGPRs. The GEMV starts its
# nine MFMAs of a step from zero every step; the VGPR form gives each its own
# destination (otherwise they share one AGPR quad and wait on each other's
# copy-out). The decode-layout GEMV's one-tile kernel reads its per-group
# sums with VALU operations (no copies out of AGPRs); its kernel for 17-64
# tokens lives in its own file, built without this flag.
SOURCE_FLAGS = {
    "w4a16_gemv.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "w4a16_gemv_blocked.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(out=LIB_PATH, defines=(), build_dir=BUILD_DIR, jobs=None, verbose=False):
    """Compile and link; returns the path of the shared library."""
    os.makedirs(build_dir, exist_ok=True)
    dflags = [f"-D{d}" for d in defines]

    def compile_one(src):
        obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
        _run([HIPCC, *FLAGS, *SOURCE_FLAGS.get(src, []), *dflags, "-c", os.path.join(CSRC, src), "-o", obj])
        return obj

    jobs = jobs or min(len(SOURCES), max(1, (os.cpu_count() or 2) // 2))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = out + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("-D", dest="defines", action="append", default=[])
    ap.add_argument("--out", default=LIB_PATH)
    ap.add_argument("--build-dir", default=BUILD_DIR)
    a = ap.parse_args(argv)
    build(a.out, a.defines, a.build_dir, verbose=True)


if __name__ == "__main__":
    sys.exit(main())
