"""Host-sanitized build of libmq.so for CPU-side checks (AddressSanitizer + UBSan).

    python -m weight_activation_quantized_amd._build_sanitized [--out PATH]

Compiles every source like ``_build`` (gfx950 device code unchanged) with the
host half instrumented by AddressSanitizer and UndefinedBehaviorSanitizer,
and links ``_build/libmq_hostsan.so``. The library's host code -- argument
validation (overlap, overflow and alignment arithmetic), status strings,
workspace sizing and launch set-up -- then runs under the sanitizers when a
test loads this build (``MQ_LIBRARY``) with the sanitizer runtime preloaded
into an uninstrumented Python (``sanitizer_env``). Device code is never
instrumented; this build is for hosts without a GPU.
"""

import argparse
import glob
import os
import sys
from concurrent.futures import ThreadPoolExecutor

from weight_activation_quantized_amd import _build

OUT = os.path.join(_build.BUILD_DIR, "libmq_hostsan.so")
OBJ_DIR = os.path.join(_build.BUILD_DIR, "hostsan")
# every sanitizer flag applies to the host compilation only
_SAN = ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
        "-fno-omit-frame-pointer", "-g")
HOST_FLAGS = [f for s in _SAN for f in ("-Xarch_host", s)]


def runtime_library():
    """Path of clang's shared ASan runtime (it carries the UBSan handlers too)."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("clang's shared AddressSanitizer runtime was not found under /opt/rocm/llvm")
    return hits[-1]


def sanitizer_env(lib=OUT):
    """Environment for a child Python that loads the sanitized library."""
    env = dict(os.environ)
    env["MQ_LIBRARY"] = lib
    env["LD_PRELOAD"] = runtime_library()
    # the interpreter itself is not instrumented: leaks at exit are its own
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return env


def build(out=OUT, jobs=None, verbose=False):
    os.makedirs(OBJ_DIR, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
        _build._run([_build.HIPCC, *_build.FLAGS, *_build.SOURCE_FLAGS.get(src, []), *HOST_FLAGS, "-c",
                     os.path.join(_build.CSRC, src), "-o", obj])
        return obj

    jobs = jobs or min(len(_build.SOURCES), max(1, (os.cpu_count() or 2) // 2))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, _build.SOURCES))
    tmp = out + ".tmp"
    # a shared library leaves the sanitizer runtime to the process (preloaded)
    _build._run([_build.HIPCC, f"--offload-arch={_build.ARCH}", "-shared", "-fPIC", *HOST_FLAGS,
                 "-shared-libsan", "-o", tmp, *objs])
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=OUT)
    a = ap.parse_args(argv)
    build(a.out, verbose=True)


if __name__ == "__main__":
    sys.exit(main())
