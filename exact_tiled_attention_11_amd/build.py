"""Build libfa355.so for gfx950 with hipcc, in the package directory.

Run as ``python -m exact_tiled_attention_11_amd.build``.  Objects go to
``_build/`` at the repository root; the shared library lands next to this
file so that the Python binding (and the tests) load it from the tree.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfa355.so")
SOURCES = ["api.cpp", "fwd.hip", "decode.hip", "bwd.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++20",
    "-fPIC",
    "-fvisibility=hidden",
    # packed-FP32 VALU forms stay off in all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + INCLUDE,
    "-I" + CSRC,
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("command failed: %s\n%s" % (" ".join(cmd), out))
    return out


def build(verbose: bool = False, defines=(), out: str = LIB) -> str:
    """Compile every source and link ``out``; ``defines`` are extra -D flags
    (tile-shape overrides for tuning builds)."""
    bdir = os.path.join(BUILD, os.path.basename(out) + ".objs")
    os.makedirs(bdir, exist_ok=True)
    objs = []
    cmds = []
    extra = ["-D" + d for d in defines]
    for src in SOURCES:
        obj = os.path.join(bdir, src + ".o")
        objs.append(obj)
        cmds.append([HIPCC] + FLAGS + extra + ["-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        outs = list(ex.map(_run, cmds))
    tmp = out + ".tmp"
    outs.append(_run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs))
    os.replace(tmp, out)
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    return out


# Host-side AddressSanitizer build of the C ABI layer (argument validation,
# dispatch), CPU only: api.cpp is compiled by g++ with the sanitizer and linked
# with the device objects of the normal build, which stay uninstrumented.  Load
# it with the sanitizer runtime preloaded (see asan_runtime()).
ASAN_DIR = os.path.join(BUILD, "asan")
ASAN_LIB = os.path.join(ASAN_DIR, "libfa355_asan.so")
HOST_ASAN = ["-fsanitize=address", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    """Path of g++'s AddressSanitizer runtime (for LD_PRELOAD)."""
    return _run(["g++", "-print-file-name=libasan.so"]).strip()


def build_asan() -> str:
    objs = [os.path.join(BUILD, "libfa355.so.objs", s + ".o") for s in SOURCES if s != "api.cpp"]
    if not all(os.path.exists(o) for o in objs):
        build()
    os.makedirs(ASAN_DIR, exist_ok=True)
    api = os.path.join(ASAN_DIR, "api.o")
    _run(["g++", "-std=c++17", "-O1", "-g", "-fPIC"] + HOST_ASAN +
         ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + INCLUDE, "-I" + CSRC,
          "-c", os.path.join(CSRC, "api.cpp"), "-o", api])
    _run(["g++", "-shared", "-o", ASAN_LIB, api] + objs +
         ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    return ASAN_LIB


if __name__ == "__main__":
    if "--asan" in sys.argv:
        print(build_asan())
    else:
        print(build(verbose="-v" in sys.argv))
