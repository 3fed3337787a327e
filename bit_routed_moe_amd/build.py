"""Build libds4moe.so (HIP, gfx950) in-tree.

Each translation unit under csrc/ is compiled by hipcc for gfx950 and linked
into ``bit_routed_moe_amd/libds4moe.so``.  Packed-fp32 VALU instructions are
disabled (-packed-fp32-ops) for every device compilation.

The native benchmark driver native/ds4moe_bench.hip is built next to it as
``bit_routed_moe_amd/ds4moe_bench``.

The library is linked against the HIP runtime that PyTorch loads (its own
``libamdhip64.so``), so that torch's device pointers and streams and the
library's launches live in one runtime.  Without torch it links the ROCm
install's runtime instead.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libds4moe.so")
NATIVE_SRC = os.path.join(HERE, "native", "ds4moe_bench.hip")
NATIVE_BIN = os.path.join(HERE, "ds4moe_bench")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-mcode-object-version=5",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC, "-Wno-unused-result",
]


def hip_runtime_dir():
    """Directory of the HIP runtime to link: torch's bundled one if present."""
    import importlib.util
    spec = importlib.util.find_spec("torch")
    if spec and spec.origin:
        d = os.path.join(os.path.dirname(spec.origin), "lib")
        if os.path.exists(os.path.join(d, "libamdhip64.so")):
            return d
    return "/opt/rocm/lib"


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src):
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose=False):
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4)), 16)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    rt = hip_runtime_dir()
    cxx = shutil.which("g++") or "c++"
    cmd = [cxx, "-shared", "-fPIC", "-o", tmp, *objs, f"-L{rt}", "-l:libamdhip64.so",
           f"-Wl,-rpath,{rt}", "-Wl,--no-undefined"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    build_native(rt, cxx)
    if verbose:
        print(f"built {LIB} and {NATIVE_BIN}")
    return LIB


def build_native(rt, cxx):
    """The native benchmark driver (for profiler counter runs without Python),
    linked against the library and the same HIP runtime."""
    obj = _compile(NATIVE_SRC)
    tmp = NATIVE_BIN + ".tmp"
    cmd = [cxx, "-o", tmp, obj, f"-L{HERE}", "-l:libds4moe.so", f"-Wl,-rpath,{HERE}", f"-L{rt}",
           "-l:libamdhip64.so", f"-Wl,-rpath,{rt}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link of the native benchmark failed:\n{r.stderr}")
    os.replace(tmp, NATIVE_BIN)


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
