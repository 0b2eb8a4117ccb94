"""Build libmoe_ffn.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Every HIP translation unit is compiled with
``-Xclang -target-feature -Xclang -packed-fp32-ops`` so that the compiler
emits no packed FP32 arithmetic (hipcc's host pass warns that it does not
know the feature; the warning is harmless).
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe_ffn.so")
# the debug build: the same sources with the kernels' device bounds checks
DEBUG_BUILD_DIR = os.path.join(HERE, "_build_debug")
DEBUG_LIB = os.path.join(HERE, "libmoe_ffn_debug.so")
SOURCES = ["route_permute.hip", "expert_gemm.hip", "expert_tile.hip", "combine.hip",
           "attn_decode.hip", "read_probe.hip", "moe_ffn_api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmoe_ffn.so)")


def compile_flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(src: str, verbose: bool, debug: bool = False) -> str:
    obj = os.path.join(DEBUG_BUILD_DIR if debug else BUILD_DIR, os.path.splitext(src)[0] + ".o")
    extra = ["-DMOE_FFN_DEVICE_CHECKS"] if debug else []
    cmd = [hipcc(), *compile_flags(), *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = [ln for ln in r.stderr.splitlines()
            if "packed-fp32-ops" not in ln and ln.strip()]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(errs))
    if verbose and errs:
        print("\n".join(errs), flush=True)
    return obj


def build(verbose: bool = False, debug: bool = False) -> str:
    """Compile all sources and link libmoe_ffn.so, or with debug=True the
    debug build libmoe_ffn_debug.so (always recompiles)."""
    out = DEBUG_LIB if debug else LIB
    os.makedirs(DEBUG_BUILD_DIR if debug else BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as pool:
        objs = list(pool.map(lambda s: _compile(s, verbose, debug), SOURCES))
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(tmp, out)
    return out


def build_all(verbose: bool = False) -> None:
    """The release and the debug library."""
    build(verbose)
    build(verbose, debug=True)


if __name__ == "__main__":
    print(build(verbose=True))
    print(build(verbose=True, debug=True))
