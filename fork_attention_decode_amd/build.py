"""Build libforkattn.so (HIP kernels for gfx950 + C++ host runtime) in-tree with hipcc.

Usage: python fork_attention_decode_amd/build.py  (run by path: importing the package
would load the library being rebuilt).
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libforkattn.so")
SOURCES = ["pool.cpp", "planner.cpp", "drop.cpp", "dagmask.cpp", "decode.hip", "compact.hip", "prefill.hip",
           "prefill_bwd.hip", "select.hip", "noalloc.hip", "probe.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 VALU forms (v_pk_*_f32) are disabled for every device pass: the kernels
# use plain fp32 VALU arithmetic only.
DEVICE_FLAGS = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Per-source device flags.  The prefill and the key-scoring kernels keep their
# matrix-core results in architectural VGPRs (the softmax and the exponential sums read
# them with VALU instructions); without this the allocator parks them in AGPRs and copies
# them back every block.
EXTRA = {"prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"], "select.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include")]


def _compile(src: str, out_dir: str) -> str:
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    cmd = [HIPCC] + COMMON + DEVICE_FLAGS + EXTRA.get(src, []) + ["-c", path, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC] + COMMON + ["-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    out_dir = os.path.join(ROOT, "_build")
    os.makedirs(out_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, out_dir), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC] + DEVICE_FLAGS + ["-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
