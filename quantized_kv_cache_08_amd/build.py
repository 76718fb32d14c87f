"""Build libkvq.so (the HIP/gfx950 kernels and the C ABI of include/kvq.h)
and libkvq_testing.so (test and measurement hooks of include/kvq_testing.h,
not part of the method).

    python -m quantized_kv_cache_08_amd.build   (or python quantized_kv_cache_08_amd/build.py)

hipcc cross-compiles for gfx950 without a GPU.  Flags:
  -fhip-fp32-correctly-rounded-divide-sqrt   IEEE division in the quantizers
  -Xclang -target-feature -Xclang -packed-fp32-ops   no packed-fp32 instructions
  -mllvm -amdgpu-mfma-vgpr-form=1   MFMA accumulators in VGPRs (no AGPR copies)
"""
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INC = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libkvq.so")
OUT_TESTING = os.path.join(PKG, "libkvq_testing.so")
BUILD = os.path.join(PKG, "_build")
ARCH = os.environ.get("KVQ_OFFLOAD_ARCH", "gfx950")

FLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
         "-fhip-fp32-correctly-rounded-divide-sqrt",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form=1",
         "-Wno-unused-command-line-argument", "-I", INC, "-I", CSRC]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def testing_sources():
    return sorted(glob.glob(os.path.join(CSRC, "testing", "*.hip")))


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = ["hipcc", *FLAGS, "-x", "hip", "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out, verbose):
    tmp = out + ".tmp"
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    tsrcs = testing_sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs) + len(tsrcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs + tsrcs))
    _link(objs[:len(srcs)], OUT, verbose)
    _link(objs[len(srcs):], OUT_TESTING, verbose)
    return OUT


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
