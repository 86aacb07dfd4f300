"""Build libpkvspec.so for gfx950 with hipcc, in-tree.

    python paged_kv_speculative_amd/csrc/build.py [--jobs N]

Every source is compiled on each call (the "does it build" check); objects go
to paged_kv_speculative_amd/csrc/_build/ and the library to
paged_kv_speculative_amd/libpkvspec.so.
"""
import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
OUT = os.path.join(PKG, "libpkvspec.so")
BUILD = os.path.join(HERE, "_build")
SOURCES = ["pool.cpp", "kernels/kv_append.hip", "kernels/verify_attn.hip", "kernels/accept.hip",
           "kernels/tree_accept.hip", "kernels/read_probe.hip"]
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         # packed fp32 VALU ops are kept out of generated code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-Wno-unused-variable"]
# Per-source additions.  The verification kernels keep their MFMA accumulators
# in architectural VGPRs: left to its heuristics the compiler runs the MFMAs on
# AGPRs and copies all O^T accumulators to VGPRs and back around every page
# (about 130 extra VALU moves per page for 20 rows x head_dim 128).
EXTRA = {"kernels/verify_attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm 7 with gfx950 support is required)")


def _compile(src):
    path = os.path.join(HERE, src)
    obj = os.path.join(BUILD, src.replace("/", "_") + ".o")
    flags = FLAGS + EXTRA.get(src, [])
    cmd = [hipcc()] + flags + ["-c", path, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [hipcc(), "-x", "hip"] + flags + ["-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    return obj, err


def build(jobs=None, verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4)
    with cf.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_compile, SOURCES))
    objs = [o for o, _ in results]
    if verbose:
        for _, err in results:
            if err.strip():
                print(err, file=sys.stderr)
    tmp = OUT + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args()
    print(build(a.jobs, a.verbose))
