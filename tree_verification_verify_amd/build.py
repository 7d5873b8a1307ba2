"""Build libtreeverify.so for gfx950 with hipcc (in-tree, no JIT cache).

Usage: python -m tree_verification_verify_amd.build [--verbose]
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libtreeverify.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["tree_attn.hip", "tree_sample.hip", "tree_sample_noalloc.hip", "tree_path.hip", "tree_commit.hip", "tree_siblings.hip",
           "tree_construct.hip", "tree_spark.hip", "api.cpp"]
ARCH = "gfx950"
# Per-source extra flags. The attention kernels are scheduled for ILP (LDS
# operand loads batched ahead of their MFMAs); their occupancy is fixed by
# LDS, not registers.
EXTRA_FLAGS = {"tree_attn.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]}


def hipcc():
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"),
              shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libtreeverify)")


def common_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # keep the compiler from forming packed fp32 ops (v_pk_*_f32)
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function",
    ]


def build(verbose=False):
    cc = hipcc()
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        cmd = [cc] + common_flags() + EXTRA_FLAGS.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
        if verbose and res.stderr.strip():
            print(res.stderr, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
