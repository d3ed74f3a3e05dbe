"""Build ``libxattn.so`` (the HIP kernels + C ABI) in-tree for gfx950.

Each source is compiled to an object in parallel, then linked into
``bwd_head_rms_amd/libxattn.so``.  Run ``python -m bwd_head_rms_amd.build``.
"""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libxattn.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
SOURCES = ["attn_fwd.hip", "attn_bwd_dq.hip", "attn_bwd_dkdv.hip", "attn_bwd_short.hip",
           "qknorm_rope.hip", "decode_attn.hip", "composed.hip", "noalloc.hip", "plan.cpp", "api.cpp"]

# Packed-fp32 VALU instructions are switched off for all device code.  MFMA
# accumulators are kept in ordinary VGPRs: the kernels post-process every score
# tile with VALU code, and the AGPR form made the compiler copy each tile
# between the two register files.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-amdgpu-mfma-vgpr-form=1"]
# Any inline-assembly warning (e.g. a statement that clobbers a register the
# compiler reserves) fails the build.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-function", "-Werror=inline-asm"]
# Per-source additions.  The dK/dV kernel is scheduled for instruction-level
# parallelism rather than occupancy (it runs two waves per SIMD either way, at
# 180 + 64 registers instead of 170 + 64): measured 1-3% faster on the
# long-context and grouped-query workloads; the forward and dq kernels were
# slower or unchanged under the same strategy.
SOURCE_FLAGS = {"attn_bwd_dkdv.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]}


def _compile(src):
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"]
    cmd = [HIPCC, *COMMON, *DEVICE_FLAGS, *SOURCE_FLAGS.get(src, []), *lang, "-c",
           os.path.join(CSRC, src), "-o", obj]
    _run(cmd)
    return obj


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature name; that note is harmless
    err = "\n".join(line for line in r.stderr.splitlines() if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{err}")
    if err.strip():
        print(err)


def build(jobs=4):
    """Compile every source and link libxattn.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
