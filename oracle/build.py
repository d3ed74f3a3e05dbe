"""Build the fp64 CPU oracles (``oracle/libxattn_ref.so`` for attention,
``oracle/libxattn_ref_norm.so`` for the QK-norm + RoPE step,
``oracle/libxattn_ref_decode.so`` for decode attention) with gcc.

Test infrastructure: the oracle is built alongside the HIP library so that the
checker exists wherever the product is built, but nothing on the product path
loads it.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ref_attn.c")
LIB = os.path.join(HERE, "libxattn_ref.so")
SRC_NORM = os.path.join(HERE, "ref_qknorm_rope.c")
LIB_NORM = os.path.join(HERE, "libxattn_ref_norm.so")
SRC_DEC = os.path.join(HERE, "ref_decode.c")
LIB_DEC = os.path.join(HERE, "libxattn_ref_decode.so")

# Strict IEEE double: no fast-math, no FMA contraction, so the oracle's rounding
# is the plain C evaluation order written in the source.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]


def build(src=SRC, out=LIB, extra=()):
    """Compile ``src`` into the shared library ``out``; returns ``out``."""
    cmd = ["gcc", *CFLAGS, *extra, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def build_all():
    """Every oracle library; returns their paths."""
    return build(), build(SRC_NORM, LIB_NORM), build(SRC_DEC, LIB_DEC)


if __name__ == "__main__":
    print(build_all())
