"""Compile oracle/lsh_ref.c into oracle/liblsh_ref.so with gcc (CPU oracle only)."""

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def build() -> str:
    src = os.path.join(HERE, "lsh_ref.c")
    out = os.path.join(HERE, "liblsh_ref.so")
    tmp = out + ".tmp"
    # No fast-math and no contraction: the loop must add in the written order.
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC",
           src, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
