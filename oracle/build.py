"""Build the CPU oracle (test infrastructure): liboracle.so from kvq_oracle.c.

IEEE fp32 semantics are required for bit-exact codes: no contraction into
fused multiply-add, no fast-math, SSE arithmetic (the x86-64 default).
"""
import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))


def build() -> str:
    src = os.path.join(_HERE, "kvq_oracle.c")
    out = os.path.join(_HERE, "liboracle.so")
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=gnu11", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", "-Wextra", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
