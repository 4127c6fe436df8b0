"""Build the CPU oracle's shared library with gcc.

Test infrastructure only (see oracle/mx_oracle.c)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mx_oracle.c")
LIB = os.path.join(HERE, "libmxoracle.so")


def build_oracle(force: bool = True) -> str:
    """Compile oracle/mx_oracle.c into oracle/libmxoracle.so and return its path."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp"
    # -ffp-contract=off: no fused multiply-add may change a rounding; -O2 only.
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_oracle())
