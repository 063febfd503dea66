"""Build the fp64 CPU oracle (``oracle/libmsa_oracle.so``) with gcc.

Test infrastructure only: the product library never links or loads it.
No fast-math and no FMA contraction, so every fp64 operation is rounded as
written in ``msa_oracle.c``.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libmsa_oracle.so")


def build(out=LIB, defines=(), quiet=True):
    """Compile msa_oracle.c into a shared library at ``out``.

    ``defines`` are extra ``-D`` switches (the mutation tests use them to
    build deliberately broken copies of the oracle in a temp directory)."""
    src = os.path.join(HERE, "msa_oracle.c")
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-Wall", "-Wextra", "-o", out, src, "-lm"]
    cmd[1:1] = ["-D" + d for d in defines]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("oracle build failed:\n" + res.stderr)
    if not quiet and res.stderr:
        sys.stderr.write(res.stderr)
    return out


if __name__ == "__main__":
    print(build(quiet=False))
