"""Builds the C oracle (test infrastructure only) with plain gcc, no fast-math."""
import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path():
    return os.path.join(_HERE, "liboracle.so")


def build():
    src = os.path.join(_HERE, "b2b_oracle.c")
    out = library_path()
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
                           "-pthread", "-Wall", "-Wextra", "-o", tmp, src, "-lm"])
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
