"""Build the CPU oracle (test infrastructure) with the host C++ compiler.

The oracle is compiled with -O2, no fast-math and no floating-point
contraction, so every fp32 step is a single IEEE operation rounded to
nearest. It is built here, beside its sources, as ``libqcast_oracle.so``; a
stamp file holds the SHA-256 of the sources it was built from.
"""
import hashlib
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCES = ["qcast_oracle.cpp", "qcast_oracle.h"]
LIB = os.path.join(HERE, "libqcast_oracle.so")
STAMP = LIB + ".sha256"
CXX = os.environ.get("ORACLE_CXX", "g++")
FLAGS = ["-std=c++17", "-O2", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
         "-Wall", "-Wextra", "-Werror"]


def source_digest():
    h = hashlib.sha256()
    for name in SOURCES:
        with open(os.path.join(HERE, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    h.update(" ".join([CXX] + FLAGS).encode())
    return h.hexdigest()


def is_current():
    if not os.path.exists(LIB) or not os.path.exists(STAMP):
        return False
    with open(STAMP) as f:
        return f.read().strip() == source_digest()


def build(force=True):
    """Compile the oracle; with force=False only when sources changed."""
    if not force and is_current():
        return LIB
    tmp = LIB + ".tmp"
    cmd = [CXX] + FLAGS + [os.path.join(HERE, "qcast_oracle.cpp"), "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    with open(STAMP, "w") as f:
        f.write(source_digest() + "\n")
    return LIB


if __name__ == "__main__":
    print(build(force="--if-needed" not in sys.argv))
