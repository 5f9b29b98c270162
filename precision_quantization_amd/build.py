"""Build libqcast.so, the gfx950 quantization-cast library, in-tree.

Every ``csrc/*.hip`` file is compiled for gfx950 with hipcc, in parallel, and
linked into ``precision_quantization_amd/libqcast.so``. A stamp file beside
the library records the SHA-256 of the sources, the public header and the
flags (their code: comments and layout do not count); the loader refuses a
library whose stamp does not match the sources it sits beside.

    python -m precision_quantization_amd.build
"""
import concurrent.futures
import glob
import hashlib
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libqcast.so")
STAMP = LIB + ".sha256"
BUILD_DIR = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no floating-point contraction: every fp32 step is one rounded operation
    "-ffp-contract=off",
    # keep packed fp32 arithmetic out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result", "-fvisibility=hidden",
]
# Include paths are absolute and differ between checkouts; they are left out
# of the source digest.
INCLUDES = [f"-I{INCLUDE}", f"-I{CSRC}"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def code_tokens(text):
    """C/C++ source with its comments removed (comment markers inside string
    and character literals are code), every line's whitespace runs made one
    space, and empty lines dropped, so that edits to comments or layout leave
    the digest alone."""
    out = []
    i, n = 0, len(text)
    while i < n:
        c = text[i]
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    lines = []
    for line in "".join(out).split("\n"):
        words = line.split()
        if words:
            lines.append(" ".join(words))
    return "\n".join(lines)


def source_digest():
    """SHA-256 of the code (comments and layout aside) of the sources, the
    headers and the flags."""
    h = hashlib.sha256()
    files = sources() + sorted(glob.glob(os.path.join(CSRC, "*.h"))) + \
        sorted(glob.glob(os.path.join(INCLUDE, "*.h")))
    for path in files:
        with open(path, encoding="utf-8") as f:
            code = code_tokens(f.read())
        h.update(os.path.basename(path).encode() + b"\0" + code.encode())
    h.update(" ".join(FLAGS).encode())
    return h.hexdigest()


def is_current():
    if not (os.path.exists(LIB) and os.path.exists(STAMP)):
        return False
    with open(STAMP) as f:
        return f.read().strip() == source_digest()


def _compile(src):
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC] + FLAGS + INCLUDES + ["-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(force=True, jobs=8):
    """Compile and link libqcast.so; with force=False only if sources changed."""
    if not force and is_current():
        return LIB
    if not os.path.exists(HIPCC) and shutil.which(HIPCC) is None:
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, sources()))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stderr)
    os.replace(tmp, LIB)
    with open(STAMP, "w") as f:
        f.write(source_digest() + "\n")
    return LIB


if __name__ == "__main__":
    print(build(force="--if-needed" not in sys.argv))
