"""Compile tests/c/abi_smoke: a plain C program that uses libqcast.so through
include/qcast.h, with no Python or torch (run by tests/test_gpu_c_abi.py).
It links the in-tree library through a relative rpath, so build the library
first."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "abi_smoke.c")
BIN = os.path.join(HERE, "abi_smoke")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build():
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-D__HIP_PLATFORM_AMD__",
           f"-I{ROCM}/include", f"-I{os.path.join(ROOT, 'include')}", SRC,
           f"-L{ROCM}/lib", "-lamdhip64",
           f"-L{os.path.join(ROOT, 'precision_quantization_amd')}", "-lqcast",
           "-Wl,-rpath,$ORIGIN/../../precision_quantization_amd", f"-Wl,-rpath,{ROCM}/lib",
           "-o", BIN]
    subprocess.run(cmd, check=True)
    return BIN


if __name__ == "__main__":
    print(build())
