"""Builds tests/abi_consumer (a plain C11 caller of include/moe.h) with gcc,
linked against the in-tree combine_dispatch_amd/libmoe_hip.so and the HIP
runtime's C API.  Test infrastructure, run on the CPU by the build step."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "abi_consumer.c")
EXE = os.path.join(HERE, "abi_consumer")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra",
           # the HIP runtime's C API headers need the platform named
           "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", f"-I{os.path.join(ROOT, 'include')}",
           SRC, "-o", EXE + ".tmp",
           f"-L{os.path.join(ROOT, 'combine_dispatch_amd')}", "-lmoe_hip",
           f"-L{ROCM}/lib", "-lamdhip64",
           # found next to the binary wherever the tree is copied
           "-Wl,-rpath,$ORIGIN/../combine_dispatch_amd", f"-Wl,-rpath,{ROCM}/lib"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed:\n{r.stdout}{r.stderr}")
    os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    print(build(verbose=True))
