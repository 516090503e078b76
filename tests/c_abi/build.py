"""Builds mx_c_driver (test infrastructure: the C program that drives the library's C ABI with no
Python in between) in-tree with the host C compiler, linked against the built libmx_gfx950.so and
the HIP runtime.

    python tests/c_abi/build.py
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "mx_c_driver.c")
EXE = os.path.join(HERE, "mx_c_driver")
LIBDIR = os.path.join(ROOT, "block_scaled_precision_act_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = False) -> str:
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler found")
    tmp = EXE + ".tmp"
    cmd = [cc, "-O2", "-std=c11", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           f"-I{ROCM}/include", SRC, "-o", tmp,
           f"-L{LIBDIR}", "-lmx_gfx950", f"-L{ROCM}/lib", "-lamdhip64",
           # found at run time next to the tree, wherever the tree is
           "-Wl,-rpath,$ORIGIN/../../block_scaled_precision_act_amd", f"-Wl,-rpath,{ROCM}/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"C build failed on {SRC}:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, EXE)
    if verbose:
        print(f"built {EXE}")
    return EXE


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
