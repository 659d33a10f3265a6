"""Builds tests/c_client/hla_c_client: a plain C99 program that calls libhla.

Usage: python tests/c_client/build_client.py   (also run by __graft_entry__.build()
after the library is built). gcc compiles it as C99 with every warning an
error; the HIP runtime header is included as a system header. The binary finds
libhla.so through a relative run path, so it runs from any copy of the tree.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "hla_c_client.c")
OUT = os.path.join(HERE, "hla_c_client")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = True) -> str:
    lib_dir = os.path.join(ROOT, "softmax_attention_amd")
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-D__HIP_PLATFORM_AMD__", "-isystem", os.path.join(ROCM, "include"),
           "-I", os.path.join(ROOT, "include"), SRC, "-o", OUT + ".tmp",
           "-L", lib_dir, "-lhla", "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../softmax_attention_amd", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed for {SRC}:\n{r.stdout}\n{r.stderr}")
    os.replace(OUT + ".tmp", OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build()
    sys.exit(0)
