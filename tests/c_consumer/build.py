"""Build kda_c_consumer (plain C11 against include/kda.h, libkda.so, the C oracle
and the HIP runtime's C API) in this folder; rpaths point at the in-tree
libraries relative to the binary."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "kda_c_consumer.c")
BIN = os.path.join(HERE, "kda_c_consumer")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def command(out: str = BIN):
    return ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
            "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), SRC,
            "-o", out,
            "-L", os.path.join(ROOT, "linear_attention_fwd_amd"), "-lkda",
            "-L", os.path.join(ROOT, "oracle"), "-lkda_oracle",
            "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
            "-Wl,-rpath,$ORIGIN/../../linear_attention_fwd_amd", "-Wl,-rpath,$ORIGIN/../../oracle",
            "-Wl,-rpath," + os.path.join(ROCM, "lib")]


def build(verbose: bool = False) -> str:
    cmd = command(BIN + ".tmp")
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(BIN + ".tmp", BIN)
    return BIN


if __name__ == "__main__":
    print(build(verbose=True))
