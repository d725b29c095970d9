"""Compile the plain C consumer of the C ABI (gcc, against include/deltalog.h,
the in-tree libdeltalog.so and the HIP runtime).  Run by the repository's
build step, before any test; the binary sits next to its source."""

from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "linear_attention_recurrent_dl_amd")
SRC = os.path.join(HERE, "dl_c_consumer.c")
BIN = os.path.join(HERE, "dl_c_consumer")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           # the HIP runtime headers need the platform named when hipcc is not the compiler
           "-D__HIP_PLATFORM_AMD__", SRC, "-o", BIN + ".tmp",
           "-L", PKG, "-ldeltalog", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../linear_attention_recurrent_dl_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"C consumer build failed:\n{' '.join(cmd)}\n{r.stderr}")
    os.replace(BIN + ".tmp", BIN)
    return BIN


if __name__ == "__main__":
    print(build())
