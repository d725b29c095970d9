"""Compile the HIP sources into ``libdeltalog.so`` (gfx950), in-tree.

    python -m linear_attention_recurrent_dl_amd.build [-j N] [--save-temps]

Each ``csrc/*.hip`` file is compiled separately (in parallel) with hipcc and
linked into one shared library next to this file.  Packed-fp32 instructions are
disabled for all device code (``-packed-fp32-ops``).  The compiler's per-kernel
resource report is read back: a kernel that needs scratch memory (register
spills, or a private array the compiler could not keep in registers) fails the
build, since it would stall every block of these bandwidth-bound kernels.
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libdeltalog.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"


def hipcc() -> str:
    h = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return h


def compile_flags() -> list:
    # kernarg preload: the decode kernel's leading arguments (launch geometry,
    # the first slot of a consecutive launch, the base and counter pointers:
    # 10 dwords) arrive in registers, no scalar load ahead of its first fetch
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-mllvm", "-amdgpu-kernarg-preload-count=10",
            "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function"]


def sources() -> list:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


_FUNC = re.compile(r"remark: Function Name: (\S+)")
_SCRATCH = re.compile(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)")


def scratch_kernels(report: str) -> list:
    """(kernel, bytes per lane) of every kernel with scratch in a resource report."""
    out, name = [], None
    for line in report.splitlines():
        m = _FUNC.search(line)
        if m:
            name = m.group(1)
            continue
        m = _SCRATCH.search(line)
        if m and int(m.group(1)) > 0:
            out.append((name, int(m.group(1))))
    return out


def _compile(src: str, extra: list) -> str:
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [hipcc()] + compile_flags() + extra + ["-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    bad = scratch_kernels(r.stderr)
    if bad:
        raise RuntimeError(f"{src}: kernels use scratch memory: " +
                           ", ".join(f"{k} ({b} B/lane)" for k, b in bad))
    return obj


PROBE_SRC = os.path.join(PKG, "probe", "stream_probe.hip")
PROBE_LIB = os.path.join(PKG, "libdl_stream_probe.so")


def build_probe(verbose: bool = True) -> str:
    """The benchmark's streaming reference kernel, a library of its own."""
    tmp = PROBE_LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + compile_flags() + ["-shared", PROBE_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {PROBE_SRC}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, PROBE_LIB)
    if verbose:
        print(f"[build] {PROBE_LIB}", flush=True)
    return PROBE_LIB


def build(jobs: int = 0, extra: list = None, verbose: bool = True) -> str:
    extra = list(extra or []) + os.environ.get("DL_EXTRA_CFLAGS", "").split()
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), os.cpu_count() or 1, 16)
    t0 = time.time()
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), srcs))
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"[build] {LIB_PATH} ({len(srcs)} sources, {time.time() - t0:.1f}s)", flush=True)
    build_probe(verbose)
    return LIB_PATH


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", "--jobs", type=int, default=0)
    ap.add_argument("--save-temps", action="store_true", help="keep device assembly in _build/")
    a = ap.parse_args(argv)
    extra = ["-save-temps=obj"] if a.save_temps else []
    build(a.jobs, extra)
    return 0


if __name__ == "__main__":
    sys.exit(main())
