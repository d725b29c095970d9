"""The host mirror of live-log lengths across a call split into launches
(csrc/dl_mirror.hpp), compiled with the host C++ compiler alone: when a later
launch fails, host and device agree on every slot (the launched prefix
advanced, the rest unchanged)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_mirror_follows_the_launched_prefix(tmp_path):
    exe = tmp_path / "mirror_check"
    src = os.path.join(ROOT, "tests", "host_unit", "mirror_check.cpp")
    inc = os.path.join(ROOT, "linear_attention_recurrent_dl_amd", "csrc")
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-Werror", "-I", inc, src, "-o", str(exe)], check=True,
                   capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout
