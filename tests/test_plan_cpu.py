"""The projection workspaces, sized on the host without a device, fit the
GEMM plan that a call makes on any device of 1..256 compute units (every
batch size up to 300 and a geometric sweep to the maximum batch). The plan
and layout code is the library's own host-only header, compiled here with
the host compiler alone, under AddressSanitizer and UndefinedBehaviorSanitizer
(an overflow in the size arithmetic aborts the sweep)."""

import os
import shutil
import subprocess

import pytest

from conftest import ROOT

CSRC = os.path.join(ROOT, "decode_attention_attn_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "native", "plan_sweep.cpp")


def test_workspace_bounds_every_device_plan(tmp_path):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.fail("no host C++ compiler")
    exe = str(tmp_path / "plan_sweep")
    subprocess.run([cxx, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-fno-omit-frame-pointer", f"-I{CSRC}", SRC, "-o", exe], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1")
    env.pop("LD_PRELOAD", None)  # the instrumented program links its own runtime
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, env=env)
    print(r.stdout[-2000:])
    assert r.returncode == 0, r.stdout[-2000:]
    assert "0 over their workspace" in r.stdout
    assert "runtime error" not in r.stdout and "AddressSanitizer" not in r.stdout
