"""The C-ABI suite (tests/test_abi_cpu.py) against a build of libmfa whose
host code runs under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU):
every validation path of every entry point, with out-of-range values, null
and misaligned pointers and short workspaces, must run without a memory error
or undefined behaviour. Device code is compiled as for the product library;
the sanitizers apply to the host side only (-Xarch_host). The build goes to
a temporary copy of the package, so the product library is left as it is."""

import glob
import os
import shutil
import subprocess
import sys

import pytest

from conftest import ROOT

sys.path.insert(0, ROOT)
from decode_attention_attn_amd import build as B  # noqa: E402

HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        pytest.fail("clang's AddressSanitizer runtime is not installed under /opt/rocm/llvm")
    return hits[-1]


def _run(cmd, **kw):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)
    return r.returncode, r.stdout


def test_abi_suite_under_host_sanitizers(tmp_path):
    pkg = tmp_path / "pkg"
    shutil.copytree(os.path.join(ROOT, "decode_attention_attn_amd"), pkg / "decode_attention_attn_amd",
                    ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    shutil.copytree(os.path.join(ROOT, "include"), pkg / "include")
    (pkg / "tests").mkdir()
    for f in ("conftest.py", "parity.py", "test_abi_cpu.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), pkg / "tests" / f)
    shutil.copy(os.path.join(ROOT, "pytest.ini"), pkg / "pytest.ini")

    csrc = pkg / "decode_attention_attn_amd" / "csrc"
    common = [f if not f.startswith("-I") else f"-I{pkg / 'include'}" for f in B.COMMON]
    common = [f for f in common if f != "-O3"] + ["-O1", "-g"]
    objs = []
    for src in B.SOURCES:
        obj = str(tmp_path / (src + ".o"))
        cmd = [B.HIPCC] + (["-x", "hip"] if src.endswith(".hip") else []) + common + B.EXTRA.get(src, [])
        cmd += HOST_SANITIZE + ["-c", str(csrc / src), "-o", obj]
        rc, out = _run(cmd)
        assert rc == 0, out[-3000:]
        objs.append(obj)
    lib = str(pkg / "decode_attention_attn_amd" / "libmfa.so")
    rc, out = _run([B.HIPCC, f"--offload-arch={B.ARCH}", "-shared", "-fPIC"] + HOST_SANITIZE[:4] + ["-o", lib] + objs)
    assert rc == 0, out[-3000:]

    env = dict(os.environ)
    pre = env.get("LD_PRELOAD", "")
    env["LD_PRELOAD"] = _asan_runtime() + (":" + pre if pre else "")  # the runtime must come first
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    rc, out = _run([sys.executable, "-m", "pytest", "tests/test_abi_cpu.py", "-q", "-x", "-p", "no:cacheprovider"],
                   cwd=str(pkg), env=env, timeout=600)
    print(out[-3000:])
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-6000:]
    assert rc == 0, out[-6000:]
    assert " passed" in out
