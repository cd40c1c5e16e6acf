"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the
CPU: the library's host side (argument checks, workspace layout, the
one-row kernel's fit test, dispatch) built with both sanitizers and driven
by the ABI tests, and the oracle built with both and driven by its own
tests. A sanitizer report fails the run (no recovery), and so does any test
failure. The device code is built as usual: sanitizers for GPU code are not
used here."""
import glob
import os
import subprocess
import sys

import pytest

import block_fp8_mixture_router_amd as moe
from block_fp8_mixture_router_amd import build as moe_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")
RUNNER = os.path.join(TESTS, "sanitize_run.py")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
HOST_SOURCES = ("api.hip", "noalloc.hip")  # the files holding the library's host logic
REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer")


def _run(preload, args, tmp_path):
    env = dict(os.environ)
    env["LD_PRELOAD"] = preload + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, RUNNER] + args, cwd=str(tmp_path), env=env,
                       capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert not any(s in out for s in REPORTS), out[-4000:]
    assert r.returncode == 0, out[-4000:]
    return out


def test_host_library_under_asan_ubsan(tmp_path):
    cc = moe_build.hipcc()
    objs = [os.path.join(moe_build.BUILD_DIR, os.path.basename(s) + ".o")
            for s in moe_build.sources() if os.path.basename(s) not in HOST_SOURCES]
    if not all(os.path.exists(o) for o in objs):
        moe_build.build()  # the kernels' objects, built as usual
    san_objs = []
    for f in HOST_SOURCES:
        o = str(tmp_path / (f + ".o"))
        subprocess.run([cc] + moe_build.HIP_FLAGS + HOST_SAN +
                       ["-I", moe_build.INCLUDE, "-I", moe_build.CSRC, "-c",
                        os.path.join(moe_build.CSRC, f), "-o", o],
                       check=True, capture_output=True)
        san_objs.append(o)
    so = str(tmp_path / "libmoe_san.so")
    subprocess.run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", so] + san_objs + objs,
                   check=True, capture_output=True)
    rt = glob.glob(os.path.join(os.path.dirname(os.path.dirname(cc)),
                                "lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    assert rt, "clang's AddressSanitizer runtime not found"
    out = _run(rt[0], [so, "-", os.path.join(TESTS, "test_abi.py")], tmp_path)
    assert " passed" in out


def test_oracle_under_asan_ubsan(tmp_path):
    so = str(tmp_path / "liboracle_san.so")
    src = os.path.join(ROOT, "oracle", "moe_oracle.c")
    flags = ["-O1", "-g", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all",
             "-fno-fast-math", "-ffp-contract=off", "-std=c11", "-D_GNU_SOURCE"]
    subprocess.run(["gcc"] + flags + ["-fsanitize=address,undefined", "-shared", "-fPIC", "-o", so, src, "-lm"],
                   check=True, capture_output=True)
    rt = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                        text=True, check=True).stdout.strip()
    assert os.path.isabs(rt), "gcc's AddressSanitizer runtime not found"
    files = sorted(glob.glob(os.path.join(TESTS, "test_oracle_*.py")))
    assert files
    out = _run(rt, ["-", so] + files, tmp_path)
    assert " passed" in out
