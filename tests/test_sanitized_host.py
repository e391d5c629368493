"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

mcs_api.cpp holds all of the library's host-side logic: argument validation,
the 128-bit stride and span arithmetic of the strided layouts, the overlap
check of output rows, workspace carving and launch set-up.  The build step
compiles it with the host compiler under ASan + UBSan (-fno-sanitize-recover,
so undefined behaviour aborts) into _build/libmcs_san.so, linked with the
unchanged kernel objects.  The C99 consumer and the ABI validation tests then
run against that library; every call they make is answered on the host, so no
GPU is needed.
"""
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
REPORTS = ("ERROR: AddressSanitizer", "ERROR: LeakSanitizer", "runtime error:")

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None,
                                reason="no host C/C++ compiler")


@pytest.fixture(scope="module")
def san_lib():
    from sparse_attention_diffusion_attn_amd import build as b
    return b.build_sanitized()


def _env(san_lib, preload):
    env = dict(os.environ)
    env["MCS_LIBRARY"] = san_lib
    env["ASAN_OPTIONS"] = "detect_leaks=0" if preload else "detect_leaks=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    if preload:
        asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
        env["LD_PRELOAD"] = asan
    return env


def _clean(r):
    out = r.stdout + r.stderr
    assert not any(m in out for m in REPORTS), out[-4000:]
    return out


def test_c_consumer_under_sanitizers(san_lib, tmp_path):
    exe = tmp_path / "consumer_san"
    libdir = os.path.dirname(san_lib)
    cmd = ["gcc", "-std=c99", "-Wall", "-Werror", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
           "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "c_abi", "consumer.c"),
           "-L", libdir, "-l:libmcs_san.so", f"-Wl,-rpath,{libdir}", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120, env=_env(san_lib, False))
    _clean(r)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr


def test_abi_validation_tests_under_sanitizers(san_lib):
    env = _env(san_lib, True)
    # the instrumented library is the one the binding loads, with the runtime
    probe = ("import sparse_attention_diffusion_attn_amd as m; m.lib(); "
             "maps = open('/proc/self/maps').read(); "
             "print('libmcs_san.so' in maps, 'libasan' in maps)")
    r = subprocess.run([sys.executable, "-c", probe], capture_output=True, text=True, cwd=ROOT, env=env,
                       timeout=120)
    assert r.returncode == 0 and r.stdout.split() == ["True", "True"], r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_abi.py")], capture_output=True, text=True, cwd=ROOT,
                       env=env, timeout=600)
    out = _clean(r)
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
