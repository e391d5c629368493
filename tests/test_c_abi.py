"""include/mcs.h is a plain C header: a C99 program compiled with the host C
compiler (warnings as errors) links against libmcs.so and runs the calls that
need no GPU (tests/c_abi/consumer.c)."""
import os
import shutil
import subprocess

import pytest

import sparse_attention_diffusion_attn_amd as mcs

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no host C compiler")
def test_c99_consumer_builds_and_runs(tmp_path):
    mcs.lib()  # the library must exist (built by the package's build step)
    exe = tmp_path / "consumer"
    libdir = os.path.dirname(mcs.LIB_PATH)
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "c_abi", "consumer.c"),
           "-L", libdir, "-l:libmcs.so", f"-Wl,-rpath,{libdir}", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip() == "ok"
