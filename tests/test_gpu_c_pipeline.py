"""The method end to end from a plain C99 program (tests/c_abi/pipeline.c):
device buffers from the HIP runtime, no PyTorch on the caller's side.  The
program runs an anchor step and one reuse step through the C ABI and writes
its inputs and outputs; every output is checked against the fp64 oracle, each
stage on the GPU's upstream outputs (as in the other parity tests)."""
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

from oracle import mcs_oracle as orc
from tests import parity as par

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
B, H, NV, NP, D, C, TOPK = 1, 2, 300, 320, 64, 64, 70


def load_bf16(path, shape):
    raw = np.fromfile(path, dtype=np.uint16).reshape(shape)
    return par.bf16_to_f64(torch.from_numpy(raw.view(np.int16)).view(torch.bfloat16))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no host C compiler")
def test_c99_program_runs_the_method(tmp_path):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_diffusion_attn_amd as mcs
    mcs.lib()
    libdir = os.path.dirname(mcs.LIB_PATH)
    exe = tmp_path / "pipeline"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           os.path.join(HERE, "c_abi", "pipeline.c"), "-o", str(exe),
           "-L", libdir, "-l:libmcs.so", f"-Wl,-rpath,{libdir}",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    print("running the C pipeline", flush=True)
    r = subprocess.run([str(exe), str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip() == "ok"

    shp = (B, H, NP, D)
    q0, k0, v0 = (load_bf16(tmp_path / f"{n}0.bin", shp) for n in "qkv")
    q1, k1, v1 = (load_bf16(tmp_path / f"{n}1.bin", shp) for n in "qkv")
    o_full, res, o = (load_bf16(tmp_path / f"{n}.bin", shp) for n in ("o_full", "r", "o"))
    perm = np.fromfile(tmp_path / "perm.bin", dtype=np.int32).reshape(B, H, NP)
    kv = np.fromfile(tmp_path / "kv.bin", dtype=np.int32).reshape(B, H, NP // C, TOPK)
    lse = np.fromfile(tmp_path / "lse.bin", dtype=np.float32).reshape(B, H, NP)
    sc = 1.0 / 8.0
    for h in range(H):
        p = perm[0, h]
        assert sorted(p.tolist()) == list(range(NP))
        for g in range(NP // C):
            assert np.all(np.diff(p[g * C:(g + 1) * C]) > 0)
        ref_o, ref_l = orc.dense_attention(q0[0, h], k0[0, h], v0[0, h], NV, sc)
        par.assert_close(o_full[0, h, :NV], ref_o[:NV], what="O_full")
        assert np.abs(lse[0, h, :NV] - ref_l[:NV]).max() < 1e-3
        a = orc.group_scores(q0[0, h], k0[0, h], p, ref_l, NV, C, sc)
        for g in range(NP // C):
            par.check_selection(kv[0, h, g], a[g], TOPK)
        o_sp = orc.sparse_attention(q0[0, h], k0[0, h], v0[0, h], p, kv[0, h], NV, C, sc)
        par.assert_close(res[0, h, :NV], (o_full[0, h] - o_sp)[:NV], what="R")
        assert np.all(res[0, h, NV:] == 0)
        ref = orc.reuse_step(q1[0, h], k1[0, h], v1[0, h], p, kv[0, h], res[0, h], NV, C, sc)
        par.assert_close(o[0, h, :NV], ref[:NV], what="reuse O")
        assert np.all(o[0, h, NV:] == 0)
