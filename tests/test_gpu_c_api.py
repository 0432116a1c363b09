"""The attention from a plain C program: tests/c_api/attn_demo.c allocates
device memory with the HIP runtime's C API, builds the step's mask with the
library, runs lvsa_attention and lvsa_attention_ws on the NULL stream and
writes the outputs, with no Python or torch in any call.  The outputs are
checked against the float64 oracle and, bit for bit, against the same calls
made through the Python binding."""

import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

import block_sparse_attention_lvsa_amd as L
import oracle.attention as oa
import oracle.mask as om
from block_sparse_attention_lvsa_amd.synth import make_random
from tests.test_gpu_parity import assert_close, say, workspace_for

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bf16_bytes(x: torch.Tensor) -> bytes:
    return x.contiguous().view(torch.int16).numpy().tobytes()


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_c_program_runs_the_attention(gpu, tmp_path):
    # two query tiles per frame (128 + 72 rows), split items in the workspace path
    B, H, T, P, D, C, W, step = 2, 3, 12, 200, 128, 5, 2, 4
    say("C caller", (B, H, T, P, D, C, W, step), "seeds 700-702")
    q, k, v = (make_random((B, H, T * P, D), 700 + i) for i in range(3))
    qkv = tmp_path / "qkv.bin"
    qkv.write_bytes(b"".join(_bf16_bytes(x) for x in (q, k, v)))

    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    lib_dir = os.path.dirname(L.library()._name)
    exe = tmp_path / "attn_demo"
    cmd = ["gcc", "-std=c99", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_api", "attn_demo.c"), "-o", str(exe),
           "-L", lib_dir, "-llvsa", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           f"-Wl,-rpath,{lib_dir}", f"-Wl,-rpath,{os.path.join(rocm, 'lib')}"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr

    outs = [tmp_path / "out_plain.bin", tmp_path / "out_ws.bin"]
    args = [str(x) for x in (B, H, T, P, D, C, W, step)] + [str(qkv)] + [str(o) for o in outs]
    r = subprocess.run([str(exe), *args], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
    got = [torch.from_numpy(np.fromfile(o, dtype=np.int16)).view(torch.bfloat16).view(B, H, T * P, D) for o in outs]

    ref = oa.block_attention(q, k, v, om.key_frames(T, C, W, step))
    assert_close(got[0], ref, "C caller, lvsa_attention")
    assert_close(got[1], ref, "C caller, lvsa_attention_ws")

    m = L.lvsa_build_mask(T, C, W, step).to(gpu)
    qd, kd, vd = q.to(gpu), k.to(gpu), v.to(gpu)
    a = L.lvsa_attention(qd, kd, vd, m)
    b = L.lvsa_attention(qd, kd, vd, m, workspace=workspace_for(qd, T))
    torch.cuda.synchronize()
    assert torch.equal(a.cpu(), got[0]), "lvsa_attention: C and Python callers differ"
    assert torch.equal(b.cpu(), got[1]), "lvsa_attention_ws: C and Python callers differ"
