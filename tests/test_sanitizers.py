"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds tests/c_api/sanitize_demo.cpp together with the library's sources --
the host mask builder, the status code and the host side of the attention
entry points (their argument checks) -- with ASan and UBSan (any report
aborts), and runs its three parts: the mask-builder sweep and validator fuzz
(with leak checking), every argument error of the attention entry points, and
the "no device" path.  CPU only: no kernel is launched.
"""

import os
import shutil
import subprocess

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_attention_lvsa_amd", "csrc")
CLANG = "/opt/rocm/llvm/bin/clang++"
HIPCC = "/opt/rocm/bin/hipcc"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
# the same flags, for the host pass of a HIP source only
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
INC = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]

pytestmark = pytest.mark.skipif(not (os.path.exists(CLANG) and os.path.exists(HIPCC)), reason="ROCm clang missing")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, " ".join(cmd) + "\n" + r.stdout[-3000:] + r.stderr[-3000:]
    return r


@pytest.fixture(scope="module")
def demo(tmp_path_factory):
    out = tmp_path_factory.mktemp("san")
    objs = []
    for src in (os.path.join(CSRC, "mask.cpp"), os.path.join(CSRC, "status.cpp"),
                os.path.join(ROOT, "tests", "c_api", "sanitize_demo.cpp")):
        obj = str(out / (os.path.basename(src) + ".o"))
        _run([CLANG, "-std=c++17", "-O1", "-g", *SAN, *INC, "-c", src, "-o", obj])
        objs.append(obj)
    obj = str(out / "attention.o")
    _run([HIPCC, "-x", "hip", "--offload-arch=gfx950", "-std=c++17", "-O1", "-g", *HOST_SAN, *INC,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-c", os.path.join(CSRC, "attention.hip"), "-o", obj])
    objs.append(obj)
    exe = str(out / "sanitize_demo")
    _run([CLANG, *SAN, *objs, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    return exe


def _env(leaks):
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = f"detect_leaks={1 if leaks else 0}:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env.pop("LD_PRELOAD", None)
    return env


def test_mask_builders_and_validator_are_clean(demo):
    r = subprocess.run([demo, "masks"], capture_output=True, text=True, timeout=600, env=_env(leaks=True))
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout[-2000:] + r.stderr[-4000:]


def test_attention_argument_checks_are_clean(demo):
    r = subprocess.run([demo, "abi"], capture_output=True, text=True, timeout=300, env=_env(leaks=True))
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout[-2000:] + r.stderr[-4000:]


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device path")
def test_no_device_path_is_clean(demo):
    # the HIP runtime is initialised here; its own allocations are not ours to
    # check for leaks
    r = subprocess.run([demo, "abi-no-device"], capture_output=True, text=True, timeout=300, env=_env(leaks=False))
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout[-2000:] + r.stderr[-4000:]
