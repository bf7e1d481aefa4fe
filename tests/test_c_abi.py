"""The C ABI from a plain C caller (tests/c_abi_caller.c, built here with gcc against
include/rmsq.h, librmsq.so, the HIP runtime and the oracle library): no Python marshalling in
between.  On the CPU the caller checks argument errors, status strings and the launch query;
on the GPU it also runs fused, batch-scale FP4 and QK-norm + RoPE launches and compares them
with the oracle's host twins."""
import os
import subprocess

import pytest

from rmsnorm_quantization_amd import binding as B
from rmsnorm_quantization_amd import build as hb
import oracle  # noqa: F401  (builds the oracle library if needed)
from oracle import build as ob

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.fixture(scope="module")
def caller(tmp_path_factory):
    B.lib()  # the library exists and has this ABI version
    ob.ensure_built()
    exe = str(tmp_path_factory.mktemp("c_abi") / "c_abi_caller")
    libdirs = [os.path.dirname(hb.LIB), os.path.dirname(ob.LIB), os.path.join(ROCM, "lib")]
    cmd = ["gcc", "-std=c11", "-O1", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "oracle"),
           "-isystem", os.path.join(ROCM, "include"), os.path.join(HERE, "c_abi_caller.c"),
           "-o", exe]
    for d in libdirs:
        cmd += ["-L", d, f"-Wl,-rpath,{d}"]
    cmd += ["-lrmsq", "-loracle_rmsq", "-lamdhip64", "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return exe


def test_c_caller_host_checks(caller):
    r = subprocess.run([caller, "validate"], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failure(s)" in r.stdout


@pytest.mark.gpu
def test_c_caller_on_the_gpu(caller):
    from tests import gpu_harness as GH

    GH.require_gpu()
    print("[c-abi] running the C caller on the GPU", flush=True)
    r = subprocess.run([caller, "gpu"], capture_output=True, text=True, timeout=120)
    print(r.stdout, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "bit-exact" in r.stdout and "DIFFERENT" not in r.stdout
