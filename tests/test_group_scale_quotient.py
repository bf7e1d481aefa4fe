"""The per-group FP8 epilogue forms absmax / 448 as an FMA-corrected product with RN(1/448)
instead of a division sequence (for absmax >= 2^-120; below that it divides).
tests/group_scale_quotient.c checks on the host, in binary32, that the product equals the IEEE
quotient it replaces; the GPU parity tests then compare every per-group scale with the oracle's
quotient bit for bit."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def test_group_scale_quotient_identity(tmp_path):
    exe = str(tmp_path / "group_scale_quotient")
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-ffp-contract=off",
           "-fno-fast-math", os.path.join(HERE, "group_scale_quotient.c"), "-o", exe, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr
