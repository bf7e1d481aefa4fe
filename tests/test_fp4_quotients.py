"""The FP4 epilogue forms (a * gs) / 6 and gs / decode(sf) without a division sequence per
chunk: an FMA-corrected product with RN(1/6), and gs / (1 + j/8) scaled by a power of two.
tests/fp4_quotients.c checks on the host, in binary32, that both equal the IEEE quotients they
replace (the first exhaustively over every significand); the GPU parity tests then compare the
kernels' FP4 codes and scales with the oracle bit for bit."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def test_fp4_quotient_identities(tmp_path):
    exe = str(tmp_path / "fp4_quotients")
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-ffp-contract=off",
           "-fno-fast-math", os.path.join(HERE, "fp4_quotients.c"), "-o", exe, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr
