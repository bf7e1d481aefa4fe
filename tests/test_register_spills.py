"""No kernel instantiation of librmsq spills registers to scratch memory, except the binary16
ones with masked chunks at many chunks per lane (fused_kernel with 6-8 chunks per lane and
SiLU+Mul with 5-8, binary16, with a residual and an inexact fit): their binary16 conversions
keep more values live than the 128 VGPRs a 1024-thread launch bound allows.  The default launch
rules avoid those (the padded-output rule caps binary16 rows at 5 chunks per lane), so a spill
anywhere else is a regression of speed, found here by compiling the instantiation tables for
gfx950 with the compiler's resource report (no GPU needed)."""
import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from rmsnorm_quantization_amd import build as hb

TABLES = [s for s in hb.SRC if os.path.basename(s).startswith("table_")]
# mangled template arguments: fused_kernel<MODE, RES, VPT, GS, EXACT, DT>,
# silu_mul_kernel<MODE, VPT, GS, EXACT, DT>
FUSED = re.compile(r"fused_kernelILi(\d)ELb(\d)ELi(\d)ELi(\d+)ELb(\d)ELi(\d)E")
SILU = re.compile(r"silu_mul_kernelILi(\d)ELi(\d)ELi(\d+)ELb(\d)ELi(\d)E")


def _report(src):
    cmd = hb.command("/dev/null", src=[src])
    cmd.remove("-shared")
    cmd[1:1] = ["-c", "--offload-device-only", "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    names = re.findall(r"Function Name: (\S+)", r.stderr)
    scratch = [int(v) for v in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", r.stderr)]
    assert len(names) == len(scratch) and names
    return list(zip(names, scratch))


def _allowed(name):
    m = FUSED.search(name)
    if m:
        mode, res, vpt, gs, exact, dt = (int(g) for g in m.groups())
        return dt == 1 and res == 1 and exact == 0 and vpt >= 6
    m = SILU.search(name)
    if m:
        mode, vpt, gs, exact, dt = (int(g) for g in m.groups())
        return dt == 1 and exact == 0 and vpt >= 5
    return False


@pytest.mark.slow
def test_no_unexpected_register_spills():
    with ThreadPoolExecutor(max_workers=min(len(TABLES), os.cpu_count() or 1)) as ex:
        reports = list(ex.map(_report, TABLES))
    spills = [(n, s) for rep in reports for n, s in rep if s > 0]
    unexpected = [(n, s) for n, s in spills if not _allowed(n)]
    assert not unexpected, f"instantiations spilling to scratch: {unexpected[:8]}"
    # every bf16 instantiation is free of spills
    assert all(not (FUSED.search(n) and FUSED.search(n).group(6) == "0") for n, _ in spills)
