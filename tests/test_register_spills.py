"""No kernel instantiation of librmsq spills registers to scratch memory.  A spill is a large
loss of speed (a binary16 padded-output row at 6 chunks per lane once took 69 us instead of
18 us), so every instantiation the tables define -- bf16 and binary16, exact and masked, 1 to 8
chunks per lane -- is compiled for gfx950 with the compiler's resource report and checked (no
GPU needed)."""
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


@pytest.mark.slow
def test_no_register_spills():
    with ThreadPoolExecutor(max_workers=min(len(TABLES), os.cpu_count() or 1)) as ex:
        reports = list(ex.map(_report, TABLES))
    names = [n for rep in reports for n, _ in rep]
    assert any(FUSED.search(n) for n in names) and any(SILU.search(n) for n in names)
    spills = [(n, s) for rep in reports for n, s in rep if s > 0]
    assert not spills, f"instantiations spilling to scratch: {spills[:8]}"
