"""Build librmsq.so (the HIP kernels + C ABI) in-tree for gfx950 with hipcc, and beside it
librmsq_probe.so (the memory-only reference kernel of include/rmsq_probe.h, for measurement).

Flags that matter for results:
  -ffp-contract=off                          no FMA contraction of the binary32 steps
  -fhip-fp32-correctly-rounded-divide-sqrt   IEEE f32 division (scales, reciprocals)
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                             no packed-f32 VALU instructions
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
# translation units of librmsq, compiled in parallel and linked into one shared library: the
# host side, and the kernel instantiation tables (rmsq_kernel_table.hpp)
SRC = [os.path.join(PKG, "csrc", f) for f in ("rmsq.hip", "table_fused_bf16.hip",
                                              "table_fused_f16.hip", "table_act.hip",
                                              "table_misc.hip", "table_rope_f16.hip")]
KERNEL_SOURCES = [os.path.join(PKG, "csrc", "rmsq_device.hpp"),
                  os.path.join(PKG, "csrc", "rmsq_kernels.hpp"),
                  os.path.join(PKG, "csrc", "rmsq_kernel_table.hpp")]
DEPS = SRC + KERNEL_SOURCES + [os.path.join(ROOT, "include", "rmsq.h")]
LIB = os.path.join(PKG, "librmsq.so")
PROBE_SRC = [os.path.join(PKG, "csrc", "rmsq_probe.hip")]
PROBE_DEPS = PROBE_SRC + [os.path.join(ROOT, "include", "rmsq_probe.h")]
PROBE_LIB = os.path.join(PKG, "librmsq_probe.so")
ARCH = "gfx950"


def hipcc():
    for c in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.sep not in c or os.path.exists(c):
            return c
    return "hipcc"


def command(out=LIB, extra=(), src=None):
    """The hipcc command line that builds `out` from `src` (default: every unit of librmsq)."""
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-fvisibility=hidden", "-Wall", "-I", os.path.join(ROOT, "include"),
        *extra, *(SRC if src is None else src), "-o", out,
    ]


def _run(cmd, verbose, what):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed to build {what}")


def build_library(verbose: bool = False) -> str:
    """Compile every unit to an object in parallel (same flags as command()), then link."""
    import tempfile
    from concurrent.futures import ThreadPoolExecutor

    with tempfile.TemporaryDirectory(prefix="rmsq_build_") as tmp:
        objs = [os.path.join(tmp, os.path.basename(src) + ".o") for src in SRC]
        jobs = []
        for src, obj in zip(SRC, objs):
            cmd = command(obj, src=[src])
            cmd.remove("-shared")
            cmd.insert(1, "-c")
            jobs.append((cmd, os.path.basename(src)))
        workers = max(1, min(len(jobs), os.cpu_count() or 1))
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(lambda j: _run(j[0], verbose, j[1]), jobs))
        link = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", LIB + ".tmp"]
        _run(link, verbose, "librmsq.so (link)")
    os.replace(LIB + ".tmp", LIB)
    return LIB


def build_probe_library(verbose: bool = False) -> str:
    cmd = command(PROBE_LIB + ".tmp", src=PROBE_SRC)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed to build librmsq_probe.so")
    os.replace(PROBE_LIB + ".tmp", PROBE_LIB)
    return PROBE_LIB


def probe_is_stale() -> bool:
    if not os.path.exists(PROBE_LIB):
        return True
    t = os.path.getmtime(PROBE_LIB)
    return any(os.path.getmtime(p) > t for p in PROBE_DEPS)


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(p) > t for p in DEPS)


if __name__ == "__main__":
    print(build_library(verbose=True))
    print(build_probe_library(verbose=True))
