"""GPU parity: librmsq (through the C ABI) against the CPU oracle on the five workloads.

Every row of every batch is compared, at every token count the workloads name (up to 16384 x
7168 and every per-group variant there); the oracle's rows are split over the host's threads.
"""
import functools

import numpy as np
import pytest

import oracle as O
from rmsnorm_quantization_amd import synth
from tests import gpu_harness as GH
from tests.parity import compare

pytestmark = pytest.mark.gpu

@pytest.fixture(scope="module", autouse=True)
def _gpu():
    GH.require_gpu()


@functools.lru_cache(maxsize=None)
def static_scale_w1():
    """Static scale of workload 1: max|y| of the fixed 512x4096 warm-up batch over 448,
    computed by the oracle."""
    xw, rw = synth.make_warmup(1)
    _, _, w = synth.make_inputs(1, 1)
    y = O.rms_y(synth.bits(xw), synth.bits(rw), synth.bits(w), synth.WORKLOADS[1].eps)
    return float(np.abs(y).max() / np.float32(448))


def fp4_global_scale(xb, rb, wb, eps):
    y = GH.rms_y_threaded(xb, rb, wb, eps)
    return float(np.float32(448 * 6) / np.abs(y).max())


def _check(workload, T, H, mode, scale_in=0.0, group_size=0, flags=0, label=""):
    eps = synth.WORKLOADS[workload].eps
    xd, rd, wd, xb, rb, wb = GH.workload_inputs(workload, T, H)
    print(f"[parity] workload={workload} T={T} H={H} mode={mode} G={group_size} flags={flags} "
          f"{label} rows=all", flush=True)
    gpu = GH.run(mode, xd, rd, wd, eps, scale_in=scale_in if mode in (O.FP8_STATIC,
                                                                      O.FP4_BLOCK16) else None,
                 group_size=group_size, flags=flags)
    ref = GH.oracle_threaded(mode, xb, rb, wb, eps, scale_in=scale_in, group_size=group_size,
                             flags=flags)
    raw = None
    if (mode == O.FP8_GROUP and flags & (O.SCALE_E8M0 | O.SCALE_E8M0_U8)
            and not np.array_equal(gpu["scales"], ref["scales"])):
        raw = GH.oracle_threaded(mode, xb, rb, wb, eps, group_size=group_size,
                                 flags=flags & O.SCALE_COLMAJOR, want_pre=False)["scales"]
    rep = compare(mode, gpu, ref, T=T, H=H, group_size=group_size, flags=flags,
                  y_ref=GH.y_ref_norm(xb, rb, wb, eps), scale_in=scale_in,
                  raw_group_scales=raw)
    print(f"[parity]   {rep}", flush=True)
    return rep


# ---------------------------------------------------------------- workload 0
def test_w0_rmsnorm_fp8_static():
    rep = _check(0, 16, 4096, O.FP8_STATIC, scale_in=0.05)
    assert rep.code_mismatch == 0


# ---------------------------------------------------------------- workload 1
@pytest.mark.parametrize("T", [1, 64, 512, 4096])
def test_w1_add_rmsnorm_fp8_static(T):
    _check(1, T, 4096, O.FP8_STATIC, scale_in=static_scale_w1())


# ---------------------------------------------------------------- workload 2
@pytest.mark.parametrize("T", [1, 256, 2048, 8192])
def test_w2_add_rmsnorm_fp8_per_token(T):
    _check(2, T, 8192, O.FP8_TOKEN)


# ---------------------------------------------------------------- workload 3
W3_FLAGS = [0, O.SCALE_COLMAJOR, O.SCALE_E8M0, O.SCALE_COLMAJOR | O.SCALE_E8M0]


@pytest.mark.parametrize("H", [5120, 7168])
@pytest.mark.parametrize("G", [128, 64])
@pytest.mark.parametrize("flags", W3_FLAGS)
@pytest.mark.parametrize("T", [1, 128, 1024])
def test_w3_add_rmsnorm_fp8_per_group(T, H, G, flags):
    _check(3, T, H, O.FP8_GROUP, group_size=G, flags=flags)


@pytest.mark.parametrize("H", [5120, 7168])
@pytest.mark.parametrize("G", [128, 64])
@pytest.mark.parametrize("flags", W3_FLAGS + [O.SCALE_E8M0_U8, O.SCALE_COLMAJOR | O.SCALE_E8M0_U8])
def test_w3_full_size_16384(H, G, flags):
    _check(3, 16384, H, O.FP8_GROUP, group_size=G, flags=flags)


@pytest.mark.parametrize("flags", [O.SCALE_E8M0_U8, O.SCALE_COLMAJOR | O.SCALE_E8M0_U8])
def test_w3_e8m0_bytes(flags):
    _check(3, 128, 7168, O.FP8_GROUP, group_size=128, flags=flags)


# ---------------------------------------------------------------- workload 4
@pytest.mark.parametrize("T", [1, 32, 256, 4096])
def test_w4_add_rmsnorm_fp4_block16(T):
    _, _, _, xb, rb, wb = GH.workload_inputs(4, T, 2048)
    gs = fp4_global_scale(xb, rb, wb, synth.WORKLOADS[4].eps)
    _check(4, T, 2048, O.FP4_BLOCK16, scale_in=gs, group_size=16)


# ---------------------------------------------------------------- batch-size launch rule
# Batches in flight all at once with 1536- or 2048-wide rows: the per-token scheme runs one wave
# per row (64 x 3 or 64 x 4), the others their per-H default (64 x 3 or 128 x 2); every scheme
# at those default shapes against the oracle.
@pytest.mark.parametrize("T,H", [(1024, 1536), (2048, 2048)])
@pytest.mark.parametrize("mode,G,flags", [(O.FP8_STATIC, 0, 0), (O.FP8_TOKEN, 0, 0),
                                          (O.FP8_GROUP, 128, O.SCALE_COLMAJOR),
                                          (O.FP8_GROUP, 64, O.SCALE_E8M0),
                                          (O.FP4_BLOCK16, 16, 0)])
def test_one_wave_row_default_shapes(T, H, mode, G, flags):
    from rmsnorm_quantization_amd import binding as B

    want = (64, 3, 1, 0) if H == 1536 else (64, 4, 1, 0) if mode == O.FP8_TOKEN else (128, 2, 1, 0)
    assert B.rmsq_query_launch(mode, T, H, G)[0].as_tuple() == want
    _, _, _, xb, rb, wb = GH.workload_inputs(4, T, H)
    scale_in = 0.0
    if mode == O.FP4_BLOCK16:
        scale_in = fp4_global_scale(xb, rb, wb, synth.WORKLOADS[4].eps)
    elif mode == O.FP8_STATIC:
        scale_in = 0.01
    rep = _check(4, T, H, mode, scale_in=scale_in, group_size=G, flags=flags, label="one-wave")
    assert rep.code_mismatch == 0
