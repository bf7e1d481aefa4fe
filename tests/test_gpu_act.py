"""GPU parity for SiLU+Mul -> quantization against the oracle (vLLM docs "Fusion
torch.compile passes", section "SiLU+Mul + quantization").

The kernel evaluates silu with expf and the hardware reciprocal, a few ulp from the exactly
rounded activation the oracle computes, so codes may differ by one step where the scaled value
sits within ~1e-6 of a rounding midpoint; the comparison rule (tests/parity.py) bounds that.
"""
import functools

import numpy as np
import pytest
import torch

import oracle as O
from rmsnorm_quantization_amd import binding as B
from rmsnorm_quantization_amd import synth
from tests import gpu_harness as GH
from tests.parity import compare

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    GH.require_gpu()


@functools.lru_cache(maxsize=4)
def act_inputs(T, I):
    x = synth.make_act_inputs(5, T, I)
    return GH.to_dev(x), synth.bits(x)


@functools.lru_cache(maxsize=None)
def static_scale():
    a = O.silu_mul(synth.bits(synth.make_act_warmup(5)))
    return float(np.abs(a).max() / np.float32(448))


def _check(T, I, mode, scale_in=0.0, G=0, flags=0, launch=None, xb=None, xd=None):
    """Every row compared; the oracle's rows split over the host's threads."""
    if xd is None:
        xd, xb = act_inputs(T, I)
    print(f"[act] T={T} I={I} mode={mode} G={G} flags={flags} rows=all", flush=True)
    gpu = GH.run_act(mode, xd, scale_in=scale_in if mode in (O.FP8_STATIC, O.FP4_BLOCK16) else None,
                     group_size=G, flags=flags, launch=launch)
    ref = GH.oracle_act_threaded(mode, xb, scale_in=scale_in, group_size=G, flags=flags)
    raw = None
    if (mode == O.FP8_GROUP and flags & (O.SCALE_E8M0 | O.SCALE_E8M0_U8)
            and not np.array_equal(gpu["scales"], ref["scales"])):
        raw = GH.oracle_act_threaded(mode, xb, group_size=G, flags=flags & O.SCALE_COLMAJOR,
                                     want_pre=False)["scales"]
    rep = compare(mode, gpu, ref, T=T, H=I, group_size=G, flags=flags, scale_in=scale_in,
                  raw_group_scales=raw, y_ref=GH.y_ref_act(xb))
    print(f"[act]   {rep}", flush=True)
    return gpu, rep


@pytest.mark.parametrize("T", [1, 256, 4096])
def test_silu_mul_fp8_static(T):
    _check(T, 14336, O.FP8_STATIC, scale_in=static_scale())


@pytest.mark.parametrize("T", [1, 256, 4096])
def test_silu_mul_fp8_per_token(T):
    _check(T, 14336, O.FP8_TOKEN)


@pytest.mark.parametrize("G", [128, 64])
@pytest.mark.parametrize("flags", [0, O.SCALE_COLMAJOR, O.SCALE_E8M0,
                                   O.SCALE_COLMAJOR | O.SCALE_E8M0_U8])
@pytest.mark.parametrize("T", [1, 256, 4096])
def test_silu_mul_fp8_per_group(T, G, flags):
    _check(T, 14336, O.FP8_GROUP, G=G, flags=flags)


@pytest.mark.parametrize("T", [1, 256, 4096])
def test_silu_mul_fp4(T):
    xd, xb = act_inputs(T, 14336)
    a = O.silu_mul(xb if T <= 256 else xb[:256])
    gs = float(np.float32(448 * 6) / np.abs(a).max())
    _check(T, 14336, O.FP4_BLOCK16, scale_in=gs, G=16)


RAGGED = [(I, mode, G, scale) for I in (8, 16, 72, 520, 1152, 2880, 65536)
          for mode, G, scale in ((O.FP8_STATIC, 0, 0.01), (O.FP8_TOKEN, 0, 0.0),
                                 (O.FP8_GROUP, 64, 0.0), (O.FP4_BLOCK16, 16, 200.0))
          if not G or I % G == 0]


@pytest.mark.parametrize("I,mode,G,scale", RAGGED)
def test_silu_mul_ragged_sizes(I, mode, G, scale):
    T = 3 if I == 65536 else 29
    g = torch.Generator().manual_seed(I)
    x = (torch.randn((T, 2 * I), generator=g) * 3).to(torch.bfloat16)
    _check(T, I, mode, scale_in=scale, G=G, xb=synth.bits(x), xd=GH.to_dev(x))


@pytest.mark.parametrize("mode,G,scale", [(O.FP8_STATIC, 0, 0.01), (O.FP8_TOKEN, 0, 0.0),
                                          (O.FP8_GROUP, 128, 0.0), (O.FP4_BLOCK16, 16, 200.0)])
def test_silu_mul_every_launch_shape_identical(mode, G, scale):
    T, I = 21, 1024
    g = torch.Generator().manual_seed(3)
    x = (torch.randn((T, 2 * I), generator=g) * 2).to(torch.bfloat16)
    xd, xb = GH.to_dev(x), synth.bits(x)
    base, _ = _check(T, I, mode, scale_in=scale, G=G, xb=xb, xd=xd)
    n = 0
    if mode != O.FP8_TOKEN:  # row tiles: any tile width, including ones that do not divide I
        for tpr in (64, 128, 192, 256, 512, 1024):
            for vpt in (1, 2, 4):
                l = B.rmsq_launch(tpr, vpt, 1, B.RMSQ_LAUNCH_ROW_TILES)
                got = GH.run_act(mode, xd, scale_in=scale if mode in (O.FP8_STATIC,
                                                                      O.FP4_BLOCK16) else None,
                                 group_size=G, launch=l)
                assert np.array_equal(got["q"], base["q"]), l.as_tuple()
                if base["scales"] is not None:
                    assert np.array_equal(got["scales"], base["scales"]), l.as_tuple()
                n += 1
    for tpr in (64, 128, 192, 256, 512, 1024):
        for vpt in range(1, 9):
            if tpr * vpt * 8 < I:
                continue
            for rpb in (1, 4):
                if rpb * tpr > 1024:
                    continue
                l = B.rmsq_launch(tpr, vpt, rpb, 0)
                got = GH.run_act(mode, xd, scale_in=scale if mode in (O.FP8_STATIC,
                                                                      O.FP4_BLOCK16) else None,
                                 group_size=G, launch=l)
                assert np.array_equal(got["q"], base["q"]), l.as_tuple()
                if base["scales"] is not None:
                    assert np.array_equal(got["scales"], base["scales"]), l.as_tuple()
                n += 1
    assert n > 10


def test_silu_mul_extremes():
    """Very negative gates (tiny activations), very positive gates (silu -> g), zeros."""
    T, I = 4, 256
    g = torch.Generator().manual_seed(5)
    x = torch.randn((T, 2 * I), generator=g)
    x[0, :I] = -60.0
    x[1, :I] = 100.0
    x[2] = 0.0
    x[3, :I] = torch.linspace(-30, 30, I)
    x = x.to(torch.bfloat16)
    for mode, G, scale in ((O.FP8_STATIC, 0, 0.5), (O.FP8_TOKEN, 0, 0.0), (O.FP8_GROUP, 128, 0.0),
                           (O.FP4_BLOCK16, 16, 20.0)):
        _check(T, I, mode, scale_in=scale, G=G, xb=synth.bits(x), xd=GH.to_dev(x))


def test_silu_mul_subnormal_rows_quantize_to_zero():
    """Gates of -100 give activations near 1e-42, below f32's normal range: the relative scale
    tolerance is meaningless there, but every code must still be a zero and scales tiny."""
    T, I = 2, 256
    x = torch.ones((T, 2 * I))
    x[:, :I] = -100.0
    x = GH.to_dev(x.to(torch.bfloat16))
    for mode, G, scale in ((O.FP8_STATIC, 0, 0.5), (O.FP8_TOKEN, 0, 0.0), (O.FP8_GROUP, 128, 0.0),
                           (O.FP4_BLOCK16, 16, 20.0)):
        out = GH.run_act(mode, x, scale_in=scale if mode in (O.FP8_STATIC, O.FP4_BLOCK16) else None,
                         group_size=G)
        mag = (O.unpack_fp4(out["q"]) & 7) if mode == O.FP4_BLOCK16 else (out["q"] & 0x7F)
        if mode in (O.FP8_STATIC, O.FP4_BLOCK16):
            assert np.all(mag == 0)
        if mode in (O.FP8_TOKEN, O.FP8_GROUP):
            assert np.all(np.abs(out["scales"]) < 1e-40)


def test_silu_mul_helper_matches_entry_point():
    xd, xb = act_inputs(256, 14336)
    q, s = B.silu_and_mul_quant(xd, B.RMSQ_FP8_GROUP, group_size=128, col_major=True)
    torch.cuda.synchronize()
    ref = GH.run_act(O.FP8_GROUP, xd, group_size=128, flags=O.SCALE_COLMAJOR)
    assert np.array_equal(q.view(torch.uint8).cpu().numpy(), ref["q"])
    assert np.array_equal(s.cpu().numpy(), ref["scales"])


def test_row_tiles_rejected_where_invalid():
    xd, _ = act_inputs(1, 14336)
    q = torch.empty((1, 14336), dtype=torch.uint8, device="cuda")
    s = torch.empty((1,), dtype=torch.float32, device="cuda")
    tiles = B.rmsq_launch(256, 2, 1, B.RMSQ_LAUNCH_ROW_TILES)
    assert B.rmsq_silu_mul_quant(xd, B.RMSQ_FP8_TOKEN, None, q, s, launch=tiles,
                                 check=False) == B.RMSQ_EINVAL  # per-token needs whole rows
    sc = torch.ones(1, device="cuda")
    bad = B.rmsq_launch(256, 2, 2, B.RMSQ_LAUNCH_ROW_TILES)
    assert B.rmsq_silu_mul_quant(xd, B.RMSQ_FP8_STATIC, sc, q, None, launch=bad,
                                 check=False) == B.RMSQ_EINVAL  # rows_per_block must be 1
    x = torch.zeros((4, 2048), dtype=torch.bfloat16, device="cuda")
    w = torch.ones(2048, dtype=torch.bfloat16, device="cuda")
    q2 = torch.empty((4, 2048), dtype=torch.uint8, device="cuda")
    assert B.rmsq_fused(x, None, w, 1e-6, B.RMSQ_FP8_STATIC, sc, q2, None, None, launch=tiles,
                        check=False) == B.RMSQ_EINVAL  # the norm needs whole rows
    torch.cuda.synchronize()
