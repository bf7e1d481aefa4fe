"""Pin gfx950's conversion instructions, as the kernels use them, against the oracle's formats.

rmsq_convert runs the kernels' own helpers (clamp + v_cvt_pk_fp8_f32, and v_cvt_pk_fp8_f32
alone over |v| <= 464; v_cvt_scalef32_pk_fp4_f32 with a unit scale and the nibble packing;
v_cvt_pk_bf16_f32) over arbitrary f32 inputs.  Checked on every bf16 value, every rounding midpoint of the target
format and +-1 ulp around it, saturation, signed zeros, and a large random sample of f32 bit
patterns.  NaN inputs are outside the contract and are left out.
"""
import numpy as np
import pytest
import torch

import oracle as O
from rmsnorm_quantization_amd import binding as B
from tests import gpu_harness as GH

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    GH.require_gpu()


def _pad8(v):
    n = (-len(v)) % 8
    return np.concatenate([v, np.zeros(n, np.float32)]).astype(np.float32)


def _midpoints(table):
    t = np.sort(np.unique(table[np.isfinite(table) & (table >= 0)].astype(np.float64)))
    mids = ((t[:-1] + t[1:]) / 2).astype(np.float32)
    lo, hi = np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(np.inf))
    v = np.concatenate([t.astype(np.float32), mids, lo, hi])
    return np.concatenate([v, -v])


def _inputs(table, sat):
    rng = np.random.default_rng(1234)
    bf = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    rnd = rng.integers(0, 2 ** 32, 2_000_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    near = (rng.standard_normal(1_000_000) * sat / 3).astype(np.float32)
    special = np.array([0.0, -0.0, sat, -sat, sat * 1.01, -sat * 1.01, 1e30, -1e30, np.inf,
                        -np.inf, 1e-40, -1e-40], np.float32)
    v = np.concatenate([bf, rnd, near, _midpoints(table), special])
    return _pad8(v[~np.isnan(v)])


def _convert(fmt, v):
    vin = torch.from_numpy(v).to("cuda")
    n = v.size
    nbytes = {B.RMSQ_CVT_E4M3: n, B.RMSQ_CVT_E4M3_IN_RANGE: n, B.RMSQ_CVT_E2M1: n // 2,
              B.RMSQ_CVT_BF16: 2 * n, B.RMSQ_CVT_INV_SQRT: 4 * n}[fmt]
    g = GH.Guarded(nbytes)
    print(f"[convert] fmt={fmt} n={n}", flush=True)
    B.rmsq_convert(fmt, vin, g.data, n)
    torch.cuda.synchronize()
    g.check("convert out")
    return g.data.cpu().numpy()


def test_e4m3_conversion_matches_oracle():
    v = _inputs(O.e4m3_table(), 448.0)
    got = _convert(B.RMSQ_CVT_E4M3, v)
    exp = O.e4m3_encode(v)
    bad = got != exp
    assert not bad.any(), f"{bad.sum()} mismatches, e.g. {v[bad][:8]} -> {got[bad][:8]} vs {exp[bad][:8]}"


def test_e4m3_in_range_conversion_matches_oracle():
    """The per-group scheme converts without a clamp: its inputs stay within
    448 (1 + 2^-20).  Up to 464 (the midpoint between 448 and the step above it) the codes are
    the saturating encoder's; every value in (448, 464], and the first values past 448 in f32
    steps, included.  Past 464 the instruction gives the NaN code of the value's sign -- the
    reason the bound matters."""
    v = _inputs(O.e4m3_table(), 448.0)
    v = v[np.abs(v) <= 464.0]
    i = np.arange(1, 4097, dtype=np.uint32)
    above = (np.uint32(np.float32(448.0).view(np.uint32)) + i).view(np.float32)
    edge = np.array([464.0, np.nextafter(np.float32(464.0), np.float32(0)), 456.0, 463.5,
                     448.0 * (1 + 2.0 ** -20)], np.float32)
    v = _pad8(np.concatenate([v, above[above <= 464.0], edge, -above[above <= 464.0], -edge]))
    got = _convert(B.RMSQ_CVT_E4M3_IN_RANGE, v)
    exp = O.e4m3_encode(v)
    bad = got != exp
    assert not bad.any(), f"{bad.sum()} mismatches, e.g. {v[bad][:8]} -> {got[bad][:8]} vs {exp[bad][:8]}"
    past = _pad8(np.array([np.nextafter(np.float32(464.0), np.float32(1e9)), 480.0, 1e30,
                           -np.nextafter(np.float32(464.0), np.float32(1e9)), -480.0], np.float32))
    got = _convert(B.RMSQ_CVT_E4M3_IN_RANGE, past)[:5]
    assert list(got) == [0x7F, 0x7F, 0x7F, 0xFF, 0xFF]


def test_e2m1_conversion_and_packing_match_oracle():
    v = _inputs(O.e2m1_table(), 6.0)
    got = _convert(B.RMSQ_CVT_E2M1, v)
    exp = O.e2m1_encode(v)
    nib = O.unpack_fp4(got)
    bad = nib != exp
    assert not bad.any(), f"{bad.sum()} mismatches, e.g. {v[bad][:8]} -> {nib[bad][:8]} vs {exp[bad][:8]}"


def test_bf16_rounding_matches_oracle():
    rng = np.random.default_rng(99)
    hi = np.arange(65536, dtype=np.uint32) << 16
    ties = np.concatenate([hi | 0x8000, hi | 0x7FFF, hi | 0x8001]).view(np.float32)
    rnd = rng.integers(0, 2 ** 32, 2_000_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    v = np.concatenate([ties, rnd])
    v = _pad8(v[~np.isnan(v)])
    got = _convert(B.RMSQ_CVT_BF16, v).view(np.uint16)
    exp = O.f32_to_bf16(v)
    bad = got != exp
    assert not bad.any(), f"{bad.sum()} mismatches, e.g. {v[bad][:8]} -> {got[bad][:8]} vs {exp[bad][:8]}"


def test_inverse_rms_sequence_matches_definition():
    """The kernels' inverse RMS of m (a refined hardware estimate, with the exact binary64
    sequence where the estimate's binary32 rounding is in doubt) against the definition the
    oracle follows: the binary64 root and quotient, each correctly rounded (numpy's binary64
    sqrt and division are), rounded once to binary32.  Inputs span every binary32 binade of
    positive m, and include every value of a large random sample whose binary64 result lies
    within 2^-38 of a binary32 rounding boundary, which the kernels resolve the slow way."""
    rng = np.random.default_rng(2024)
    bits = rng.integers(1, 0x7F800000, 4_000_000, dtype=np.uint64).astype(np.uint32)
    m = bits.view(np.float32)
    exact = 1.0 / np.sqrt(m.astype(np.float64))
    f = exact.astype(np.float32)
    # distance to the nearest binary32 rounding boundary, relative to the value
    up = np.nextafter(f, np.float32(np.inf)).astype(np.float64)
    dn = np.nextafter(f, np.float32(0)).astype(np.float64)
    fd = f.astype(np.float64)
    gap = np.minimum(np.abs(exact - (fd + up) / 2), np.abs(exact - (fd + dn) / 2)) / exact
    hard = m[gap < 2.0 ** -38]
    assert hard.size > 100
    special = np.array([np.float32(2.0 ** -149), np.finfo(np.float32).tiny, 1.0, 2.0, 4.0, 0.5,
                        1e-5, 1e-6, np.finfo(np.float32).max], np.float32)
    powers = (2.0 ** np.arange(-149, 128)).astype(np.float32)
    v = _pad8(np.concatenate([m[:1_000_000], hard, special, powers]).astype(np.float32))
    v[v == 0] = 1.0
    got = _convert(B.RMSQ_CVT_INV_SQRT, v).view(np.float32)
    exp = (1.0 / np.sqrt(v.astype(np.float64))).astype(np.float32)
    bad = got.view(np.uint32) != exp.view(np.uint32)
    assert not bad.any(), f"{bad.sum()} mismatches, e.g. {v[bad][:8]} -> {got[bad][:8]} vs {exp[bad][:8]}"
