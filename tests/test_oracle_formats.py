"""Pins for the oracle's number formats (CPU only).

The pages name the formats (FP8 e4m3 codes with per-tensor/per-token/per-group scales, FP4
with block scales, E8M0 power-of-two scales; vLLM "Fusion torch.compile passes" section
"RMSNorm + quantization", PR #51925 summary "Motivation", blog "[vLLM] Compilation Fusion
Passes" section "Why this design") but never their bit layouts; the OCP definitions are used.
Each converter is pinned by (a) torch's own library conversion where torch has one, (b) the
closed-form set of representable values and rounding midpoints, and (c) hand-derived cases.
"""
import numpy as np
import pytest
import torch


def _torch_e4m3(v):
    """torch's float32 -> float8_e4m3fn conversion (round to nearest even, NaN above 464)."""
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def _f32_neighbours(v):
    v = np.asarray(v, np.float32)
    return np.nextafter(v, np.float32(-np.inf)), np.nextafter(v, np.float32(np.inf))


# ------------------------------------------------------------------ e4m3fn
def test_e4m3_decode_matches_torch_for_every_byte(orc):
    ours = orc.e4m3_table()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2  # 0x7F and 0xFF
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_e4m3_closed_form_values(orc):
    t = orc.e4m3_table()
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x01] == 2.0 ** -9 and t[0x07] == 7 * 2.0 ** -9  # subnormals
    assert t[0x08] == 2.0 ** -6  # smallest normal
    assert t[0x38] == 1.0 and t[0x6E] == 112.0 and t[0x76] == 224.0 and t[0x7B] == 352.0
    assert t[0x80] == 0.0 and np.signbit(t[0x80])
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0), "codes 0x00..0x7E must be strictly increasing"


def test_e4m3_every_code_round_trips(orc):
    t = orc.e4m3_table()
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    assert np.array_equal(orc.e4m3_encode(t[codes]), codes)


def test_e4m3_midpoints_go_to_even_code_and_neighbours_to_nearest(orc):
    t = orc.e4m3_table().astype(np.float64)
    lo = np.arange(0, 0x7E)
    mids = ((t[lo] + t[lo + 1]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (t[lo] + t[lo + 1]) / 2)  # exact in f32
    even = np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint8)
    assert np.array_equal(orc.e4m3_encode(mids), even)
    assert np.array_equal(orc.e4m3_encode(-mids), even | 0x80)
    below, above = _f32_neighbours(mids)
    assert np.array_equal(orc.e4m3_encode(below), lo.astype(np.uint8))
    assert np.array_equal(orc.e4m3_encode(above), (lo + 1).astype(np.uint8))


def test_e4m3_saturates_and_keeps_sign(orc):
    v = np.array([448, 449, 463.99, 464, 465, 1e6, 3e38, np.inf], np.float32)
    assert np.all(orc.e4m3_encode(v) == 0x7E)
    assert np.all(orc.e4m3_encode(-v) == 0xFE)
    assert orc.e4m3_encode(np.array([np.nan], np.float32))[0] == 0x7F
    z = orc.e4m3_encode(np.array([0.0, -0.0, -1e-9, 1e-9, 2.0 ** -10, -(2.0 ** -10)], np.float32))
    assert z.tolist() == [0x00, 0x80, 0x80, 0x00, 0x00, 0x80]


def test_e4m3_agrees_with_torch_on_dense_sample(orc):
    rng = np.random.default_rng(7)
    bf = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)  # every bf16 value
    rnd = rng.integers(0, 2 ** 32, size=1_500_000, dtype=np.uint64).astype(np.uint32).view(
        np.float32)
    v = np.concatenate([bf, rnd])
    v = v[np.isfinite(v)]
    ours = orc.e4m3_encode(v)
    ref = _torch_e4m3(v)
    big = np.abs(v) > 464  # torch returns NaN there, the oracle saturates
    assert np.array_equal(ours[~big], ref[~big])
    assert np.all((ours[big] & 0x7F) == 0x7E)


# ------------------------------------------------------------------ e2m1
E2M1_MAGS = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_decode_closed_form(orc):
    t = orc.e2m1_table()
    assert t[:8].tolist() == E2M1_MAGS
    assert t[8:].tolist() == [-m for m in E2M1_MAGS]
    assert np.signbit(t[8])


def test_e2m1_hand_table(orc):
    # midpoints between neighbours go to the even code; every magnitude maps to itself
    cases = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6,
             0.26: 1, 0.74: 1, 1.26: 3, 2.49: 4, 2.51: 5, 4.99: 6, 5.01: 7, 6.0: 7, 100.0: 7,
             0.0: 0, 0.1: 0, 0.4: 1, 1.2: 2, 2.8: 5, 3.6: 6, 4.4: 6, 5.2: 7}
    for m, c in zip(E2M1_MAGS, range(8)):
        cases[m] = c
    v = np.array(list(cases), np.float32)
    exp = np.array(list(cases.values()), np.uint8)
    assert np.array_equal(orc.e2m1_encode(v), exp)
    assert np.array_equal(orc.e2m1_encode(-v), exp | 0x8)


def test_e2m1_threshold_formulation(orc):
    """Independent formulation: count the rounding midpoints below |v|; at a midpoint, round
    up only when that lands on an even code."""
    rng = np.random.default_rng(11)
    v = np.concatenate([rng.uniform(-8, 8, 400_000).astype(np.float32),
                        (rng.standard_normal(100_000) * 0.3).astype(np.float32)])
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    a = np.abs(v).astype(np.float64)
    below = np.searchsorted(mids, a, side="left")    # midpoints strictly below a
    at = np.searchsorted(mids, a, side="right") - below  # 1 when a is a midpoint
    code = below + at * ((below + 1) % 2 == 0)
    code = code.astype(np.uint8) | np.where(np.signbit(v), 8, 0).astype(np.uint8)
    assert np.array_equal(orc.e2m1_encode(v), code)


# ------------------------------------------------------------------ bf16
def test_bf16_matches_torch_on_sample_and_all_ties(orc):
    rng = np.random.default_rng(3)
    hi = np.arange(65536, dtype=np.uint32) << 16
    ties = (hi | 0x8000).view(np.float32)               # exact halfway cases
    near = np.concatenate([(hi | 0x7FFF), (hi | 0x8001), (hi | 0x0001)]).view(np.float32)
    rnd = rng.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32).view(
        np.float32)
    v = np.concatenate([ties, near, rnd])
    ours = orc.f32_to_bf16(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(v)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.all((ours[nan] & 0x7F80) == 0x7F80) and np.all(ours[nan] & 0x007F)


def test_bf16_overflow_rule(orc):
    mx = np.float32(3.3895313892515355e38)  # largest finite bf16 (0x7F7F)
    assert orc.f32_to_bf16(np.array([mx], np.float32))[0] == 0x7F7F
    just_below_half = np.uint32(0x7F7F7FFF).view(np.float32)
    half = np.uint32(0x7F7F8000).view(np.float32)
    assert orc.f32_to_bf16(np.array([just_below_half], np.float32))[0] == 0x7F7F
    assert orc.f32_to_bf16(np.array([half], np.float32))[0] == 0x7F80  # rounds to infinity


# ------------------------------------------------------------------ E8M0
def test_e8m0_ceil_exponent(orc):
    rng = np.random.default_rng(5)
    s = np.abs(rng.standard_normal(200_000)).astype(np.float32) * np.float32(2.0) ** rng.integers(
        -60, 60, 200_000).astype(np.float32)
    s = s[s > 0]
    k = orc.e8m0_ceil_exp(s)
    assert np.all(np.ldexp(1.0, k) >= s.astype(np.float64))
    assert np.all(np.ldexp(1.0, k - 1) < s.astype(np.float64))
    p2 = np.ldexp(np.float32(1.0), np.arange(-126, 127)).astype(np.float32)
    assert np.array_equal(orc.e8m0_ceil_exp(p2), np.arange(-126, 127))
    assert orc.e8m0_ceil_exp(np.array([0.0], np.float32))[0] == -127
    tiny = np.array([2.0 ** -127, 2.0 ** -128, 2.0 ** -149, 2.0 ** -126 * 0.75], np.float32)
    assert orc.e8m0_ceil_exp(tiny).tolist() == [-127, -127, -127, -126]
