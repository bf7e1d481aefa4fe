"""Pins for the oracle's FP4 block-16 quantization with the global scale taken from the batch.

The PR #51925 summary's test derives an NVFP4 global scale as the largest e4m3 magnitude times
the largest e2m1 magnitude (448 * 6) over a tensor's absmax; the dynamic form applies that to the
normalized batch y itself, then quantizes exactly as the static FP4 path does.  Pinned by
composition with the already-pinned y and static FP4 path, by what the format forces on the block
that holds the batch's absmax (its scale is e4m3's largest, its code e2m1's largest), by the
dequantization error bound, and by the zero and tiny-batch special cases.
"""
import numpy as np
import pytest

from tests.test_oracle_pins import bf16_bits

FLT_MAX = np.float32(np.finfo(np.float32).max)


def _inputs(T, H, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    x = bf16_bits(rng.standard_normal((T, H)) * scale)
    r = bf16_bits(rng.standard_normal((T, H)) * scale)
    w = bf16_bits(rng.uniform(0.5, 1.5, H))
    return x, r, w


def test_global_scale_special_cases(orc):
    assert orc.fp4_global_scale(1.0) == 2688.0 and orc.fp4_global_scale(448.0) == 6.0
    assert orc.fp4_global_scale(0.0) == FLT_MAX
    tiny = np.float32(2688.0) / FLT_MAX  # below this the quotient exceeds FLT_MAX
    assert orc.fp4_global_scale(np.nextafter(tiny, np.float32(0)) / 2) == FLT_MAX
    rng = np.random.default_rng(1)
    a = (rng.uniform(-30, 30, 1000)).astype(np.float32)
    a = np.exp2(a).astype(np.float32)
    got = np.array([orc.fp4_global_scale(v) for v in a], np.float32)
    assert np.array_equal(got, np.float32(2688.0) / a)  # numpy's IEEE f32 division


@pytest.mark.parametrize("residual", [True, False])
def test_composes_with_the_static_path(orc, residual):
    x, r, w = _inputs(9, 2048, 2)
    r = r if residual else None
    d = orc.fused_fp4_dynamic(x, r, w, 1e-6)
    y = orc.rms_y(x, r, w, 1e-6)
    gs = d["global_scale"]
    assert gs == orc.fp4_global_scale(np.abs(y).max())
    st = orc.fused(x, r, w, 1e-6, orc.FP4_BLOCK16, scale_in=float(gs), group_size=16)
    assert np.array_equal(d["q"], st["q"]) and np.array_equal(d["scales"], st["scales"])
    if residual:
        assert np.array_equal(d["residual_out"], st["residual_out"])


def test_block_of_the_absmax_takes_the_largest_codes(orc):
    """amax * gs / 6 is 448 up to two f32 roundings, which e4m3 rounds to 448 (0x7E); that
    element then scales to 6 up to rounding: e2m1's largest magnitude (code 7)."""
    for seed in range(5):
        x, r, w = _inputs(7, 1024, 10 + seed, scale=float(2.0 ** (4 * seed - 8)))
        d = orc.fused_fp4_dynamic(x, r, w, 1e-6)
        y = orc.rms_y(x, r, w, 1e-6)
        t, i = np.unravel_index(np.argmax(np.abs(y)), y.shape)
        assert d["scales"][t, i // 16] == 0x7E
        nib = (d["q"][t, i // 2] >> (4 * (i % 2))) & 0xF
        assert nib == (0xF if y[t, i] < 0 else 0x7)
        assert d["scales"].max() <= 0x7E  # no block scale above 448


def test_dequantization_error_bound(orc):
    """value = e2m1 * decode(sf) / gs is within decode(sf) / gs of y: half of e2m1's widest step
    (4 -> 6), which also covers the clamp to 6 after a block scale rounded down by e4m3."""
    x, r, w = _inputs(16, 2048, 3)
    d = orc.fused_fp4_dynamic(x, r, w, 1e-6)
    y = orc.rms_y(x, r, w, 1e-6)
    gs = np.float64(d["global_scale"])
    sf = np.asarray(orc.e4m3_decode(np.arange(256, dtype=np.uint8)), np.float64)[d["scales"]]
    e2 = np.asarray(orc.e2m1_decode(np.arange(16, dtype=np.uint8)), np.float64)
    lo, hi = d["q"] & 0xF, d["q"] >> 4
    codes = np.empty(y.shape, np.int64)
    codes[:, 0::2], codes[:, 1::2] = lo, hi
    step = np.repeat(sf, 16, axis=1) / gs
    deq = e2[codes] * step
    assert np.all(np.abs(deq - y) <= step * (1 + 1e-6))


def test_zero_batch_and_binary16(orc):
    H = 256
    z = np.zeros((3, H), np.uint16)
    w = bf16_bits(np.ones(H))
    d = orc.fused_fp4_dynamic(z, None, w, 1e-6)
    assert d["global_scale"] == FLT_MAX
    assert not d["q"].any() and not d["scales"].any()
    rng = np.random.default_rng(4)
    f16 = (lambda a: np.asarray(a, np.float32).astype(np.float16).view(np.uint16))
    x, r, w16 = f16(rng.standard_normal((5, H))), f16(rng.standard_normal((5, H))), f16(
        rng.uniform(0.5, 1.5, H))
    d = orc.fused_fp4_dynamic(x, r, w16, 1e-6, flags=orc.INPUT_F16)
    y = orc.rms_y(x, r, w16, 1e-6, f16=True)
    gs = d["global_scale"]
    assert gs == orc.fp4_global_scale(np.abs(y).max())
    st = orc.fused(x, r, w16, 1e-6, orc.FP4_BLOCK16, scale_in=float(gs), group_size=16,
                   flags=orc.INPUT_F16)
    assert np.array_equal(d["q"], st["q"]) and np.array_equal(d["scales"], st["scales"])
    with pytest.raises(ValueError):
        orc.fused_fp4_dynamic(x, r, w16, 1e-6, flags=orc.SCALE_COLMAJOR)
