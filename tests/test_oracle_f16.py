"""Pins for the oracle's IEEE binary16 input path (CPU only).

The fused ops of the pages take the model's activation dtype, and the pages require x and the
weight to share it; besides bf16 that is IEEE half precision.  The reading is the bf16 path with
binary16 in its place: the residual sum rounded to binary16 (nearest even, overflow to infinity)
is the new residual and what is normalized; everything after that (f32 y, quantizers) is
unchanged.  Pinned against numpy's binary16 conversions (an independent implementation), torch's
rms_norm in float64 and the already-pinned quantizers.
"""
import numpy as np
import pytest
import torch

from tests.test_oracle_pins import torch_e4m3


def f16_bits(a):
    return np.asarray(a, np.float32).astype(np.float16).view(np.uint16)


def test_decode_every_pattern(orc):
    bits = np.arange(65536, dtype=np.uint16)
    got = orc.f16_to_f32(bits)
    want = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


def test_encode_matches_numpy(orc):
    finite = np.arange(0x7C00, dtype=np.uint16)
    vals = finite.view(np.float16).astype(np.float32)
    mids = ((vals[:-1].astype(np.float64) + vals[1:]) / 2).astype(np.float32)  # exact in f32
    near = np.concatenate([np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))])
    over = np.linspace(65000, 70000, 20001, dtype=np.float32)
    rng = np.random.default_rng(16)
    rand = rng.integers(0, 1 << 32, 2_000_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    rand = rand[~np.isnan(rand)]
    v = np.concatenate([vals, mids, near, over, rand, [np.inf, 65519.996, 65520.0, 65520.004]])
    v = np.concatenate([v, -v]).astype(np.float32)
    with np.errstate(over="ignore"):
        want = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(orc.f32_to_f16(v), want)
    # ties go to the even code: 1 + 2^-11 lies halfway between 1 and 1 + 2^-10
    assert orc.f32_to_f16(np.float32(1 + 2.0 ** -11)) == 0x3C00
    assert orc.f32_to_f16(np.float32(1 + 3 * 2.0 ** -11)) == 0x3C02


def _inputs(T, H, seed, scale=3.0):
    rng = np.random.default_rng(seed)
    x = f16_bits(rng.standard_normal((T, H)) * scale)
    r = f16_bits(rng.standard_normal((T, H)) * scale)
    w = f16_bits(rng.uniform(0.5, 1.5, H))
    return x, r, w


def test_residual_sum_rounded_to_binary16(orc):
    x, r, w = _inputs(4, 256, 1)
    # large residuals so that the f32 sum needs rounding and some sums overflow binary16
    r[0, :8] = f16_bits([60000, -60000, 40000, 1e-7, 3e-8, 65504, -65504, 2048])
    x[0, :8] = f16_bits([10000, -10000, 30000, 1e-7, 2e-8, 16, -16, 1])
    out = orc.fused(x, r, w, 1e-6, orc.FP8_TOKEN, flags=orc.INPUT_F16)
    with np.errstate(over="ignore"):
        want = (x.view(np.float16).astype(np.float32) + r.view(np.float16).astype(np.float32)
                ).astype(np.float16).view(np.uint16)
    assert np.array_equal(out["residual_out"], want)
    assert out["residual_out"][0, 0] == 0x7C00 and out["residual_out"][0, 1] == 0xFC00


def test_normalized_rows_match_torch_float64(orc):
    x, r, w = _inputs(6, 512, 2)
    y = orc.rms_y(x, r, w, 1e-6, f16=True)
    h = orc.fused(x, r, w, 1e-6, orc.FP8_TOKEN, flags=orc.INPUT_F16)["residual_out"]
    ht = torch.from_numpy(h.view(np.float16).astype(np.float64))
    wt = torch.from_numpy(w.view(np.float16).astype(np.float64))
    ref = torch.nn.functional.rms_norm(ht, (512,), wt, 1e-6).numpy()
    assert np.allclose(y, ref, rtol=4e-7, atol=0)
    # the same 16-bit patterns read as bf16 give something else entirely
    assert not np.allclose(orc.rms_y(x, r, w, 1e-6), y)


def test_quantizers_compose(orc):
    x, r, w = _inputs(5, 256, 3)
    y = orc.rms_y(x, r, w, 1e-6, f16=True)
    tk = orc.fused(x, r, w, 1e-6, orc.FP8_TOKEN, flags=orc.INPUT_F16)
    s = np.abs(y).max(axis=1) / np.float32(448)
    assert np.array_equal(tk["scales"], s)
    assert np.array_equal(tk["q"], torch_e4m3(y * (np.float32(1) / s)[:, None]))
    st = orc.fused(x, r, w, 1e-6, orc.FP8_STATIC, scale_in=0.01, flags=orc.INPUT_F16)
    assert np.array_equal(st["q"], torch_e4m3(y * (np.float32(1) / np.float32(0.01))))
    for mode, G in ((orc.FP8_GROUP, 64), (orc.FP4_BLOCK16, 16)):
        f = orc.fused(x, r, w, 1e-6, mode, scale_in=300.0, group_size=G, flags=orc.INPUT_F16)
        for t in range(5):
            q, sc, _ = orc.quantize_row(y[t], mode, scale_in=300.0, group_size=G)
            assert np.array_equal(f["q"][t], q) and np.array_equal(f["scales"][t], sc)


@pytest.mark.parametrize("flags", [0, 1 << 8])
def test_plain_norm_ignores_missing_residual(orc, flags):
    x, _, w = _inputs(3, 128, 4)
    a = orc.fused(x, None, w, 1e-6, orc.FP8_TOKEN, flags=flags)
    z = np.zeros_like(x)  # +0 in both formats
    b = orc.fused(x, z, w, 1e-6, orc.FP8_TOKEN, flags=flags)
    assert np.array_equal(a["q"], b["q"]) and np.array_equal(b["residual_out"], x)


def test_silu_mul_on_binary16(orc):
    """SiLU+Mul on binary16 gate/up: torch's silu in float64 on the decoded values, rounded once
    to f32 (within the last bit of exp), and the quantizers compose as for bf16."""
    rng = np.random.default_rng(20)
    x = f16_bits(rng.standard_normal((4, 2 * 512)) * 4.0)
    a = orc.silu_mul(x, f16=True)
    xt = torch.from_numpy(x.view(np.float16).astype(np.float64))
    ref = (torch.nn.functional.silu(xt[:, :512]) * xt[:, 512:]).float().numpy()
    ulp = np.abs(a.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
    assert ulp.max() <= 1
    tk = orc.silu_mul_quant(x, orc.FP8_TOKEN, flags=orc.INPUT_F16)
    s = np.abs(a).max(axis=1) / np.float32(448)
    assert np.array_equal(tk["scales"], s)
    assert np.array_equal(tk["q"], torch_e4m3(a * (np.float32(1) / s)[:, None]))
    assert not np.array_equal(orc.silu_mul(x), a)  # read as bf16 it is another activation
