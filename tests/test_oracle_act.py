"""Pins for the oracle's SiLU+Mul -> quantization (CPU only).

The operation (vLLM docs "Fusion torch.compile passes", section "SiLU+Mul + quantization
(fuse_act_quant)"): silu_and_mul on the gated up-projection, then FP8 static per-tensor, FP8
dynamic per-group (128/64) or FP4 quantization, without materializing the activation.  The page
does not spell out silu_and_mul; the reading is a = silu(g) * u with g the first and u the second
half of each row, silu(g) = g / (1 + exp(-g)).  Pinned against torch's own silu in float64,
closed forms, the half-split, and the already-pinned quantizers.
"""
import numpy as np
import pytest
import torch

from rmsnorm_quantization_amd import synth
from tests.test_oracle_pins import bf16_bits, torch_e4m3


def _rows(T, I, seed, scale=2.0):
    rng = np.random.default_rng(seed)
    return bf16_bits(rng.standard_normal((T, 2 * I)) * scale)


def test_silu_mul_matches_torch_float64(orc):
    x = _rows(64, 4096, 1, scale=4.0)
    a = orc.silu_mul(x)
    xt = synth.from_bits(x).double()
    g, u = xt[:, :4096], xt[:, 4096:]
    ref = (torch.nn.functional.silu(g) * u).float().numpy()  # float64 rounded once to f32
    ulp = np.abs(a.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
    assert ulp.max() <= 1
    assert (ulp != 0).mean() < 1e-4  # differences only from the last bit of exp


def test_closed_forms_and_split(orc):
    g = np.array([0.0, 0.0, 20.0, 20.0, 100.0, -100.0, 1.0, -1.0], np.float32)
    u = np.array([5.0, -3.0, 0.5, 1.0, 2.0, 2.0, 1.0, 1.0], np.float32)
    x = bf16_bits(np.concatenate([g, u]))[None, :]
    a = orc.silu_mul(x)[0]
    assert a[0] == 0.0 and a[1] == 0.0                        # silu(0) = 0
    assert np.isclose(a[2], 20.0 * 0.5, rtol=1e-7)             # silu(g) -> g for large g
    assert np.isclose(a[3], 20.0, rtol=1e-7)
    assert a[4] == np.float32(200.0)                           # exp(-100) vanishes in f32
    assert 0.0 > a[5] > -1e-40                                 # -100 * 2 * e^-100, subnormal
    sig1 = 1.0 / (1.0 + np.exp(-1.0))
    assert a[6] == np.float32(sig1) and a[7] == np.float32(-(1.0 - sig1))
    # swapping the halves changes the result: the gate is the first half
    xs = bf16_bits(np.concatenate([u, g]))[None, :]
    assert not np.allclose(orc.silu_mul(xs)[0], a)


def test_static_and_group_codes_compose(orc):
    x = _rows(6, 1024, 2)
    a = orc.silu_mul(x)
    scale = np.float32(0.011)
    st = orc.silu_mul_quant(x, orc.FP8_STATIC, scale_in=scale)
    assert np.array_equal(st["q"], torch_e4m3(a * (np.float32(1) / scale)))
    for G in (64, 128):
        gp = orc.silu_mul_quant(x, orc.FP8_GROUP, group_size=G)
        ag = a.reshape(6, 1024 // G, G)
        s = np.abs(ag).max(axis=2) / np.float32(448)
        assert np.array_equal(gp["scales"], s)
        assert np.array_equal(gp["q"], torch_e4m3(ag * (np.float32(1) / s)[:, :, None]).reshape(6, 1024))
        col = orc.silu_mul_quant(x, orc.FP8_GROUP, group_size=G, flags=orc.SCALE_COLMAJOR)
        assert np.array_equal(col["scales"], s.T) and np.array_equal(col["q"], gp["q"])


def test_token_and_fp4_equal_the_row_quantizer(orc):
    x = _rows(5, 512, 3)
    a = orc.silu_mul(x)
    tk = orc.silu_mul_quant(x, orc.FP8_TOKEN)
    f4 = orc.silu_mul_quant(x, orc.FP4_BLOCK16, scale_in=900.0, group_size=16)
    for t in range(5):
        q, s, _ = orc.quantize_row(a[t], orc.FP8_TOKEN)
        assert np.array_equal(tk["q"][t], q) and tk["scales"][t] == s[0]
        q4, s4, _ = orc.quantize_row(a[t], orc.FP4_BLOCK16, scale_in=900.0, group_size=16)
        assert np.array_equal(f4["q"][t], q4) and np.array_equal(f4["scales"][t], s4)
    assert np.all(np.any((tk["q"] & 0x7F) == 0x7E, axis=1))


def test_invalid(orc):
    x = _rows(2, 96, 4)
    with pytest.raises(ValueError):
        orc.silu_mul_quant(x, orc.FP8_GROUP, group_size=64)  # 96 % 64
    with pytest.raises(ValueError):
        orc.silu_mul_quant(x, orc.FP4_BLOCK16, group_size=8)
    assert orc.silu_mul_quant(x[:0], orc.FP8_TOKEN)["q"].shape == (0, 96)
