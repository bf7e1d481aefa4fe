"""Pins for the oracle's residual add + RMSNorm -> padded bf16 output (CPU only).

The operation (vLLM docs "Fusion torch.compile passes", section "RMSNorm + padding
(fuse_act_padding)"): residual add and RMSNorm fused with padding the hidden dimension (2880
for the model named there) up to the multiple a downstream GEMM needs.  The page gives neither
the output dtype nor the multiple; the readings are a bf16 output (the activation dtype) with a
caller-chosen padded row stride whose extra columns are zero.
"""
import numpy as np
import pytest
import torch

from rmsnorm_quantization_amd import synth
from tests.test_oracle_pins import bf16_bits


def _inputs(T, H, seed):
    rng = np.random.default_rng(seed)
    return (bf16_bits(rng.standard_normal((T, H))), bf16_bits(rng.standard_normal((T, H))),
            bf16_bits(rng.uniform(0.5, 1.5, H)))


@pytest.mark.parametrize("ld", [2880, 2944, 3072])
def test_pad_is_rounded_norm_then_zeros(orc, ld):
    x, r, w = _inputs(5, 2880, ld)
    out, rout = orc.rms_norm_pad(x, r, w, 1e-6, ld)
    y = orc.rms_y(x, r, w, 1e-6)
    ref = torch.from_numpy(y).to(torch.bfloat16)          # torch's own f32 -> bf16 rounding
    assert np.array_equal(out[:, :2880], synth.bits(ref))
    assert np.all(out[:, 2880:] == 0)
    assert np.array_equal(rout, orc.residual_add(x, r))


def test_pad_matches_torch_rms_norm(orc):
    x, r, w = _inputs(4, 2880, 1)
    out, rout = orc.rms_norm_pad(x, r, w, 1e-5, 3072)
    h = synth.from_bits(rout).double()
    ref = torch.nn.functional.rms_norm(h, (2880,), synth.from_bits(w).double(), 1e-5)
    got = synth.from_bits(out[:, :2880]).double()
    # bf16 output: within half a bf16 ulp of the float64 value plus the f32 steps
    assert torch.all((got - ref).abs() <= ref.abs() * (2.0 ** -8 + 2.0 ** -21))


def test_pad_without_residual_and_invalid(orc):
    x, _, w = _inputs(3, 64, 2)
    out, rout = orc.rms_norm_pad(x, None, w, 1e-6, 128)
    assert rout is None and np.all(out[:, 64:] == 0)
    with pytest.raises(ValueError):
        orc.rms_norm_pad(x, None, w, 1e-6, 32)  # out_ld < H
