"""Pins for the oracle's QK-norm + RoPE (CPU only).

The operation (vLLM docs "Fusion torch.compile passes", section "QK Norm + RoPE"): for models
with per-head Q/K normalization, q and k are split out of the packed qkv tensor, each head is
RMS-normalized (q and k with their own weights), and the rotary embedding is applied -- the
fused op does this on qkv in one pass.  The page shows the unfused sequence only; readings:
in-place on the q and k heads, v untouched, full rotary over the head dimension, NeoX
(half-split) or GPT-J (interleaved) pairing, cos/sin from the model's f32 cache.
"""
import numpy as np
import pytest
import torch

from rmsnorm_quantization_amd import synth
from tests.test_oracle_pins import bf16_bits

HQ, HKV, D = 4, 2, 64


def _inputs(T, seed, scale=2.0):
    rng = np.random.default_rng(seed)
    qkv = bf16_bits(rng.standard_normal((T, (HQ + 2 * HKV) * D)) * scale)
    qw = bf16_bits(rng.uniform(0.5, 1.5, D))
    kw = bf16_bits(rng.uniform(0.5, 1.5, D))
    return qkv, qw, kw


def test_cache_matches_numpy_and_closed_forms(orc):
    cache = orc.rope_cache(512, 128, 10000.0)
    p = np.arange(512, dtype=np.float64)[:, None]
    th = p * 10000.0 ** (-2.0 * np.arange(64) / 128)
    ref = np.concatenate([np.cos(th), np.sin(th)], axis=1).astype(np.float32)
    ulp = np.abs(cache.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
    assert ulp.max() <= 1 and (ulp != 0).mean() < 1e-3
    assert np.all(cache[0, :64] == 1.0) and np.all(cache[0, 64:] == 0.0)
    assert np.allclose(cache[:, :64] ** 2 + cache[:, 64:] ** 2, 1.0, atol=1e-6)


def _heads(a, T):
    return a.reshape(T, HQ + 2 * HKV, D)


def test_position_zero_is_the_identity_rotation(orc):
    T = 3
    qkv, qw, kw = _inputs(T, 1)
    cache = orc.rope_cache(16, D)
    out = orc.qk_norm_rope(qkv, qw, kw, cache, np.zeros(T, np.int64), 1e-6, HQ, HKV, D)
    h_in, h_out = _heads(qkv, T), _heads(out, T)
    for hd in range(HQ + HKV):
        y = orc.rms_y(np.ascontiguousarray(h_in[:, hd]), None, qw if hd < HQ else kw, 1e-6)
        assert np.array_equal(h_out[:, hd], orc.f32_to_bf16(y))
    assert np.array_equal(h_out[:, HQ + HKV:], h_in[:, HQ + HKV:])  # v untouched


@pytest.mark.parametrize("neox", [True, False])
def test_quarter_turn_pairs_and_signs(orc, neox):
    """A cache with cos = 0, sin = 1 exactly rotates every pair by 90 degrees:
    (a, b) -> (-b, a); which elements pair up is the NeoX / GPT-J difference."""
    T = 2
    qkv, qw, kw = _inputs(T, 2)
    cache = np.zeros((4, D), np.float32)
    cache[:, D // 2:] = 1.0
    out = orc.qk_norm_rope(qkv, qw, kw, cache, np.full(T, 3, np.int64), 1e-6, HQ, HKV, D, neox)
    h_in, h_out = _heads(qkv, T), _heads(out, T)
    for hd in range(HQ + HKV):
        y = orc.rms_y(np.ascontiguousarray(h_in[:, hd]), None, qw if hd < HQ else kw, 1e-6)
        if neox:
            a, b = y[:, :D // 2], y[:, D // 2:]
            exp = np.concatenate([-b, a], axis=1)
        else:
            a, b = y[:, 0::2], y[:, 1::2]
            exp = np.empty_like(y)
            exp[:, 0::2], exp[:, 1::2] = -b, a
        assert np.array_equal(h_out[:, hd], orc.f32_to_bf16(exp.astype(np.float32)))


@pytest.mark.parametrize("neox", [True, False])
def test_matches_torch_float64(orc, neox):
    T = 8
    qkv, qw, kw = _inputs(T, 3)
    cache = orc.rope_cache(100, D, 10000.0)
    pos = np.random.default_rng(4).integers(0, 100, T)
    out = orc.qk_norm_rope(qkv, qw, kw, cache, pos, 1e-6, HQ, HKV, D, neox)
    x = synth.from_bits(qkv).double().reshape(T, HQ + 2 * HKV, D)
    c = torch.from_numpy(cache[pos, :D // 2]).double()[:, None, :]
    s = torch.from_numpy(cache[pos, D // 2:]).double()[:, None, :]
    res = []
    for hs, w in ((slice(0, HQ), qw), (slice(HQ, HQ + HKV), kw)):
        y = torch.nn.functional.rms_norm(x[:, hs], (D,), synth.from_bits(w).double(), 1e-6)
        if neox:
            a, b = y[..., :D // 2], y[..., D // 2:]
            res.append(torch.cat([a * c - b * s, b * c + a * s], dim=-1))
        else:
            a, b = y[..., 0::2], y[..., 1::2]
            r = torch.empty_like(y)
            r[..., 0::2], r[..., 1::2] = a * c - b * s, b * c + a * s
            res.append(r)
    ref = torch.cat(res, dim=1)
    got = synth.from_bits(out).double().reshape(T, HQ + 2 * HKV, D)[:, :HQ + HKV]
    # bf16 output: half a bf16 ulp of the value plus the f32 steps, relative to the pair size
    tol = ref.abs().amax(dim=-1, keepdim=True) * 2.0 ** -8 * 1.01
    assert torch.all((got - ref).abs() <= tol)


def test_q_and_k_weights_and_out_of_range_tokens(orc):
    T = 4
    qkv, qw, kw = _inputs(T, 5)
    cache = orc.rope_cache(32, D)
    pos = np.array([1, -1, 32, 7], np.int64)
    out = orc.qk_norm_rope(qkv, qw, kw, cache, pos, 1e-6, HQ, HKV, D)
    assert np.array_equal(out[1], qkv[1]) and np.array_equal(out[2], qkv[2])  # left unchanged
    swapped = orc.qk_norm_rope(qkv, kw, qw, cache, pos, 1e-6, HQ, HKV, D)
    assert not np.array_equal(_heads(out, T)[0, :HQ], _heads(swapped, T)[0, :HQ])
    with pytest.raises(ValueError):
        orc.qk_norm_rope(qkv, qw, kw, cache, pos, 1e-6, HQ, HKV, 63)  # odd head size
