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


def test_padding_on_binary16(orc):
    """RMSNorm + padding on binary16: the first H outputs are the pinned y rounded by numpy to
    binary16, the rest zero; the new residual is the fused op's; read as bf16 it differs."""
    x, r, w = _inputs(5, 2880, 11)
    out, rout = orc.rms_norm_pad(x, r, w, 1e-5, 3072, flags=orc.INPUT_F16)
    y = orc.rms_y(x, r, w, 1e-5, f16=True)
    assert np.array_equal(out[:, :2880], f16_bits(y))
    assert np.all(out[:, 2880:] == 0)
    fused = orc.fused(x, r, w, 1e-5, orc.FP8_TOKEN, flags=orc.INPUT_F16)
    assert np.array_equal(rout, fused["residual_out"])
    plain, none = orc.rms_norm_pad(x, None, w, 1e-5, 2880, flags=orc.INPUT_F16)
    assert none is None and np.array_equal(plain, f16_bits(orc.rms_y(x, None, w, 1e-5, f16=True)))
    assert not np.array_equal(orc.rms_norm_pad(x, r, w, 1e-5, 3072)[0], out)


def test_padding_output_overflows_to_infinity(orc):
    """A row with one non-zero element a normalizes to sqrt(H) * sign(a) there: with H = 64 and a
    weight of 10000 that is 80000, past binary16's 65504, so the output is +-infinity (bf16,
    with its wider range, stays finite)."""
    H = 64
    x = np.zeros((2, H), np.uint16)
    x[0, 0], x[1, 0] = f16_bits(3.0), f16_bits(-3.0)
    w = f16_bits(np.full(H, 10000.0))
    out, _ = orc.rms_norm_pad(x, None, w, 1e-6, H, flags=orc.INPUT_F16)
    assert out[0, 0] == 0x7C00 and out[1, 0] == 0xFC00
    assert np.all(out[:, 1:] == 0)
    xb = np.zeros((1, H), np.uint16)
    xb[0, 0] = 0x4040  # 3.0 in bf16
    wb = np.full(H, 0x461C, np.uint16)  # 9984 in bf16
    outb, _ = orc.rms_norm_pad(xb, None, wb, 1e-6, H)
    assert np.isfinite(orc.bf16_to_f32(outb[0, 0]))


RQ, RKV, RD = 4, 2, 64


def _rope_inputs(T, seed, scale=2.0):
    rng = np.random.default_rng(seed)
    qkv = f16_bits(rng.standard_normal((T, (RQ + 2 * RKV) * RD)) * scale)
    qw = f16_bits(rng.uniform(0.5, 1.5, RD))
    kw = f16_bits(rng.uniform(-1.5, 1.5, RD))
    return qkv, qw, kw


def test_rope_position_zero_and_quarter_turn_on_binary16(orc):
    """Position 0 (cos 1, sin 0) leaves the normalized head, rounded to binary16; a cache with
    cos 0 and sin 1 maps each NeoX pair (a, b) to (-b, a).  v heads are not touched."""
    T = 3
    qkv, qw, kw = _rope_inputs(T, 12)
    heads = qkv.reshape(T, RQ + 2 * RKV, RD)
    cache = orc.rope_cache(8, RD)
    out = orc.qk_norm_rope(qkv, qw, kw, cache, np.zeros(T, np.int64), 1e-6, RQ, RKV, RD,
                           flags=orc.INPUT_F16).reshape(heads.shape)
    turn = np.zeros((4, RD), np.float32)
    turn[:, RD // 2:] = 1.0
    out_t = orc.qk_norm_rope(qkv, qw, kw, turn, np.full(T, 2, np.int64), 1e-6, RQ, RKV, RD,
                             flags=orc.INPUT_F16).reshape(heads.shape)
    for hd in range(RQ + RKV):
        y = orc.rms_y(np.ascontiguousarray(heads[:, hd]), None, qw if hd < RQ else kw, 1e-6,
                      f16=True)
        assert np.array_equal(out[:, hd], f16_bits(y))
        a, b = y[:, :RD // 2], y[:, RD // 2:]
        assert np.array_equal(out_t[:, hd], f16_bits(np.concatenate([-b, a], axis=1)))
    assert np.array_equal(out[:, RQ + RKV:], heads[:, RQ + RKV:])


@pytest.mark.parametrize("neox", [True, False])
def test_rope_on_binary16_matches_torch_float64(orc, neox):
    T = 8
    qkv, qw, kw = _rope_inputs(T, 13)
    cache = orc.rope_cache(100, RD, 10000.0)
    pos = np.random.default_rng(14).integers(0, 100, T)
    out = orc.qk_norm_rope(qkv, qw, kw, cache, pos, 1e-6, RQ, RKV, RD, neox, flags=orc.INPUT_F16)
    x = torch.from_numpy(qkv.view(np.float16).astype(np.float64)).reshape(T, RQ + 2 * RKV, RD)
    c = torch.from_numpy(cache[pos, :RD // 2]).double()[:, None, :]
    s = torch.from_numpy(cache[pos, RD // 2:]).double()[:, None, :]
    res = []
    for hs, w in ((slice(0, RQ), qw), (slice(RQ, RQ + RKV), kw)):
        wt = torch.from_numpy(w.view(np.float16).astype(np.float64))
        y = torch.nn.functional.rms_norm(x[:, hs], (RD,), wt, 1e-6)
        if neox:
            a, b = y[..., :RD // 2], y[..., RD // 2:]
            res.append(torch.cat([a * c - b * s, b * c + a * s], dim=-1))
        else:
            a, b = y[..., 0::2], y[..., 1::2]
            rr = torch.empty_like(y)
            rr[..., 0::2], rr[..., 1::2] = a * c - b * s, b * c + a * s
            res.append(rr)
    ref = torch.cat(res, dim=1)
    got = torch.from_numpy(out.view(np.float16).astype(np.float64)).reshape(
        T, RQ + 2 * RKV, RD)[:, :RQ + RKV]
    # binary16 output: half a binary16 ulp of the value plus the f32 steps, relative to the pair
    tol = ref.abs().amax(dim=-1, keepdim=True) * 2.0 ** -11 * 1.05
    assert torch.all((got - ref).abs() <= tol)
    # the same bits read as bf16 are another input altogether
    assert not np.array_equal(out, orc.qk_norm_rope(qkv, qw, kw, cache, pos, 1e-6, RQ, RKV, RD,
                                                    neox))
