"""GPU parity of QK-norm + RoPE (rmsq_qk_norm_rope, through the C ABI) against the oracle.

The op (vLLM docs "Fusion torch.compile passes", section "QK Norm + RoPE") rewrites the q and k
heads of the packed qkv tensor in place.  Both sides sum the squares of a head in binary64 (exact
for bf16 and binary16 inputs), round the same inverse RMS to f32, and form y = (h * inv) * w and
the rotated pair (a c - b s, b c + a s) from separately rounded f32 products, so the 16-bit
result (bf16, or IEEE binary16 with RMSQ_INPUT_F16) is asserted bit-exact: every element of every head, v heads and skipped tokens included (they must come back
unchanged).  A guard band around qkv catches stray writes.
"""
import numpy as np
import pytest
import torch

import oracle as O
from rmsnorm_quantization_amd import binding as B
from rmsnorm_quantization_amd import synth
from tests import gpu_harness as G

pytestmark = pytest.mark.gpu

WL = 7


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    G.require_gpu()


_CACHES = {}


def cache_for(max_pos, D, base=1e6):
    key = (max_pos, D, base)
    if key not in _CACHES:
        c = O.rope_cache(max_pos, D, base)
        _CACHES[key] = (c, torch.from_numpy(c).to("cuda"))
    return _CACHES[key]


def run_rope(qkv_bits, qw_bits, kw_bits, pos, hq, hkv, D, neox=True, eps=1e-6, max_pos=None,
             hpb=0, hpl=0, base=1e6, flags=0):
    """Run the kernel on a guarded copy of qkv; returns (gpu bits, oracle bits).  flags:
    RMSQ_INPUT_F16 reads the bit patterns as IEEE binary16 on both sides."""
    T = qkv_bits.shape[0]
    cache, cache_d = cache_for(max_pos if max_pos is not None else 4096, D, base)
    g = G.Guarded(qkv_bits.size * 2)
    dev = g.data.view(torch.int16)
    dev.copy_(torch.from_numpy(qkv_bits.reshape(-1).view(np.int16)))
    qw = torch.from_numpy(qw_bits.view(np.int16)).to("cuda")
    kw = torch.from_numpy(kw_bits.view(np.int16)).to("cuda")
    pos_d = torch.as_tensor(np.asarray(pos, np.int64)).to("cuda")
    print(f"[rope] T={T} hq={hq} hkv={hkv} D={D} neox={neox} hpb={hpb} hpl={hpl} flags={flags}",
          flush=True)
    B.rmsq_qk_norm_rope(dev, qw, kw, cache_d, pos_d, eps, hq, hkv, D, neox, tokens=T,
                        heads_per_block=hpb, heads_per_lane=hpl, flags=flags)
    torch.cuda.synchronize()
    g.check("qkv")
    got = dev.cpu().numpy().view(np.uint16).reshape(qkv_bits.shape)
    ref = O.qk_norm_rope(qkv_bits, qw_bits, kw_bits, cache, pos, eps, hq, hkv, D, neox,
                         flags=flags)
    return got, ref


def assert_same(got, ref, what=""):
    bad = got != ref
    n = int(bad.sum())
    if n:
        t, c = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {n} of {got.size} bf16 values differ; first at token {t} "
                             f"column {c}: gpu {got[t, c]:#06x} oracle {ref[t, c]:#06x}")


def wl_inputs(T, hq=None, hkv=None, D=None, max_pos=4096):
    qkv, qw, kw, pos = synth.make_rope_inputs(WL, T, hq, hkv, D, max_pos)
    return synth.bits(qkv), synth.bits(qw), synth.bits(kw), pos.numpy()


@pytest.mark.parametrize("T", [1, 256, 4096])
@pytest.mark.parametrize("neox", [True, False])
def test_workload_shapes(T, neox):
    """The full workload: 32 q heads, 8 kv heads, head size 128, 32768 positions."""
    x, qw, kw, pos = wl_inputs(T, max_pos=32768)
    print(f"rope workload T={T} neox={neox}", flush=True)
    got, ref = run_rope(x, qw, kw, pos, 32, 8, 128, neox, max_pos=32768)
    assert_same(got, ref, f"T={T}")
    assert not np.array_equal(got, x)


def test_largest_batch_default_shape():
    """16384 tokens: the default shape switches to 2 heads per lane (multi-round grid)."""
    x, qw, kw, pos = wl_inputs(16384, max_pos=32768)
    print("rope workload T=16384", flush=True)
    got, ref = run_rope(x, qw, kw, pos, 32, 8, 128, True, max_pos=32768)
    assert_same(got, ref, "T=16384")


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("neox", [True, False])
@pytest.mark.parametrize("hq,hkv", [(1, 1), (4, 2), (12, 4), (64, 8)])
def test_head_sizes_and_counts(D, neox, hq, hkv):
    T = 37  # ragged
    x, qw, kw, pos = wl_inputs(T, hq, hkv, D)
    print(f"rope D={D} neox={neox} hq={hq} hkv={hkv}", flush=True)
    got, ref = run_rope(x, qw, kw, pos, hq, hkv, D, neox)
    assert_same(got, ref, f"D={D} hq={hq} hkv={hkv}")


@pytest.mark.parametrize("hpb,hpl", [(1, 1), (2, 1), (7, 1), (64, 1), (8, 2), (16, 2), (30, 3), (16, 4),
                                     (40, 4), (40, 5), (36, 6), (48, 6), (6, 6), (20, 5)])
def test_launch_shapes(hpb, hpl):
    """Every launch shape gives the same bits: partial waves ((hpb / hpl) * 8 lanes not a
    multiple of 64), a partial last workgroup per token, and lane groups past the last head."""
    x, qw, kw, pos = wl_inputs(19)
    print(f"rope hpb={hpb} hpl={hpl}", flush=True)
    for neox in (True, False):
        got, ref = run_rope(x, qw, kw, pos, 32, 8, 128, neox, hpb=hpb, hpl=hpl)
        assert_same(got, ref, f"hpb={hpb} hpl={hpl} neox={neox}")


@pytest.mark.parametrize("D,hpb,hpl", [(64, 3, 3), (64, 5, 1), (64, 8, 2), (256, 1, 1),
                                       (256, 6, 2), (256, 8, 4)])
def test_launch_shapes_other_sizes(D, hpb, hpl):
    x, qw, kw, pos = wl_inputs(11, 6, 2, D)
    for neox in (True, False):
        got, ref = run_rope(x, qw, kw, pos, 6, 2, D, neox, hpb=hpb, hpl=hpl)
        assert_same(got, ref, f"D={D} hpb={hpb} hpl={hpl} neox={neox}")


def test_positions_out_of_range_leave_tokens_unchanged():
    x, qw, kw, _ = wl_inputs(8)
    pos = np.array([0, -1, 4095, 4096, 1 << 40, -(1 << 40), 17, 4096 * 2], np.int64)
    got, ref = run_rope(x, qw, kw, pos, 32, 8, 128, max_pos=4096)
    assert_same(got, ref, "positions")
    for t in (1, 3, 4, 5, 7):
        assert np.array_equal(got[t], x[t])
    for t in (0, 2, 6):
        assert not np.array_equal(got[t], x[t])


def test_position_zero_and_v_heads():
    """Position 0 rotates by nothing: the output is bf16 of the normalized head; v stays."""
    x, qw, kw, _ = wl_inputs(5)
    got, ref = run_rope(x, qw, kw, np.zeros(5, np.int64), 32, 8, 128)
    assert_same(got, ref, "pos 0")
    assert np.array_equal(got[:, 40 * 128:], x[:, 40 * 128:])


def test_extreme_values():
    """Zero heads (y = 0), bf16 values near the top of the range (their squares overflow f32,
    not binary64), subnormal heads (eps dominates), and a single spike per head."""
    T, hq, hkv, D = 6, 4, 2, 128
    x, qw, kw, pos = wl_inputs(T, hq, hkv, D)
    h = synth.from_bits(x).float().reshape(T, hq + 2 * hkv, D)
    h[0] = 0.0
    h[1] *= 1e37
    h[2] *= 1e-39
    h[3] = 0.0
    h[3, :, 5] = -3.0
    h[4, :, ::2] = 65504.0
    x = synth.bits(h.reshape(T, -1).to(torch.bfloat16))
    for neox in (True, False):
        got, ref = run_rope(x, qw, kw, pos, hq, hkv, D, neox)
        assert_same(got, ref, f"extreme neox={neox}")
        assert np.all(got[0, :(hq + hkv) * D] & 0x7FFF == 0)


def test_eps_and_weights_reach_the_kernel():
    x, qw, kw, pos = wl_inputs(4, 4, 2, 64)
    a, ra = run_rope(x, qw, kw, pos, 4, 2, 64, eps=1.0)
    b, rb = run_rope(x, kw, qw, pos, 4, 2, 64, eps=1e-6)
    assert_same(a, ra, "eps 1")
    assert_same(b, rb, "swapped weights")
    assert not np.array_equal(a, b)


def test_zero_tokens_is_a_no_op():
    qkv = torch.zeros((0, 6 * 128), dtype=torch.bfloat16, device="cuda")
    w = torch.ones(128, dtype=torch.bfloat16, device="cuda")
    _, cache_d = cache_for(4096, 128)
    pos = torch.zeros(0, dtype=torch.int64, device="cuda")
    B.rmsq_qk_norm_rope(qkv, w, w, cache_d, pos, 1e-6, 4, 1, 128)
    torch.cuda.synchronize()


def test_fused_op_helper():
    x, qw, kw, pos = wl_inputs(16)
    cache, cache_d = cache_for(4096, 128)
    qkv = synth.from_bits(x).to("cuda")
    out = B.qk_norm_rope(qkv, torch.as_tensor(pos).to("cuda"), synth.from_bits(qw).to("cuda"),
                         synth.from_bits(kw).to("cuda"), cache_d, 1e-6, 32, 8)
    torch.cuda.synchronize()
    assert out.data_ptr() == qkv.data_ptr()
    ref = O.qk_norm_rope(x, qw, kw, cache, pos, 1e-6, 32, 8, 128)
    assert_same(synth.bits(out), ref, "helper")


# ------------------------------------------------------------------ IEEE binary16 (RMSQ_INPUT_F16)
F16 = B.RMSQ_INPUT_F16


def f16_inputs(T, hq, hkv, D, seed, scale=1.0, max_pos=4096):
    rng = np.random.default_rng(seed)
    f16 = (lambda a: np.asarray(a, np.float32).astype(np.float16).view(np.uint16))
    qkv = f16(rng.standard_normal((T, (hq + 2 * hkv) * D)) * scale)
    qw = f16(rng.uniform(-1.5, 1.5, D))
    kw = f16(rng.uniform(0.5, 1.5, D))
    pos = rng.integers(0, max_pos, T).astype(np.int64)
    return qkv, qw, kw, pos


@pytest.mark.parametrize("T", [1, 256, 4096])
def test_binary16_workload_shape(T):
    x, qw, kw, pos = f16_inputs(T, 32, 8, 128, T, max_pos=32768)
    for neox in (True, False):
        got, ref = run_rope(x, qw, kw, pos, 32, 8, 128, neox, max_pos=32768, flags=F16)
        assert_same(got, ref, f"binary16 T={T} neox={neox}")
        assert not np.array_equal(got, x)


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("hq,hkv", [(1, 1), (12, 4), (64, 8)])
def test_binary16_head_sizes_and_counts(D, hq, hkv):
    x, qw, kw, pos = f16_inputs(37, hq, hkv, D, D + hq)
    for neox in (True, False):
        got, ref = run_rope(x, qw, kw, pos, hq, hkv, D, neox, flags=F16)
        assert_same(got, ref, f"binary16 D={D} hq={hq} hkv={hkv} neox={neox}")


@pytest.mark.parametrize("hpb,hpl", [(1, 1), (7, 1), (8, 2), (30, 3), (40, 5), (36, 6)])
def test_binary16_launch_shapes(hpb, hpl):
    x, qw, kw, pos = f16_inputs(19, 32, 8, 128, 3)
    got, ref = run_rope(x, qw, kw, pos, 32, 8, 128, True, hpb=hpb, hpl=hpl, flags=F16)
    assert_same(got, ref, f"binary16 hpb={hpb} hpl={hpl}")


def test_binary16_extremes_and_type_selection():
    """Zero heads, binary16 subnormal heads, values near 65504, out-of-range positions, and
    outputs that overflow binary16 (weights of 10000 on a one-hot head); the same bits read as
    bf16 give another result."""
    T, hq, hkv, D = 7, 4, 2, 128
    x, qw, kw, pos = f16_inputs(T, hq, hkv, D, 9)
    h = x.view(np.float16).astype(np.float32).reshape(T, hq + 2 * hkv, D)
    h[0] = 0.0
    h[1] *= 1e-6
    h[2] = np.clip(h[2] * 30000.0, -65504, 65504)
    h[3] = 0.0
    h[3, :, 9] = 2.0
    x2 = h.reshape(T, -1).astype(np.float16).view(np.uint16)
    big = np.full(D, np.float16(10000.0)).view(np.uint16)
    pos = pos.copy()
    pos[5], pos[6] = -1, 4096
    for neox in (True, False):
        got, ref = run_rope(x2, big, qw, pos, hq, hkv, D, neox, flags=F16)
        assert_same(got, ref, f"binary16 extremes neox={neox}")
        assert np.all(got[0, :(hq + hkv) * D] & 0x7FFF == 0)
        # y = sqrt(D) * 10000 at the spike; its larger rotated part exceeds 65504
        assert np.any((got[3, :hq * D] & 0x7FFF) == 0x7C00)
        assert np.array_equal(got[5:], x2[5:])
    as_bf16, _ = run_rope(x, qw, kw, pos, hq, hkv, D)
    as_f16, _ = run_rope(x, qw, kw, pos, hq, hkv, D, flags=F16)
    assert not np.array_equal(as_bf16, as_f16)


def test_binary16_helper_follows_the_dtype():
    x, qw, kw, pos = f16_inputs(16, 32, 8, 128, 10)
    cache, cache_d = cache_for(4096, 128)
    t16 = (lambda b: torch.from_numpy(b.view(np.float16)).to("cuda"))
    qkv = t16(x)
    out = B.qk_norm_rope(qkv, torch.as_tensor(pos).to("cuda"), t16(qw), t16(kw), cache_d, 1e-6,
                         32, 8)
    torch.cuda.synchronize()
    ref = O.qk_norm_rope(x, qw, kw, cache, pos, 1e-6, 32, 8, 128, flags=O.INPUT_F16)
    assert_same(out.cpu().view(torch.int16).numpy().view(np.uint16), ref, "binary16 helper")
    with pytest.raises(TypeError):
        B.qk_norm_rope(qkv, torch.as_tensor(pos).to("cuda"), t16(qw).to(torch.bfloat16), t16(kw),
                       cache_d, 1e-6, 32, 8)


@pytest.mark.parametrize("hq,hkv,D", [(4064, 8, 256), (8176, 8, 128), (16352, 8, 64)])
def test_widest_rows(hq, hkv, D):
    """qkv rows at the documented maximum of 2^20 elements (one of them exactly), default and
    explicit launch shapes, bf16 and binary16."""
    x, qw, kw, pos = wl_inputs(3, hq, hkv, D)
    got, ref = run_rope(x, qw, kw, pos, hq, hkv, D)
    assert_same(got, ref, f"widest D={D}")
    got, ref = run_rope(x, qw, kw, pos, hq, hkv, D, False, hpb=12, hpl=3)
    assert_same(got, ref, f"widest D={D} hpb=12 hpl=3")
    x16, qw16, kw16, pos16 = f16_inputs(2, hq, hkv, D, D)
    got, ref = run_rope(x16, qw16, kw16, pos16, hq, hkv, D, flags=F16)
    assert_same(got, ref, f"widest binary16 D={D}")
