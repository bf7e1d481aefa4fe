"""The Python binding refuses tensors that cannot hold what a call reads or writes (CPU only).

Every check runs before any pointer is taken, so CPU tensors reach it: a wrong dtype or a buffer
too small raises ValueError naming the argument, while well-formed CPU tensors get as far as the
device check ("must live on the GPU").  Without these checks such a call would read or write
past the end of a buffer on the GPU."""
import pytest
import torch

from rmsnorm_quantization_amd import binding as B

bf, f16 = torch.bfloat16, torch.float16


def _fused(T=4, H=256, mode=B.RMSQ_FP8_TOKEN, G=0, flags=0, ld=0, **over):
    a = dict(x=torch.zeros(T, H, dtype=bf), residual=torch.zeros(T, H, dtype=bf),
             weight=torch.ones(H, dtype=bf), eps=1e-6, mode=mode,
             scale_in=torch.ones(1) if mode in (B.RMSQ_FP8_STATIC, B.RMSQ_FP4_BLOCK16) else None,
             out_q=torch.zeros(T * H // (2 if mode == B.RMSQ_FP4_BLOCK16 else 1),
                               dtype=torch.uint8),
             out_scales={B.RMSQ_FP8_STATIC: None, B.RMSQ_FP8_TOKEN: torch.zeros(T),
                         B.RMSQ_FP8_GROUP: torch.zeros(T * H // max(G, 1)),
                         B.RMSQ_FP4_BLOCK16: torch.zeros(T * H // 16, dtype=torch.uint8)}[mode],
             residual_out=torch.zeros(T, H, dtype=bf), group_size=G, flags=flags, scale_ld=ld)
    a.update(over)
    return a


def test_well_formed_cpu_tensors_pass_the_checks():
    for mode, G in ((B.RMSQ_FP8_STATIC, 0), (B.RMSQ_FP8_TOKEN, 0), (B.RMSQ_FP8_GROUP, 128),
                    (B.RMSQ_FP4_BLOCK16, 16)):
        with pytest.raises(ValueError, match="must live on the GPU"):
            B.rmsq_fused(**_fused(mode=mode, G=G))


@pytest.mark.parametrize("over,match", [
    (dict(x=torch.zeros(2, 2, 256, dtype=bf)), "x must be a 2-D tensor"),
    (dict(x=torch.zeros(4, 256)), "x must have 16-bit elements"),
    (dict(weight=torch.ones(255, dtype=bf)), "weight holds 510 bytes, the call needs 512"),
    (dict(weight=torch.ones(256, dtype=torch.int8)), "weight must have 16-bit elements"),
    (dict(residual=torch.zeros(3, 256, dtype=bf)), "residual holds"),
    (dict(residual_out=torch.zeros(4, 128, dtype=bf)), "residual_out holds"),
    (dict(out_q=torch.zeros(1023, dtype=torch.uint8)), "out_q holds"),
    (dict(out_q=torch.zeros(1024, dtype=torch.float32)), "out_q must have 1-byte elements"),
    (dict(out_scales=torch.zeros(3)), "out_scales holds 12 bytes, the call needs 16"),
    (dict(out_scales=torch.zeros(4, dtype=torch.float64)), "out_scales must be float32"),
])
def test_fused_refuses(over, match):
    with pytest.raises(ValueError, match=match):
        B.rmsq_fused(**_fused(**over))


def test_flags_decide_the_activation_type():
    """At the ABI level the flag, not the tensor's dtype, says how the 16-bit bits are read (raw
    binary16 bits may travel in a bfloat16 tensor); the allocating helpers take the flag from the
    dtype and refuse mixed dtypes."""
    a = _fused(flags=B.RMSQ_INPUT_F16)
    with pytest.raises(ValueError, match="must live on the GPU"):
        B.rmsq_fused(**a)
    with pytest.raises(TypeError, match="x is torch.bfloat16 but another input is torch.float16"):
        B.rms_norm_dynamic_per_token_quant(torch.zeros(4, 256, dtype=bf),
                                           torch.ones(256, dtype=f16), 1e-6)


def test_group_scale_extents():
    T, H = 4, 512
    # column-major with a padded leading dimension: (H/G - 1) * ld + T f32
    a = _fused(T=T, H=H, mode=B.RMSQ_FP8_GROUP, G=128, flags=B.RMSQ_SCALE_COLMAJOR, ld=8,
               out_scales=torch.zeros(3 * 8 + 3))
    with pytest.raises(ValueError, match="out_scales holds 108 bytes, the call needs 112"):
        B.rmsq_fused(**a)
    a["out_scales"] = torch.zeros(3 * 8 + 4)
    with pytest.raises(ValueError, match="must live on the GPU"):
        B.rmsq_fused(**a)
    # E8M0 bytes: one byte per group
    a = _fused(T=T, H=H, mode=B.RMSQ_FP8_GROUP, G=64, flags=B.RMSQ_SCALE_E8M0_U8,
               out_scales=torch.zeros(T * H // 64 - 1, dtype=torch.uint8))
    with pytest.raises(ValueError, match="out_scales holds 31 bytes, the call needs 32"):
        B.rmsq_fused(**a)


def test_static_and_fp4_scale_inputs():
    with pytest.raises(ValueError, match="scale_in must be float32"):
        B.rmsq_fused(**_fused(mode=B.RMSQ_FP8_STATIC, scale_in=torch.ones(1, dtype=torch.float64)))
    with pytest.raises(ValueError, match="scale_in holds 0 bytes"):
        B.rmsq_fused(**_fused(mode=B.RMSQ_FP4_BLOCK16, G=16, scale_in=torch.ones(0)))
    with pytest.raises(ValueError, match="out_scales holds"):
        B.rmsq_fused(**_fused(mode=B.RMSQ_FP4_BLOCK16, G=16,
                              out_scales=torch.zeros(63, dtype=torch.uint8)))


def test_fp4_dynamic_global_scale():
    T, H = 4, 256
    args = (torch.zeros(T, H, dtype=bf), None, torch.ones(H, dtype=bf), 1e-6,
            torch.zeros(T * H // 2, dtype=torch.uint8), torch.zeros(T * H // 16, dtype=torch.uint8),
            None)
    with pytest.raises(ValueError, match="scale_in must be float32"):
        B.rmsq_fused_fp4_dynamic(*args, torch.zeros(1, dtype=torch.float16))
    with pytest.raises(ValueError, match="must live on the GPU"):
        B.rmsq_fused_fp4_dynamic(*args, torch.zeros(1))


def test_silu_mul_refuses():
    T, I = 3, 512
    x = torch.zeros(T, 2 * I, dtype=bf)
    with pytest.raises(ValueError, match="out_q holds"):
        B.rmsq_silu_mul_quant(x, B.RMSQ_FP8_TOKEN, None, torch.zeros(T * I - 1, dtype=torch.uint8),
                              torch.zeros(T))
    with pytest.raises(ValueError, match="x must be a 2-D tensor"):
        B.rmsq_silu_mul_quant(x.view(-1), B.RMSQ_FP8_TOKEN, None,
                              torch.zeros(T * I, dtype=torch.uint8), torch.zeros(T))
    with pytest.raises(ValueError, match="must live on the GPU"):
        B.rmsq_silu_mul_quant(x, B.RMSQ_FP8_TOKEN, None, torch.zeros(T * I, dtype=torch.uint8),
                              torch.zeros(T))


def test_pad_refuses():
    T, H = 3, 2880
    x, w = torch.zeros(T, H, dtype=bf), torch.ones(H, dtype=bf)
    with pytest.raises(ValueError, match="out holds"):
        B.rmsq_rms_norm_pad(x, None, w, 1e-5, torch.zeros(T * 3072 - 1, dtype=bf), None,
                            out_ld=3072)
    with pytest.raises(ValueError, match="out must be a 2-D tensor"):
        B.rmsq_rms_norm_pad(x, None, w, 1e-5, torch.zeros(T * 3072, dtype=bf), None)
    with pytest.raises(ValueError, match="must live on the GPU"):
        B.rmsq_rms_norm_pad(x, None, w, 1e-5, torch.zeros(T, 3072, dtype=bf), None)


def _rope(**over):
    T, hq, hkv, D, mp = 5, 4, 2, 128, 64
    a = dict(qkv=torch.zeros(T, (hq + 2 * hkv) * D, dtype=bf), q_weight=torch.ones(D, dtype=bf),
             k_weight=torch.ones(D, dtype=bf), cos_sin_cache=torch.zeros(mp, D),
             positions=torch.zeros(T, dtype=torch.int64), eps=1e-6, num_q_heads=hq,
             num_kv_heads=hkv, head_dim=D)
    a.update(over)
    return a


@pytest.mark.parametrize("over,match", [
    (dict(cos_sin_cache=torch.zeros(64, 128, dtype=bf)), "cos_sin_cache must be float32"),
    (dict(cos_sin_cache=torch.zeros(64 * 128)), "cos_sin_cache must be a 2-D tensor"),
    (dict(positions=torch.zeros(5, dtype=torch.int32)), "positions must be int64"),
    (dict(positions=torch.zeros(4, dtype=torch.int64)), "positions holds 32 bytes"),
    (dict(k_weight=torch.ones(64, dtype=bf)), "k_weight holds 128 bytes, the call needs 256"),
    (dict(q_weight=torch.ones(128)), "q_weight must have 16-bit elements"),
    (dict(qkv=torch.zeros(5, 7 * 128, dtype=bf)), "qkv rows hold 896 values, the heads need 1024"),
])
def test_qk_norm_rope_refuses(over, match):
    with pytest.raises(ValueError, match=match):
        B.rmsq_qk_norm_rope(**_rope(**over))


def test_qk_norm_rope_well_formed():
    with pytest.raises(ValueError, match="must live on the GPU"):
        B.rmsq_qk_norm_rope(**_rope())


def test_helpers_check_before_allocating_on_the_device():
    """The allocating helpers pass their tensors through the same checks."""
    x, w = torch.zeros(4, 256, dtype=bf), torch.ones(128, dtype=bf)
    with pytest.raises(ValueError, match="weight holds"):
        B.rms_norm_dynamic_per_token_quant(x, w, 1e-6)
