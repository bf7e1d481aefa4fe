"""The binding's allocating helpers (named after the pages' fused ops) against the oracle, for
bf16 and float16 activations: each must produce the oracle's codes, scales and new residual
and lay its outputs out as documented."""
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


def _bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _inputs(T, H, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((T, H), generator=g).to(dtype).cuda()
    r = torch.randn((T, H), generator=g).to(dtype).cuda()
    w = (torch.rand((H,), generator=g) + 0.5).to(dtype).cuda()
    return x, r, w


DTYPES = [torch.bfloat16, torch.float16]


def _flag(dtype):
    return O.INPUT_F16 if dtype == torch.float16 else 0


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("inplace", [True, False])
def test_static_fp8(dtype, inplace):
    x, r, w = _inputs(17, 2048, dtype, 1)
    r0 = _bits(r)
    q, rout = B.rms_norm_static_fp8_quant(x, w, 0.01, 1e-6, residual=r, inplace=inplace)
    torch.cuda.synchronize()
    ref = O.fused(_bits(x), r0, _bits(w), 1e-6, O.FP8_STATIC, scale_in=0.01,
                  flags=_flag(dtype))
    assert q.dtype == torch.float8_e4m3fn and q.shape == x.shape
    assert np.array_equal(q.view(torch.uint8).cpu().numpy(), ref["q"])
    assert np.array_equal(_bits(rout), ref["residual_out"])
    assert (rout.data_ptr() == r.data_ptr()) == inplace
    q2 = B.fused_add_rms_norm_static_fp8_quant(x, torch.from_numpy(r0.view(np.int16)).view(
        dtype).cuda(), w, 0.01, 1e-6)
    torch.cuda.synchronize()
    assert torch.equal(q2.view(torch.uint8), q.view(torch.uint8))


@pytest.mark.parametrize("dtype", DTYPES)
def test_per_token(dtype):
    x, r, w = _inputs(9, 4096, dtype, 2)
    q, s, rout = B.rms_norm_dynamic_per_token_quant(x, w, 1e-6)
    torch.cuda.synchronize()
    ref = O.fused(_bits(x), None, _bits(w), 1e-6, O.FP8_TOKEN, flags=_flag(dtype))
    assert rout is None and s.shape == (9,)
    assert np.array_equal(q.view(torch.uint8).cpu().numpy(), ref["q"])
    assert np.array_equal(s.cpu().numpy(), ref["scales"])


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("col_major,e8m0,e8m0_bytes", [(False, False, False), (True, False, False),
                                                     (False, True, False), (True, False, True)])
def test_per_group(dtype, col_major, e8m0, e8m0_bytes):
    x, r, w = _inputs(6, 1024, dtype, 3)
    r0 = _bits(r)
    q, s, rout = B.rms_norm_per_block_quant(x, w, 1e-6, group_size=64, residual=r,
                                            col_major=col_major, e8m0=e8m0,
                                            e8m0_bytes=e8m0_bytes, scale_ld=8 if col_major else 0)
    torch.cuda.synchronize()
    flags = ((O.SCALE_COLMAJOR if col_major else 0) | (O.SCALE_E8M0 if e8m0 else 0) |
             (O.SCALE_E8M0_U8 if e8m0_bytes else 0) | _flag(dtype))
    ref = O.fused(_bits(x), r0, _bits(w), 1e-6, O.FP8_GROUP, group_size=64, flags=flags,
                  scale_ld=8 if col_major else 0)
    assert np.array_equal(q.view(torch.uint8).cpu().numpy(), ref["q"])
    sg = s.cpu().numpy()
    if col_major:
        assert sg.shape == (16, 8)
        sg, sr = sg[:, :6], ref["scales"][:, :6]
    else:
        sr = ref["scales"]
    assert np.array_equal(sg, sr)
    assert np.array_equal(_bits(rout), ref["residual_out"])


@pytest.mark.parametrize("dtype", DTYPES)
def test_fp4(dtype):
    x, r, w = _inputs(5, 2048, dtype, 4)
    r0 = _bits(r)
    q, sf, rout = B.fused_add_rms_norm_fp4_quant(x, r, w, 700.0, 1e-6)
    torch.cuda.synchronize()
    ref = O.fused(_bits(x), r0, _bits(w), 1e-6, O.FP4_BLOCK16, scale_in=700.0, group_size=16,
                  flags=_flag(dtype))
    assert q.shape == (5, 1024) and sf.shape == (5, 128)
    assert np.array_equal(q.cpu().numpy(), ref["q"])
    assert np.array_equal(sf.cpu().numpy(), ref["scales"])
    assert np.array_equal(_bits(rout), ref["residual_out"])


def test_silu_and_mul_and_padding_helpers():
    g = torch.Generator().manual_seed(5)
    x = torch.randn((7, 2 * 1024), generator=g).to(torch.bfloat16).cuda()
    q, s = B.silu_and_mul_quant(x, B.RMSQ_FP8_GROUP, group_size=128)
    torch.cuda.synchronize()
    ref = O.silu_mul_quant(_bits(x), O.FP8_GROUP, group_size=128)
    assert q.shape == (7, 1024) and s.shape == (7, 8)
    # the activation is within a few ulp of the oracle's: codes may differ at exact ties only
    assert (q.view(torch.uint8).cpu().numpy() != ref["q"]).mean() < 1e-3
    xb, rb, wb = _inputs(3, 2880, torch.bfloat16, 6)
    r0 = _bits(rb)
    out, rout = B.fused_add_rms_norm_pad(xb, rb, wb, 1e-5, multiple=256)
    torch.cuda.synchronize()
    ro, rr = O.rms_norm_pad(_bits(xb), r0, _bits(wb), 1e-5, 3072)
    assert out.shape == (3, 3072)
    assert np.array_equal(_bits(out), ro) and np.array_equal(_bits(rout), rr)


def test_mixed_dtypes_are_refused():
    x, r, w = _inputs(2, 256, torch.float16, 7)
    with pytest.raises(TypeError):
        B.rms_norm_static_fp8_quant(x, w.to(torch.bfloat16), 0.01, 1e-6)
    with pytest.raises(TypeError):
        B.fused_add_rms_norm_fp4_quant(x, r.to(torch.bfloat16), w, 700.0, 1e-6)
    with pytest.raises(TypeError):
        B.rms_norm_dynamic_per_token_quant(x.float(), w.float(), 1e-6)
