"""The measurement probe (include/rmsq_probe.h) moves exactly the bytes it claims: every chunk
of both inputs is read and every output chunk written, in the fused kernel's layout."""
import ctypes

import pytest
import torch

from tests import gpu_harness as GH

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    GH.require_gpu()
    from rmsnorm_quantization_amd import build

    lib = ctypes.CDLL(build.PROBE_LIB)
    p = ctypes.c_void_p
    i32 = ctypes.c_int
    lib.rmsq_probe_stream.argtypes = [p, p, p, p, p, ctypes.c_int64, ctypes.c_int64, i32, i32,
                                      i32, i32, i32, p, p, p]
    return lib


@pytest.mark.parametrize("H,tpr,vpt,out1", [(4096, 256, 2, 8), (2048, 128, 2, 4), (512, 64, 1, 8),
                                            (7168, 448, 2, 8)])
def test_probe_outputs(L, H, tpr, vpt, out1):
    T = 37
    g = torch.Generator().manual_seed(H)
    a = torch.randint(-2**31, 2**31 - 1, (T, H // 2), generator=g, dtype=torch.int32).cuda()
    b = torch.randint(-2**31, 2**31 - 1, (T, H // 2), generator=g, dtype=torch.int32).cuda()
    c = GH.Guarded(T * H * 2)
    d = GH.Guarded(T * H * out1 // 8)
    st = L.rmsq_probe_stream(a.data_ptr(), b.data_ptr(), c.data.data_ptr(), d.data.data_ptr(),
                             None, T, H, out1, 0, 0, tpr, vpt, None, None,
                             torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    c.check("out0")
    d.check("out1")
    x = (a ^ b).view(T, H // 8, 4)
    assert torch.equal(c.data.view(torch.int32).view(T, H // 8, 4), x)
    if out1 == 8:
        ref = torch.stack([x[..., 0] ^ x[..., 2], x[..., 1] ^ x[..., 3]], dim=-1)
    else:
        ref = (x[..., 0] ^ x[..., 1] ^ x[..., 2] ^ x[..., 3])[..., None]
    assert torch.equal(d.data.view(torch.int32).view(T, H // 8, out1 // 4), ref)


@pytest.mark.parametrize("with_in1,with_out0,out1", [(False, True, 0), (False, False, 8),
                                                     (True, False, 4), (False, True, 8)])
def test_probe_stream_subsets(L, with_in1, with_out0, out1):
    """The probe with streams left out (a plain copy, codes-only output, ...): each present
    output holds its function of the present inputs, and nothing else is written."""
    T, H, tpr, vpt = 29, 2048, 128, 2
    g = torch.Generator().manual_seed(7 + out1)
    a = torch.randint(-2**31, 2**31 - 1, (T, H // 2), generator=g, dtype=torch.int32).cuda()
    b = torch.randint(-2**31, 2**31 - 1, (T, H // 2), generator=g, dtype=torch.int32).cuda()
    c = GH.Guarded(T * H * 2)
    d = GH.Guarded(max(1, T * H * out1 // 8))
    print(f"[probe] in1={with_in1} out0={with_out0} out1={out1}", flush=True)
    st = L.rmsq_probe_stream(a.data_ptr(), b.data_ptr() if with_in1 else None,
                             c.data.data_ptr() if with_out0 else None,
                             d.data.data_ptr() if out1 else None, None, T, H, out1, 0, 0, tpr,
                             vpt, None, None, torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    c.check("out0")
    d.check("out1")
    x = (a ^ b if with_in1 else a).view(T, H // 8, 4)
    if with_out0:
        assert torch.equal(c.data.view(torch.int32).view(T, H // 8, 4), x)
    else:
        assert torch.all(c.data == GH.FILL)
    if out1 == 8:
        ref = torch.stack([x[..., 0] ^ x[..., 2], x[..., 1] ^ x[..., 3]], dim=-1)
        assert torch.equal(d.data.view(torch.int32).view(T, H // 8, 2), ref)
    elif out1 == 4:
        ref = (x[..., 0] ^ x[..., 1] ^ x[..., 2] ^ x[..., 3])[..., None]
        assert torch.equal(d.data.view(torch.int32).view(T, H // 8, 1), ref)


@pytest.mark.parametrize("shift,nbytes", [(-1, 4), (4, 4), (3, 4), (4, 1), (1, 1)])
def test_probe_scale_stream(L, shift, nbytes):
    """The scale-like stream: one element per row (shift -1) or per 2^shift chunks, written by
    the thread of the element's first chunk with the XOR of that chunk's words 0 and 3."""
    T, H, tpr, vpt = 23, 2048, 128, 2
    g = torch.Generator().manual_seed(11 + shift)
    a = torch.randint(-2**31, 2**31 - 1, (T, H // 2), generator=g, dtype=torch.int32).cuda()
    per_row = 1 if shift < 0 else (H // 8) >> shift
    e = GH.Guarded(T * per_row * nbytes)
    print(f"[probe] scale stream shift={shift} bytes={nbytes}", flush=True)
    st = L.rmsq_probe_stream(a.data_ptr(), None, None, None, e.data.data_ptr(), T, H, 0, shift,
                             nbytes, tpr, vpt, None, None, torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    e.check("out2")
    x = a.view(T, H // 8, 4)
    starts = x[:, :1] if shift < 0 else x[:, ::1 << shift]
    val = starts[..., 0] ^ starts[..., 3]
    if nbytes == 4:
        assert torch.equal(e.data.view(torch.int32).view(T, per_row), val)
    else:
        assert torch.equal(e.data.view(T, per_row), (val & 0xFF).to(torch.uint8))
    # shapes the stream does not fit are refused
    assert L.rmsq_probe_stream(a.data_ptr(), None, None, None, e.data.data_ptr(), T, H, 0, 7,
                               nbytes, tpr, vpt, None, None, None) == -1
    assert L.rmsq_probe_stream(a.data_ptr(), None, None, None, e.data.data_ptr(), T, H, 0, shift,
                               2, tpr, vpt, None, None, None) == -1
