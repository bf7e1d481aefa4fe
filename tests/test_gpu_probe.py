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
    lib.rmsq_probe_stream.argtypes = [p, p, p, p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_int, p, p, p]
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
                             T, H, out1, tpr, vpt, None, None,
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
