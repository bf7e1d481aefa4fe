"""GPU parity for residual add + RMSNorm -> padded output (vLLM docs "Fusion torch.compile
passes", section "RMSNorm + padding"), bf16 and IEEE binary16: bit-exact against the oracle,
padding columns zero, guard bands intact."""
import numpy as np
import pytest
import torch

import oracle as O
from rmsnorm_quantization_amd import binding as B
from rmsnorm_quantization_amd import synth
from tests import gpu_harness as GH

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    GH.require_gpu()


def run_pad(x, r, w, eps, ld, launch=None, inplace=False, rows=None, flags=0):
    T, H = x.shape
    go = GH.Guarded(T * ld * 2)
    gr = None
    rd = None if r is None else GH.to_dev(r).clone()
    if rd is not None:
        if inplace:
            rout = rd
        else:
            gr = GH.Guarded(T * H * 2)
            rout = gr.data.view(r.dtype)
    else:
        rout = None
    B.rmsq_rms_norm_pad(GH.to_dev(x), rd, GH.to_dev(w), eps, go.data.view(torch.bfloat16), rout,
                        tokens=T, hidden=H, out_ld=ld, launch=launch, flags=flags)
    torch.cuda.synchronize()
    go.check("out")
    if gr is not None:
        gr.check("residual_out")
    out = go.data.view(torch.bfloat16).view(T, ld)
    sel = None if rows is None else torch.as_tensor(np.asarray(rows), device="cuda")
    o = synth.bits(out if sel is None else out[sel])
    ro = None if rout is None else synth.bits(rout.view(T, H) if sel is None else rout.view(T, H)[sel])
    return o, ro


def _check(x, r, w, eps, ld, **kw):
    """x, r, w: CPU tensors, all bfloat16 or all float16 (then RMSQ_INPUT_F16 is passed)."""
    T, H = x.shape
    flags = B.RMSQ_INPUT_F16 if x.dtype == torch.float16 else 0
    rows = None  # every row compared
    print(f"[pad] T={T} H={H} ld={ld} flags={flags} rows=all {kw}", flush=True)
    o, ro = run_pad(x, r, w, eps, ld, rows=rows, flags=flags, **kw)
    xb = synth.bits(x) if rows is None else synth.bits(x)[rows]
    rb = None if r is None else (synth.bits(r) if rows is None else synth.bits(r)[rows])
    ref, rref = O.rms_norm_pad(xb, rb, synth.bits(w), eps, ld, flags=flags)
    assert np.array_equal(o, ref), f"{int((o != ref).sum())} output elements differ"
    if r is not None:
        assert np.array_equal(ro, rref)
    assert np.all(o[:, H:] == 0)
    return o


@pytest.mark.parametrize("T", [1, 256, 4096])
@pytest.mark.parametrize("multiple", [128, 256])
def test_gpt_oss_hidden(T, multiple):
    x, r, w = synth.make_inputs(6, T)
    ld = -(-2880 // multiple) * multiple
    _check(x, r, w, 1e-5, ld)


@pytest.mark.parametrize("H,ld", [(8, 8), (8, 64), (72, 128), (520, 520), (520, 1024),
                                  (4096, 4096), (4096, 4352), (65528, 65536)])
@pytest.mark.parametrize("residual", [False, True])
def test_ragged_and_unpadded(H, ld, residual):
    T = 3 if H > 60000 else 37
    g = torch.Generator().manual_seed(H + ld)
    x = torch.randn((T, H), generator=g).to(torch.bfloat16)
    r = torch.randn((T, H), generator=g).to(torch.bfloat16) if residual else None
    w = (torch.rand((H,), generator=g) + 0.5).to(torch.bfloat16)
    _check(x, r, w, 1e-6, ld)


def test_inplace_residual():
    x, r, w = synth.make_inputs(6, 64)
    _check(x, r, w, 1e-5, 3072, inplace=True)


def test_every_launch_shape_identical():
    x, r, w = synth.make_inputs(6, 21)
    base = _check(x, r, w, 1e-5, 3072)
    n = 0
    for tpr in (64, 128, 192, 256, 384, 512, 1024):
        for vpt in range(1, 9):
            if tpr * vpt * 8 < 3072:
                continue
            for rpb in (1, 2):
                if rpb * tpr > 1024:
                    continue
                o, _ = run_pad(x, r, w, 1e-5, 3072, launch=B.rmsq_launch(tpr, vpt, rpb, 0))
                assert np.array_equal(o, base), (tpr, vpt, rpb)
                n += 1
    assert n > 10
    # a shape that covers H (360 chunks) but not a 4096-wide padded row (512 chunks) is refused
    st = B.rmsq_rms_norm_pad(GH.to_dev(x), None, GH.to_dev(w), 1e-5,
                             torch.empty((21, 4096), dtype=torch.bfloat16, device="cuda"), None,
                             launch=B.rmsq_launch(192, 2, 1, 0), check=False)
    assert st == B.RMSQ_EINVAL
    torch.cuda.synchronize()


def test_helper_pads_to_multiple():
    x, r, w = synth.make_inputs(6, 16)
    out, rout = B.fused_add_rms_norm_pad(GH.to_dev(x), GH.to_dev(r).clone(), GH.to_dev(w), 1e-5)
    torch.cuda.synchronize()
    assert out.shape == (16, 3072)
    ref, rref = O.rms_norm_pad(synth.bits(x), synth.bits(r), synth.bits(w), 1e-5, 3072)
    assert np.array_equal(synth.bits(out), ref) and np.array_equal(synth.bits(rout), rref)


# ------------------------------------------------------------------ IEEE binary16 (RMSQ_INPUT_F16)
def _f16_inputs(T, H, seed, scale=1.0, residual=True, signed_w=True):
    g = torch.Generator().manual_seed(seed)
    x = (torch.randn((T, H), generator=g) * scale).to(torch.float16)
    r = (torch.randn((T, H), generator=g) * scale).to(torch.float16) if residual else None
    w = torch.rand((H,), generator=g) * 3 - 1.5 if signed_w else torch.rand((H,), generator=g) + 0.5
    return x, r, w.to(torch.float16)


@pytest.mark.parametrize("T,H,ld", [(1, 2880, 3072), (37, 2880, 3072), (4096, 2880, 3072),
                                    (19, 8, 64), (23, 4000, 4096), (5, 6144, 6144),
                                    (3, 65528, 65536)])
@pytest.mark.parametrize("residual", [False, True])
def test_binary16(T, H, ld, residual):
    x, r, w = _f16_inputs(T, H, T * 31 + H, residual=residual)
    _check(x, r, w, 1e-5, ld)


@pytest.mark.parametrize("launch", [(64, 6, 1), (192, 2, 1), (128, 3, 2), (384, 1, 2),
                                    (1024, 1, 1)])
def test_binary16_launch_shapes(launch):
    x, r, w = _f16_inputs(21, 2880, 3)
    _check(x, r, w, 1e-5, 3072, launch=B.rmsq_launch(*launch, 0))


def test_binary16_inplace_and_extremes():
    """In place; binary16 subnormal inputs; large inputs whose sums stay finite; outputs past
    65504 (infinity).  (Sums that overflow make NaN rows, outside the contract.)"""
    x, r, w = _f16_inputs(16, 2880, 4)
    _check(x, r, w, 1e-5, 3072, inplace=True)
    x, r, w = _f16_inputs(16, 2880, 5, scale=1e-5)
    _check(x, r, w, 1e-6, 3072)
    x, r, w = _f16_inputs(4, 512, 6, scale=8000.0)
    _check(x, r, w, 1e-6, 512)
    H = 64
    x = torch.zeros((3, H), dtype=torch.float16)
    x[0, 0], x[1, 7], x[2, :] = 3.0, -5.0, 1.0
    w = torch.full((H,), 10000.0, dtype=torch.float16)
    o = _check(x, None, w, 1e-6, 128)
    assert o[0, 0] == 0x7C00 and o[1, 7] == 0xFC00   # 8 * 10000 overflows binary16


def test_binary16_helper_follows_the_dtype():
    x, r, w = _f16_inputs(16, 2880, 7)
    xd, rd, wd = GH.to_dev(x), GH.to_dev(r).clone(), GH.to_dev(w)
    out, rout = B.fused_add_rms_norm_pad(xd, rd, wd, 1e-5)
    torch.cuda.synchronize()
    assert out.dtype == torch.float16 and out.shape == (16, 3072)
    ref, rref = O.rms_norm_pad(synth.bits(x), synth.bits(r), synth.bits(w), 1e-5, 3072,
                               flags=O.INPUT_F16)
    assert np.array_equal(synth.bits(out), ref) and np.array_equal(synth.bits(rout), rref)
    with pytest.raises(TypeError):
        B.fused_add_rms_norm_pad(xd, rd, wd.to(torch.bfloat16), 1e-5)
    # the same bits as bf16 are another input
    b16, _ = run_pad(x.view(torch.bfloat16), r.view(torch.bfloat16), w.view(torch.bfloat16), 1e-5,
                     3072)
    assert not np.array_equal(b16, ref)
