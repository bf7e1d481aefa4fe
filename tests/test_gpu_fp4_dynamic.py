"""GPU parity of FP4 block-16 with the global scale taken from the batch
(rmsq_fused_fp4_dynamic, through the C ABI) against the oracle.

Two launches: residual add + RMSNorm with each workgroup's largest |y|, and the block
quantization of the normalized input, whose first workgroup reduces those maxima to
gs = (448 * 6) / amax and hands it to the others through global_scale; with more maxima than that
workgroup reduces in one round, a one-workgroup reduction launch runs between the two (covered by
test_middle_reduction_launch).  The global scale is
asserted bit-exact (both sides take the same f32 maximum and the same IEEE division); codes,
block scales and the new residual follow the static FP4 comparison rule of tests/parity.py.
Guard bands around every output catch stray writes.
"""
import numpy as np
import pytest
import torch

import oracle as O
from rmsnorm_quantization_amd import binding as B
from tests import gpu_harness as GH
from tests.parity import compare

pytestmark = pytest.mark.gpu
FLT_MAX = np.float32(np.finfo(np.float32).max)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    GH.require_gpu()


def _inputs(T, H, seed, dtype=torch.bfloat16, scale=1.0, residual=True):
    g = torch.Generator().manual_seed(seed)
    x = (torch.randn((T, H), generator=g) * scale).to(dtype)
    r = (torch.randn((T, H), generator=g) * scale).to(dtype) if residual else None
    w = (torch.rand((H,), generator=g) + 0.5).to(dtype)
    return x, r, w


def _bits(t):
    return None if t is None else t.contiguous().view(torch.int16).numpy().view(np.uint16)


def run(x, r, w, eps=1e-6, launch=None, inplace=False, scale_offset=0):
    """Run on device copies of CPU tensors; returns (gpu dict, oracle dict).  scale_offset: place
    the block scales that many bytes into their buffer (1: not 4-byte aligned)."""
    T, H = x.shape
    f16 = x.dtype == torch.float16
    flags = B.RMSQ_INPUT_F16 if f16 else 0
    print(f"[fp4dyn] T={T} H={H} residual={r is not None} f16={f16} inplace={inplace} "
          f"launch={None if launch is None else launch.as_tuple()} scale_offset={scale_offset}",
          flush=True)
    gq, gg = GH.Guarded(T * H // 2), GH.Guarded(4)
    gs_ = GH.Guarded(T * H // 16 + scale_offset)
    sdata = gs_.data[scale_offset:]
    rd = None if r is None else GH.to_dev(r).clone()
    grs = None
    if rd is None:
        rout = None
    elif inplace:
        rout = rd
    else:
        grs = GH.Guarded(T * H * 2)
        rout = grs.data.view(x.dtype)
    B.rmsq_fused_fp4_dynamic(GH.to_dev(x), rd, GH.to_dev(w), eps, gq.data, sdata, rout,
                             gg.data.view(torch.float32), flags=flags, launch=launch)
    torch.cuda.synchronize()
    for g, what in ((gq, "out_q"), (gs_, "out_scales"), (gg, "global_scale")):
        g.check(what)
    if grs is not None:
        grs.check("residual_out")
    gpu = {"q": gq.data.view(T, H // 2).cpu().numpy(),
           "scales": sdata.view(T, H // 16).cpu().numpy(),
           "residual_out": None if rout is None else _bits(rout.cpu()).reshape(T, H),
           "global_scale": gg.data.view(torch.float32).cpu().numpy()[0]}
    ref = O.fused_fp4_dynamic(_bits(x), _bits(r), _bits(w), eps, flags=flags, want_pre=True)
    return gpu, ref


def check(x, r, w, **kw):
    gpu, ref = run(x, r, w, **kw)
    T, H = x.shape
    assert gpu["global_scale"].view(np.uint32) == ref["global_scale"].view(np.uint32), (
        gpu["global_scale"], ref["global_scale"])
    eps = kw.get("eps", 1e-6)
    compare(O.FP4_BLOCK16, gpu, ref, T=T, H=H, group_size=16,
            scale_in=float(ref["global_scale"]),
            y_ref=GH.y_ref_norm(_bits(x), _bits(r), _bits(w), eps,
                                f16=x.dtype == torch.float16))
    return gpu, ref


# H % 64 == 0 and H <= 4096: the block pass reads the row pass's inverse RMS (one wave per row);
# the others (H 16, 48, 80, 4160, 5120, 65536) normalize again with the row pass's launch shape
@pytest.mark.parametrize("T,H", [(1, 2048), (32, 2048), (256, 2048), (4096, 2048), (37, 5120),
                                 (5, 16), (9, 48), (3, 65536), (33, 64), (17, 1024), (20, 4096),
                                 (7, 80), (5, 4160)])
@pytest.mark.parametrize("residual", [True, False])
def test_shapes(T, H, residual):
    x, r, w = _inputs(T, H, T * 3 + H, residual=residual)
    check(x, r, w)


@pytest.mark.parametrize("launch", [None, (64, 1, 1)])
def test_middle_reduction_launch(launch):
    """8200 rows of 64: the default shape takes 16 rows to a workgroup in both passes (513
    maxima, one round for the block pass's first workgroup: two launches); a caller's one row to
    a workgroup leaves 8200 maxima, more than eight per thread of a 1024-thread workgroup, so
    the one-workgroup reduction runs between the passes.  Both against the oracle."""
    x, r, w = _inputs(8200, 64, 10)
    check(x, r, w, launch=None if launch is None else B.rmsq_launch(*launch, 0))


def test_concurrent_calls_on_several_streams():
    """Four calls in flight at once on four streams (default priority), each with its own
    buffers: every workgroup 0 hands its global scale to its own call's workgroups only, through
    that call's global_scale, so each result equals the oracle's for its own batch."""
    T, H = 2048, 2048
    batches = [_inputs(T, H, 100 + i) for i in range(4)]
    streams = [torch.cuda.Stream() for _ in range(4)]
    outs = []
    for (x, r, w), st in zip(batches, streams):
        o = dict(q=torch.empty((T, H // 2), dtype=torch.uint8, device="cuda"),
                 s=torch.empty((T, H // 16), dtype=torch.uint8, device="cuda"),
                 ro=torch.empty((T, H), dtype=torch.bfloat16, device="cuda"),
                 g=torch.full((1,), 7.0, dtype=torch.float32, device="cuda"),
                 x=GH.to_dev(x), r=GH.to_dev(r), w=GH.to_dev(w))
        outs.append(o)
    torch.cuda.synchronize()
    print("[fp4dyn] four concurrent calls", flush=True)
    for o, st in zip(outs, streams):
        B.rmsq_fused_fp4_dynamic(o["x"], o["r"], o["w"], 1e-6, o["q"], o["s"], o["ro"], o["g"],
                                 stream=st)
    torch.cuda.synchronize()
    for (x, r, w), o in zip(batches, outs):
        ref = O.fused_fp4_dynamic(_bits(x), _bits(r), _bits(w), 1e-6)
        assert o["g"].cpu().numpy().view(np.uint32)[0] == ref["global_scale"].view(np.uint32)
        assert np.array_equal(o["q"].cpu().numpy(), ref["q"])
        assert np.array_equal(o["s"].cpu().numpy(), ref["scales"])
        assert np.array_equal(_bits(o["ro"].cpu()).reshape(T, H), ref["residual_out"])


def test_row_pass_packs_rows_for_one_round():
    """65536 rows of 64: the row pass's default four rows per workgroup would leave 16384 maxima,
    more than the block pass's first 1024-thread workgroup reduces in one round (8192), so the
    row pass takes eight rows per workgroup (8192 maxima) and there is no middle launch."""
    x, r, w = _inputs(65536, 64, 12)
    check(x, r, w)


@pytest.mark.parametrize("T,H", [(1, 2048), (37, 2048), (512, 4096), (1024, 2048)])
def test_binary16(T, H):
    x, r, w = _inputs(T, H, T + H + 1, dtype=torch.float16)
    check(x, r, w)
    x, _, w = _inputs(T, H, T + H + 2, dtype=torch.float16, residual=False)
    check(x, None, w)


@pytest.mark.parametrize("launch", [(64, 4, 1), (128, 2, 2), (256, 1, 4), (192, 2, 1),
                                    (1024, 1, 1), (64, 8, 1)])
def test_launch_shapes(launch):
    x, r, w = _inputs(21, 2048, 5)
    check(x, r, w, launch=B.rmsq_launch(*launch, 0))


def test_inplace_and_value_ranges():
    x, r, w = _inputs(64, 2048, 6)
    check(x, r, w, inplace=True)
    for scale in (1e-30, 1e-3, 1e4, 1e30):   # the global scale follows the batch's magnitude
        x, r, w = _inputs(16, 2048, 7, scale=scale)
        gpu, _ = check(x, r, w)


@pytest.mark.parametrize("H", [1024, 2048])
def test_unaligned_block_scales(H):
    """Block scales not 4-byte aligned: no staging, the block pass normalizes again -- the same
    results."""
    x, r, w = _inputs(29, H, H + 3)
    check(x, r, w, scale_offset=1)
    check(x, r, w, scale_offset=2, launch=B.rmsq_launch(128, H // 1024 or 1, 2, 0))


def test_zero_batch_gives_flt_max_and_zero_codes():
    T, H = 8, 1024
    x = torch.zeros((T, H), dtype=torch.bfloat16)
    w = torch.ones(H, dtype=torch.bfloat16)
    gpu, ref = check(x, None, w)
    assert gpu["global_scale"] == FLT_MAX
    assert not gpu["q"].any() and not gpu["scales"].any()


def test_one_row_decides_the_scale():
    """A one-hot row normalizes to sqrt(H) * w at its spike, far above the other rows' values:
    it sets the global scale, and every other row's codes move with it.  (Scaling a row does
    nothing: RMSNorm is scale-invariant.)"""
    x, r, w = _inputs(33, 2048, 8)
    g1, _ = check(x, r, w)
    x2, r2 = x.clone(), r.clone()
    x2[17], r2[17] = 0.0, 0.0
    x2[17, 5] = 3.0
    g2, _ = check(x2, r2, w)
    assert g2["global_scale"] < g1["global_scale"] / 4
    assert not np.array_equal(g1["q"][:17], g2["q"][:17])


def test_helper_and_dequantization():
    """The allocating helper returns gs; dequantized values stay within decode(sf) / gs of y."""
    x, r, w = _inputs(16, 2048, 9)
    q, sf, gs, rout = B.fused_add_rms_norm_fp4_quant_dynamic(GH.to_dev(x), GH.to_dev(r).clone(),
                                                             GH.to_dev(w), 1e-6)
    torch.cuda.synchronize()
    ref = O.fused_fp4_dynamic(_bits(x), _bits(r), _bits(w), 1e-6)
    assert gs.item() == float(ref["global_scale"])
    assert np.array_equal(q.cpu().numpy(), ref["q"]) and np.array_equal(sf.cpu().numpy(),
                                                                          ref["scales"])
    y = O.rms_y(_bits(x), _bits(r), _bits(w), 1e-6)
    d = O.e4m3_decode(sf.cpu().numpy()).astype(np.float64)
    nib = np.empty(y.shape, np.int64)
    qc = q.cpu().numpy()
    nib[:, 0::2], nib[:, 1::2] = qc & 0xF, qc >> 4
    step = np.repeat(d, 16, axis=1) / gs.item()
    deq = O.e2m1_decode(nib.astype(np.uint8)).astype(np.float64) * step
    assert np.all(np.abs(deq - y) <= step * (1 + 1e-6))
    with pytest.raises(TypeError):
        B.fused_add_rms_norm_fp4_quant_dynamic(GH.to_dev(x), GH.to_dev(r),
                                               GH.to_dev(w).to(torch.float16), 1e-6)
