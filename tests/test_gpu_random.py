"""Seeded random sweep of every entry point against the oracle: shapes, modes, flags, value
scales, weights of either sign, residual or not, and random valid launch shapes -- the
combinations the hand-picked parity tests do not enumerate.  Each case prints its parameters
before it runs; the comparison rule is the one of tests/parity.py (bit-exact where the method is
exact)."""
import numpy as np
import pytest
import torch

import oracle as O
from rmsnorm_quantization_amd import binding as B
from rmsnorm_quantization_amd import synth
from tests import gpu_harness as GH
from tests.parity import compare

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    GH.require_gpu()


def _bf16(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16)


def _to16(flags):
    """float array -> 16-bit patterns of the type flags selects (bf16, or binary16)."""
    if flags & O.INPUT_F16:
        return lambda a: np.asarray(a, np.float32).astype(np.float16).view(np.uint16)
    return lambda a: synth.bits(_bf16(a))


def _random_launch(rng, n_chunks):
    """A valid launch shape covering n_chunks 16-byte chunks per row, or None (the default)."""
    if rng.random() < 0.3:
        return None
    for _ in range(100):
        tpr = 64 * int(rng.integers(1, 17))
        vpt = int(rng.integers(1, 9))
        rpb = int(rng.choice([1, 2, 4]))
        if tpr * vpt >= n_chunks and rpb * tpr <= 1024 and tpr * (vpt - 1) < n_chunks:
            return B.rmsq_launch(tpr, vpt, rpb, 0)
    return None


def _fused_case(seed):
    rng = np.random.default_rng(seed)
    mode = int(rng.integers(0, 4))
    G = {O.FP8_GROUP: int(rng.choice([64, 128])), O.FP4_BLOCK16: 16}.get(mode, 0)
    gran = max(G, 8)
    H = gran * int(rng.integers(1, max(2, 8192 // gran)))
    T = int(rng.integers(1, 70))
    flags = 0
    if mode == O.FP8_GROUP:
        flags = int(rng.choice([0, O.SCALE_COLMAJOR, O.SCALE_E8M0, O.SCALE_E8M0_U8,
                                O.SCALE_COLMAJOR | O.SCALE_E8M0_U8]))
    ld = T + int(rng.integers(0, 5)) if flags & O.SCALE_COLMAJOR else 0
    residual = bool(rng.random() < 0.7)
    sigma = float(rng.choice([1e-3, 1.0, 30.0]))
    x = rng.standard_normal((T, H)) * sigma
    r = rng.standard_normal((T, H)) * sigma if residual else None
    w = rng.uniform(-1.5, 1.5, H) if rng.random() < 0.3 else rng.uniform(0.5, 1.5, H)
    eps = float(rng.choice([1e-6, 1e-5]))
    f16 = bool(rng.random() < 0.3)  # IEEE binary16 activations instead of bf16
    to16 = ((lambda a: np.asarray(a, np.float32).astype(np.float16).view(np.uint16)) if f16
            else (lambda a: synth.bits(_bf16(a))))
    xb, wb = to16(x), to16(w)
    rb = None if r is None else to16(r)
    if f16:
        flags |= O.INPUT_F16
    y = O.rms_y(xb, rb, wb, eps, f16=f16)
    amax = float(np.abs(y).max()) or 1.0
    scale = 0.0
    if mode == O.FP8_STATIC:
        scale = float(np.float32(amax / 448 * rng.uniform(0.5, 2.0)))
    elif mode == O.FP4_BLOCK16:
        scale = float(np.float32(448 * 6 / amax * rng.uniform(0.5, 2.0)))
    launch = _random_launch(rng, H // 8)
    return dict(mode=mode, G=G, H=H, T=T, flags=flags, ld=ld, eps=eps, scale=scale,
                launch=launch, xb=xb, rb=rb, wb=wb)


@pytest.mark.parametrize("seed", range(240))
def test_random_fused(seed):
    c = _fused_case(9000 + seed)
    shape = None if c["launch"] is None else c["launch"].as_tuple()
    print(f"[random] seed={seed} mode={c['mode']} T={c['T']} H={c['H']} G={c['G']} "
          f"flags={c['flags']} ld={c['ld']} residual={c['rb'] is not None} launch={shape}",
          flush=True)
    to_dev = (lambda b: None if b is None else synth.from_bits(b).to("cuda"))
    gpu = GH.run(c["mode"], to_dev(c["xb"]), to_dev(c["rb"]), to_dev(c["wb"]), c["eps"],
                 scale_in=c["scale"] if c["mode"] in (O.FP8_STATIC, O.FP4_BLOCK16) else None,
                 group_size=c["G"], flags=c["flags"], scale_ld=c["ld"], launch=c["launch"])
    ref = O.fused(c["xb"], c["rb"], c["wb"], c["eps"], c["mode"], scale_in=c["scale"],
                  group_size=c["G"], flags=c["flags"], scale_ld=c["ld"], want_pre=True)
    raw = None
    if c["mode"] == O.FP8_GROUP and c["flags"] & (O.SCALE_E8M0 | O.SCALE_E8M0_U8):
        raw = O.fused(c["xb"], c["rb"], c["wb"], c["eps"], c["mode"], group_size=c["G"],
                      flags=c["flags"] & (O.SCALE_COLMAJOR | O.INPUT_F16),
                      scale_ld=c["ld"])["scales"]
    if c["flags"] & O.SCALE_COLMAJOR and c["ld"] > c["T"]:
        # columns past T are padding the library never writes: compare the written part only
        gpu["scales"] = gpu["scales"][:, :c["T"]]
        ref["scales"] = ref["scales"][:, :c["T"]]
        if raw is not None:
            raw = raw[:, :c["T"]]
    compare(c["mode"], gpu, ref, T=c["T"], H=c["H"], group_size=c["G"], flags=c["flags"],
            scale_in=c["scale"], raw_group_scales=raw,
            y_ref=GH.y_ref_norm(c["xb"], c["rb"], c["wb"], c["eps"],
                                f16=bool(c["flags"] & O.INPUT_F16)))


@pytest.mark.parametrize("seed", range(96))
def test_random_silu_mul_quant(seed):
    rng = np.random.default_rng(9100 + seed)
    mode = int(rng.integers(0, 4))
    G = {O.FP8_GROUP: int(rng.choice([64, 128])), O.FP4_BLOCK16: 16}.get(mode, 0)
    gran = max(G, 8)
    I = gran * int(rng.integers(1, max(2, 8192 // gran)))
    T = int(rng.integers(1, 40))
    flags = int(rng.choice([0, O.SCALE_COLMAJOR, O.SCALE_E8M0])) if mode == O.FP8_GROUP else 0
    x = rng.standard_normal((T, 2 * I)) * float(rng.choice([0.5, 3.0, 12.0]))
    xb = synth.bits(_bf16(x))
    a = O.silu_mul(xb)
    amax = float(np.abs(a).max()) or 1.0
    scale = 0.0
    if mode == O.FP8_STATIC:
        scale = float(np.float32(amax / 448 * rng.uniform(0.5, 2.0)))
    elif mode == O.FP4_BLOCK16:
        scale = float(np.float32(448 * 6 / amax * rng.uniform(0.5, 2.0)))
    launch = _random_launch(rng, I // 8)
    shape = None if launch is None else launch.as_tuple()
    print(f"[random] seed={seed} silu mode={mode} T={T} I={I} G={G} flags={flags} "
          f"launch={shape}", flush=True)
    gpu = GH.run_act(mode, synth.from_bits(xb).to("cuda"),
                     scale_in=scale if mode in (O.FP8_STATIC, O.FP4_BLOCK16) else None,
                     group_size=G, flags=flags, launch=launch)
    ref = O.silu_mul_quant(xb, mode, scale_in=scale, group_size=G, flags=flags, want_pre=True)
    raw = None
    if mode == O.FP8_GROUP and flags & O.SCALE_E8M0:
        raw = O.silu_mul_quant(xb, mode, group_size=G, flags=flags & O.SCALE_COLMAJOR)["scales"]
    compare(mode, gpu, ref, T=T, H=I, group_size=G, flags=flags, scale_in=scale,
            raw_group_scales=raw, y_ref=GH.y_ref_act(xb))


@pytest.mark.parametrize("seed", range(30))
def test_random_rms_norm_pad(seed):
    rng = np.random.default_rng(9200 + seed)
    H = 8 * int(rng.integers(1, 1200))
    ld = H + 8 * int(rng.integers(0, 40))
    T = int(rng.integers(1, 50))
    residual = bool(rng.random() < 0.7)
    x = rng.standard_normal((T, H)) * float(rng.choice([1e-2, 1.0, 50.0]))
    r = rng.standard_normal((T, H)) if residual else None
    w = rng.uniform(-1.5, 1.5, H)
    launch = _random_launch(rng, ld // 8)
    flags = O.INPUT_F16 if rng.random() < 0.3 else 0  # IEEE binary16 instead of bf16
    to16 = _to16(flags)
    xb, wb = to16(x), to16(w)
    rb = None if r is None else to16(r)
    shape = None if launch is None else launch.as_tuple()
    print(f"[random] seed={seed} pad T={T} H={H} ld={ld} residual={residual} launch={shape} "
          f"flags={flags}", flush=True)
    out = GH.Guarded(T * ld * 2)
    rout = GH.Guarded(T * H * 2) if residual else None
    B.rmsq_rms_norm_pad(synth.from_bits(xb).to("cuda"),
                        None if rb is None else synth.from_bits(rb).to("cuda"),
                        synth.from_bits(wb).to("cuda"), 1e-5, out.data.view(torch.bfloat16),
                        None if rout is None else rout.data.view(torch.bfloat16),
                        tokens=T, hidden=H, out_ld=ld, launch=launch, flags=flags)
    torch.cuda.synchronize()
    out.check("out")
    ref, rref = O.rms_norm_pad(xb, rb, wb, 1e-5, ld, flags=flags)
    assert np.array_equal(out.data.view(torch.int16).cpu().numpy().view(np.uint16).reshape(T, ld),
                          ref)
    if residual:
        rout.check("residual_out")
        assert np.array_equal(
            rout.data.view(torch.int16).cpu().numpy().view(np.uint16).reshape(T, H), rref)


@pytest.mark.parametrize("seed", range(36))
def test_random_qk_norm_rope(seed):
    rng = np.random.default_rng(9300 + seed)
    D = int(rng.choice([64, 128, 256]))
    hkv = int(rng.integers(1, 9))
    hq = hkv * int(rng.choice([1, 2, 4, 8]))
    T = int(rng.integers(1, 60))
    mp = int(rng.integers(1, 300))
    neox = bool(rng.random() < 0.5)
    qkv = rng.standard_normal((T, (hq + 2 * hkv) * D)) * float(rng.choice([0.1, 1.0, 20.0]))
    qw = rng.uniform(-1.5, 1.5, D)
    kw = rng.uniform(0.5, 1.5, D)
    pos = rng.integers(-3, mp + 3, T).astype(np.int64)
    cache = O.rope_cache(mp, D, float(rng.choice([1e4, 1e6])))
    hpl = hpb = 0
    if rng.random() < 0.6:
        L = D // 16
        hpl = int(rng.integers(1, 7))
        groups = int(rng.integers(1, 1024 // L + 1))
        hpb = hpl * groups
    flags = O.INPUT_F16 if rng.random() < 0.3 else 0  # IEEE binary16 instead of bf16
    to16 = _to16(flags)
    qkvb, qwb, kwb = to16(qkv), to16(qw), to16(kw)
    print(f"[random] seed={seed} rope T={T} hq={hq} hkv={hkv} D={D} neox={neox} mp={mp} "
          f"hpb={hpb} hpl={hpl} flags={flags}", flush=True)
    g = GH.Guarded(qkvb.size * 2)
    dev = g.data.view(torch.int16)
    dev.copy_(torch.from_numpy(qkvb.reshape(-1).view(np.int16)))
    B.rmsq_qk_norm_rope(dev, synth.from_bits(qwb).to("cuda"), synth.from_bits(kwb).to("cuda"),
                        torch.from_numpy(cache).to("cuda"), torch.from_numpy(pos).to("cuda"),
                        1e-6, hq, hkv, D, neox, tokens=T, heads_per_block=hpb,
                        heads_per_lane=hpl, flags=flags)
    torch.cuda.synchronize()
    g.check("qkv")
    got = dev.cpu().numpy().view(np.uint16).reshape(qkvb.shape)
    ref = O.qk_norm_rope(qkvb, qwb, kwb, cache, pos, 1e-6, hq, hkv, D, neox, flags=flags)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("seed", range(60))
def test_random_fp4_dynamic(seed):
    rng = np.random.default_rng(9400 + seed)
    H = 16 * int(rng.integers(1, 512))
    T = int(rng.integers(1, 60))
    residual = bool(rng.random() < 0.7)
    sigma = float(rng.choice([1e-3, 1.0, 30.0]))
    x = rng.standard_normal((T, H)) * sigma
    r = rng.standard_normal((T, H)) * sigma if residual else None
    w = rng.uniform(-1.5, 1.5, H)
    launch = _random_launch(rng, H // 8)
    flags = O.INPUT_F16 if rng.random() < 0.3 else 0
    to16 = _to16(flags)
    xb, wb = to16(x), to16(w)
    rb = None if r is None else to16(r)
    shape = None if launch is None else launch.as_tuple()
    print(f"[random] seed={seed} fp4dyn T={T} H={H} residual={residual} launch={shape} "
          f"flags={flags}", flush=True)
    gq, gsf, gg = GH.Guarded(T * H // 2), GH.Guarded(T * H // 16), GH.Guarded(4)
    grs = GH.Guarded(T * H * 2) if residual else None
    dev = (lambda b: None if b is None else synth.from_bits(b).to("cuda"))
    B.rmsq_fused_fp4_dynamic(dev(xb), dev(rb), dev(wb), 1e-6, gq.data, gsf.data,
                             None if grs is None else grs.data.view(torch.bfloat16),
                             gg.data.view(torch.float32), tokens=T, hidden=H, flags=flags,
                             launch=launch)
    torch.cuda.synchronize()
    for g, what in ((gq, "out_q"), (gsf, "out_scales"), (gg, "global_scale")):
        g.check(what)
    ref = O.fused_fp4_dynamic(xb, rb, wb, 1e-6, flags=flags, want_pre=True)
    gs = gg.data.view(torch.float32).cpu().numpy()[0]
    assert gs.view(np.uint32) == ref["global_scale"].view(np.uint32)
    gpu = {"q": gq.data.view(T, H // 2).cpu().numpy(),
           "scales": gsf.data.view(T, H // 16).cpu().numpy(),
           "residual_out": None if grs is None else
           grs.data.view(torch.int16).cpu().numpy().view(np.uint16).reshape(T, H)}
    if grs is not None:
        grs.check("residual_out")
    compare(O.FP4_BLOCK16, gpu, ref, T=T, H=H, group_size=16, scale_in=float(gs),
            y_ref=GH.y_ref_norm(xb, rb, wb, 1e-6, f16=bool(flags & O.INPUT_F16)))
