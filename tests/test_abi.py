"""The C ABI on the CPU: the library loads, exports every function include/rmsq.h declares,
and the host-side argument checks return the documented status for each kind of bad call.

Nothing here touches a device: rmsq_validate makes no HIP call, and rmsq_fused is only called
with arguments rmsq_validate has already rejected (it then returns the same status before
reaching the device)."""
import ctypes as C
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rmsq.h")


@pytest.fixture(scope="module")
def B():
    from rmsnorm_quantization_amd import binding, build

    if build.is_stale():
        build.build_library()
    binding.lib()
    return binding


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"RMSQ_API\s+[\w\s\*]*?\b(rmsq_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("rmsq_fused", "rmsq_fused_with_launch", "rmsq_fused_timed", "rmsq_validate",
              "rmsq_silu_mul_quant", "rmsq_silu_mul_quant_ex", "rmsq_silu_mul_quant_validate",
              "rmsq_silu_mul_query_launch", "rmsq_rms_norm_pad", "rmsq_rms_norm_pad_ex",
              "rmsq_rms_norm_pad_validate", "rmsq_rms_norm_pad_query_launch",
              "rmsq_qk_norm_rope", "rmsq_qk_norm_rope_ex",
              "rmsq_qk_norm_rope_validate", "rmsq_qk_norm_rope_query_launch",
              "rmsq_query_launch",
              "rmsq_block_to_rowblock", "rmsq_convert", "rmsq_status_string",
              "rmsq_abi_version"):
        assert n in names


def test_library_exports_every_declared_symbol(B):
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(\w+)$", out, flags=re.M))
    for n in declared_functions():
        assert n in exported, n
        assert hasattr(B.lib(), n)
    # nothing else leaks out of the library under an rmsq name
    assert {e for e in exported if "rmsq" in e} == set(declared_functions())


def test_abi_version_and_status_strings(B):
    assert B.rmsq_abi_version() == B.RMSQ_ABI_VERSION == 5
    for st in (0, -1, -2, -3, -4, -5, -6):
        assert B.rmsq_status_string(st) and B.rmsq_status_string(st) != "unknown status"
    assert B.rmsq_status_string(-99) == "unknown status"


# ------------------------------------------------------------------ argument checks
# Fake, well-separated, 256-byte-aligned addresses: never dereferenced.
X, R, W, Q, S, RO, SC = (0x10000000 * (i + 1) for i in range(7))
T, H = 4, 256


def V(B, x=X, r=R, w=W, eps=1e-6, mode=1, sc=None, q=Q, s=S, ro=RO, t=T, h=H, g=0, f=0, ld=0):
    return B.rmsq_validate(x, r, w, eps, mode, sc, q, s, ro, t, h, g, f, ld)


def test_valid_calls(B):
    assert V(B) == B.RMSQ_OK
    assert V(B, mode=0, sc=SC, s=None) == B.RMSQ_OK
    assert V(B, mode=2, g=128) == B.RMSQ_OK
    assert V(B, mode=2, g=64, f=B.RMSQ_SCALE_COLMAJOR | B.RMSQ_SCALE_E8M0, ld=8) == B.RMSQ_OK
    assert V(B, mode=3, g=16, sc=SC) == B.RMSQ_OK
    assert V(B, r=None, ro=None) == B.RMSQ_OK
    assert V(B, ro=R) == B.RMSQ_OK  # in-place residual
    assert V(B, t=0, x=None, q=None) == B.RMSQ_OK  # empty batch


@pytest.mark.parametrize("kw,status", [
    (dict(t=-1), "EINVAL"), (dict(h=0), "EINVAL"), (dict(h=12), "EINVAL"),
    (dict(h=65536 + 8), "EINVAL"), (dict(eps=0.0), "EINVAL"), (dict(eps=-1e-6), "EINVAL"),
    (dict(eps=float("inf")), "EINVAL"), (dict(eps=float("nan")), "EINVAL"),
    (dict(mode=4), "EINVAL"), (dict(mode=-1), "EINVAL"),
    (dict(x=None), "EINVAL"), (dict(w=None), "EINVAL"), (dict(q=None), "EINVAL"),
    (dict(ro=None), "EINVAL"), (dict(r=None), "EINVAL"),
    (dict(s=None), "EINVAL"), (dict(sc=SC), "EINVAL"),                    # token mode
    (dict(mode=0, s=None), "EINVAL"), (dict(mode=0, sc=SC), "EINVAL"),    # static: scales
    (dict(mode=0, sc=SC, s=None, g=64), "EINVAL"),
    (dict(mode=2, g=32), "EINVAL"), (dict(mode=2, g=128, h=192), "EINVAL"),
    (dict(mode=2, g=0), "EINVAL"), (dict(mode=3, g=16), "EINVAL"),         # fp4 needs gs
    (dict(mode=3, sc=SC, g=8), "EINVAL"), (dict(mode=3, sc=SC, g=16, h=264), "EINVAL"),
    (dict(mode=2, g=64, f=1, ld=3), "EINVAL"),                    # ld < T
    (dict(mode=2, g=64, ld=8), "EINVAL"),                                  # ld without colmajor
    (dict(f=1), "EUNSUPPORTED"), (dict(mode=3, sc=SC, g=16, f=2), "EUNSUPPORTED"),
    (dict(mode=2, g=64, f=8), "EUNSUPPORTED"), (dict(mode=2, g=64, f=6), "EUNSUPPORTED"),
    (dict(x=X + 8), "EALIGN"), (dict(w=W + 4), "EALIGN"), (dict(r=R + 2), "EALIGN"),
    (dict(ro=RO + 8), "EALIGN"), (dict(q=Q + 4), "EALIGN"), (dict(s=S + 2), "EALIGN"),
    (dict(mode=0, s=None, sc=SC + 1), "EALIGN"), (dict(mode=3, g=16, sc=SC, q=Q + 2), "EALIGN"),
    (dict(q=X), "EALIAS"), (dict(s=X + 16), "EALIAS"), (dict(ro=X), "EALIAS"),
    (dict(q=W), "EALIAS"), (dict(q=R), "EALIAS"), (dict(ro=R + 16), "EALIAS"),
    (dict(s=Q + 16), "EALIAS"), (dict(ro=Q), "EALIAS"), (dict(mode=0, s=None, sc=Q), "EALIAS"),
    (dict(s=R), "EALIAS"),
])
def test_bad_arguments(B, kw, status):
    code = getattr(B, "RMSQ_" + status)
    assert V(B, **kw) == code
    # rmsq_fused returns the same status without going near a device
    assert B.lib().rmsq_fused(kw.get("x", X), kw.get("r", R), kw.get("w", W),
                              kw.get("eps", 1e-6), kw.get("mode", 1), kw.get("sc", None),
                              kw.get("q", Q), kw.get("s", S), kw.get("ro", RO), kw.get("t", T),
                              kw.get("h", H), kw.get("g", 0), kw.get("f", 0), kw.get("ld", 0),
                              None) == code


def test_colmajor_scale_extent_is_checked(B):
    # col-major scales [H/G, ld]: the last column of the last group ends at ((ng-1)*ld + T)*4
    ng, ld = H // 64, 16
    end = ((ng - 1) * ld + T) * 4
    assert V(B, mode=2, g=64, f=1, ld=ld, s=S, q=S + end) == B.RMSQ_OK
    assert V(B, mode=2, g=64, f=1, ld=ld, s=S, q=S + end - 16) == B.RMSQ_EALIAS


def test_query_launch(B):
    for h in (8, 64, 1024, 2048, 2880, 4096, 5120, 7168, 8192, 16384, 65536):
        l, grid = B.rmsq_query_launch(1, 1000, h)
        tpr, vpt, rpb, _ = l.as_tuple()
        assert tpr % 64 == 0 and 64 <= tpr <= 1024
        assert 1 <= vpt <= 8 and tpr * vpt * 8 >= h
        assert rpb >= 1 and rpb * tpr <= 1024
        assert grid == -(-1000 // rpb)
    with pytest.raises(B.RmsqError):
        B.rmsq_query_launch(1, 10, 12)


def test_query_launch_takes_the_calls_flags(B):
    """The query checks the flags as rmsq_fused does; the shape depends on T and H only."""
    base = B.rmsq_query_launch(2, 1024, 5120, 128)[0].as_tuple()
    for f in (B.RMSQ_SCALE_COLMAJOR, B.RMSQ_SCALE_E8M0, B.RMSQ_SCALE_E8M0_U8,
              B.RMSQ_SCALE_COLMAJOR | B.RMSQ_SCALE_E8M0, B.RMSQ_INPUT_F16,
              B.RMSQ_INPUT_F16 | B.RMSQ_SCALE_COLMAJOR):
        assert B.rmsq_query_launch(2, 1024, 5120, 128, f)[0].as_tuple() == base
    for mode, G in ((0, 0), (1, 0), (3, 16)):
        plain = B.rmsq_query_launch(mode, 4096, 2048, G)[0].as_tuple()
        assert B.rmsq_query_launch(mode, 4096, 2048, G, B.RMSQ_INPUT_F16)[0].as_tuple() == plain
        with pytest.raises(B.RmsqError):  # scale-layout flags belong to the per-group mode
            B.rmsq_query_launch(mode, 4096, 2048, G, B.RMSQ_SCALE_COLMAJOR)
    with pytest.raises(B.RmsqError):
        B.rmsq_query_launch(2, 1024, 5120, 128, B.RMSQ_SCALE_E8M0 | B.RMSQ_SCALE_E8M0_U8)


@pytest.mark.parametrize("T,H,shape", [
    (4096, 2048, (64, 4, 1, 0)),     # in flight at once: one wave per row (per-token)
    (1024, 2048, (64, 4, 1, 0)),
    (2048, 1536, (64, 3, 1, 0)),
    (8192, 2048, (128, 2, 1, 0)),    # more than 2^20 chunks: several waves per row
    (1024, 4096, (256, 2, 1, 0)),    # rows of more than four waves' worth of chunks
    (2048, 4096, (256, 2, 1, 0)),
    (1023, 2048, (128, 2, 1, 0)),    # below 1024 rows
    (64, 2048, (128, 2, 1, 0)),
    (1024, 2880, (192, 2, 1, 0)),    # rows that do not fill whole waves
    (1024, 5120, (320, 2, 1, 0)),    # longer than one wave's 8 chunks per lane
    (4096, 1024, (64, 2, 4, 0)),     # short rows: four to a workgroup
])
def test_query_launch_batch_rule(B, T, H, shape):
    """The per-token scheme's shapes; the others take the plain per-H default except where the
    per-token batch rule gives one wave per row (H 1536 = 64 x 3 is that default anyway)."""
    l, grid = B.rmsq_query_launch(B.RMSQ_FP8_TOKEN, T, H, 0)
    assert l.as_tuple() == shape
    assert grid == -(-T // shape[2])
    plain = (128, 2, 1, 0) if H == 2048 else shape
    G128 = 128 if H % 128 == 0 else 64
    for mode, G in ((B.RMSQ_FP8_STATIC, 0), (B.RMSQ_FP8_GROUP, G128), (B.RMSQ_FP4_BLOCK16, 16)):
        l, grid = B.rmsq_query_launch(mode, T, H, G)
        assert l.as_tuple() == plain, (mode, l.as_tuple())
        assert grid == -(-T // plain[2])


@pytest.mark.parametrize("grid", [1, 2, 7, 8, 9, 15, 16, 17, 255, 256, 1000, 4096, 16385])
def test_block_to_rowblock_is_a_bijection(B, grid):
    got = [B.rmsq_block_to_rowblock(b, grid) for b in range(grid)]
    assert sorted(got) == list(range(grid))
    # each XCD (b % 8) gets one contiguous run of row blocks
    for x in range(8):
        mine = [got[b] for b in range(x, grid, 8)]
        assert mine == list(range(mine[0], mine[0] + len(mine))) if mine else True
    assert B.rmsq_block_to_rowblock(grid, grid) == -1


def test_convert_argument_checks(B):
    L = B.lib()
    assert L.rmsq_convert(7, X, Q, 8, None) == B.RMSQ_EINVAL
    assert L.rmsq_convert(5, X, Q, 8, None) == B.RMSQ_EINVAL
    assert L.rmsq_convert(B.RMSQ_CVT_E4M3_IN_RANGE, X, X + 16, 8, None) == B.RMSQ_EALIAS
    assert L.rmsq_convert(B.RMSQ_CVT_E4M3_IN_RANGE, X, Q, 12, None) == B.RMSQ_EINVAL
    assert L.rmsq_convert(0, X, Q, 12, None) == B.RMSQ_EINVAL
    assert L.rmsq_convert(0, X, Q, 0, None) == B.RMSQ_OK
    assert L.rmsq_convert(0, X + 4, Q, 8, None) == B.RMSQ_EALIGN
    assert L.rmsq_convert(0, X, X + 16, 8, None) == B.RMSQ_EALIAS
    # the inverse-RMS output is 4 bytes per value: 32 bytes just below the 8 inputs overlap
    # them from 16 bytes below, where 8 e4m3 bytes do not
    assert L.rmsq_convert(3, X, X - 16, 8, None) == B.RMSQ_EALIAS
    assert L.rmsq_convert(0, X, X - 16, 8, None) != B.RMSQ_EALIAS
    assert L.rmsq_convert(3, X, X - 32, 8, None) != B.RMSQ_EALIAS


# ------------------------------------------------------------------ SiLU+Mul -> quant checks
def VA(B, x=X, mode=1, sc=None, q=Q, s=S, t=T, i=H, g=0, f=0, ld=0):
    return B.rmsq_silu_mul_quant_validate(x, mode, sc, q, s, t, i, g, f, ld)


def test_act_valid_calls(B):
    assert VA(B) == B.RMSQ_OK
    assert VA(B, mode=0, sc=SC, s=None) == B.RMSQ_OK
    assert VA(B, mode=2, g=64, f=B.RMSQ_SCALE_COLMAJOR | B.RMSQ_SCALE_E8M0_U8, ld=9) == B.RMSQ_OK
    assert VA(B, mode=3, g=16, sc=SC) == B.RMSQ_OK
    assert VA(B, t=0, x=None, q=None) == B.RMSQ_OK


@pytest.mark.parametrize("kw,status", [
    (dict(t=-1), "EINVAL"), (dict(i=12), "EINVAL"), (dict(i=0), "EINVAL"),
    (dict(i=65536 + 8), "EINVAL"), (dict(mode=5), "EINVAL"), (dict(x=None), "EINVAL"),
    (dict(q=None), "EINVAL"), (dict(s=None), "EINVAL"), (dict(sc=SC), "EINVAL"),
    (dict(mode=2, g=128, i=192), "EINVAL"), (dict(mode=3, g=16), "EINVAL"),
    (dict(f=1), "EUNSUPPORTED"), (dict(mode=2, g=64, f=6), "EUNSUPPORTED"),
    (dict(x=X + 8), "EALIGN"), (dict(q=Q + 4), "EALIGN"), (dict(s=S + 1), "EALIGN"),
    # x spans T * 2I bf16 = 4 * T * I bytes
    (dict(q=X + 4 * T * H - 16), "EALIAS"), (dict(s=X + 16), "EALIAS"), (dict(s=Q + 8), "EALIAS"),
    (dict(mode=0, s=None, sc=Q), "EALIAS"),
])
def test_act_bad_arguments(B, kw, status):
    code = getattr(B, "RMSQ_" + status)
    assert VA(B, **kw) == code
    assert B.lib().rmsq_silu_mul_quant(kw.get("x", X), kw.get("mode", 1), kw.get("sc", None),
                                       kw.get("q", Q), kw.get("s", S), kw.get("t", T),
                                       kw.get("i", H), kw.get("g", 0), kw.get("f", 0),
                                       kw.get("ld", 0), None) == code


def test_act_x_extent_is_two_rows_wide(B):
    assert VA(B, q=X + 4 * T * H) == B.RMSQ_OK   # just past x [T, 2I] bf16


def test_act_query_launch(B):
    l, grid = B.rmsq_silu_mul_query_launch(B.RMSQ_FP8_TOKEN, 100, 14336)
    assert l.options == 0 and l.threads_per_row * l.chunks_per_thread * 8 >= 14336
    for mode, G in ((B.RMSQ_FP8_STATIC, 0), (B.RMSQ_FP8_GROUP, 128)):
        l, grid = B.rmsq_silu_mul_query_launch(mode, 100, 14336, G)
        assert l.as_tuple() == B.rmsq_query_launch(mode, 100, 14336, G)[0].as_tuple()
        assert grid == -(-100 // l.rows_per_block)
    # FP4: tiles of one wave x 2 chunks, 14 to a 1792-chunk row (11 at I = 11008, the last one partial)
    l, grid = B.rmsq_silu_mul_query_launch(B.RMSQ_FP4_BLOCK16, 100, 14336, 16)
    assert l.as_tuple() == (64, 2, 1, B.RMSQ_LAUNCH_ROW_TILES) and grid == 100 * 14
    l, grid = B.rmsq_silu_mul_query_launch(B.RMSQ_FP4_BLOCK16, 100, 11008, 16)
    assert l.as_tuple() == (64, 2, 1, B.RMSQ_LAUNCH_ROW_TILES) and grid == 100 * 11


# ------------------------------------------------------------------ RMSNorm -> padded bf16
def VP(B, x=X, r=R, w=W, eps=1e-6, out=Q, ro=RO, t=T, h=H, ld=H + 64, f=0):
    return B.rmsq_rms_norm_pad_validate(x, r, w, eps, out, ro, t, h, ld, f)


def test_pad_query_launch(B):
    l, grid = B.rmsq_rms_norm_pad_query_launch(4096, 2880, 3072)
    assert l.as_tuple() == (64, 6, 1, 0) and grid == 4096   # one wave per padded row
    # binary16 rows take one wave per row only up to 6 chunks per lane
    l, grid = B.rmsq_rms_norm_pad_query_launch(4096, 2880, 3072, B.RMSQ_INPUT_F16)
    assert l.as_tuple() == (64, 6, 1, 0) and grid == 4096
    l, _ = B.rmsq_rms_norm_pad_query_launch(64, 4000, 4096, B.RMSQ_INPUT_F16)
    assert l.as_tuple() == (256, 2, 1, 0)
    l, _ = B.rmsq_rms_norm_pad_query_launch(64, 4000, 4096)
    assert l.as_tuple() == (64, 8, 1, 0)
    with pytest.raises(B.RmsqError):
        B.rmsq_rms_norm_pad_query_launch(4, 64, 64, 1 << 7)
    l, grid = B.rmsq_rms_norm_pad_query_launch(100, 8192, 8192)
    assert l.as_tuple() == B.rmsq_query_launch(0, 100, 8192, 0)[0].as_tuple()
    l, _ = B.rmsq_rms_norm_pad_query_launch(8, 520, 1024)
    assert l.threads_per_row * l.chunks_per_thread * 8 >= 1024
    for bad in ((4, 2880, 2872), (4, 12, 16), (-1, 64, 64), (4, 64, 65536 + 8)):
        with pytest.raises(B.RmsqError):
            B.rmsq_rms_norm_pad_query_launch(*bad)


def test_pad_valid_calls(B):
    assert VP(B) == B.RMSQ_OK
    assert VP(B, ld=H) == B.RMSQ_OK
    assert VP(B, r=None, ro=None) == B.RMSQ_OK
    assert VP(B, ro=R) == B.RMSQ_OK
    assert VP(B, t=0, x=None, out=None) == B.RMSQ_OK


@pytest.mark.parametrize("kw,status", [
    (dict(ld=H - 8), "EINVAL"), (dict(ld=H + 4), "EINVAL"), (dict(ld=65536 + 8), "EINVAL"),
    (dict(h=12), "EINVAL"), (dict(eps=0.0), "EINVAL"), (dict(t=-1), "EINVAL"),
    (dict(out=None), "EINVAL"), (dict(ro=None), "EINVAL"), (dict(x=None), "EINVAL"),
    (dict(out=Q + 8), "EALIGN"), (dict(x=X + 2), "EALIGN"), (dict(ro=RO + 4), "EALIGN"),
    (dict(out=X), "EALIAS"), (dict(out=W), "EALIAS"), (dict(out=R), "EALIAS"),
    (dict(ro=Q), "EALIAS"), (dict(ro=X + 16), "EALIAS"), (dict(ro=R + 16), "EALIAS"),
    # out spans T * ld * 2 bytes
    (dict(ro=Q + T * (H + 64) * 2 - 16), "EALIAS"),
])
def test_pad_bad_arguments(B, kw, status):
    code = getattr(B, "RMSQ_" + status)
    assert VP(B, **kw) == code
    assert B.lib().rmsq_rms_norm_pad(kw.get("x", X), kw.get("r", R), kw.get("w", W),
                                     kw.get("eps", 1e-6), kw.get("out", Q), kw.get("ro", RO),
                                     kw.get("t", T), kw.get("h", H), kw.get("ld", H + 64),
                                     0, None) == code


# ------------------------------------------------------------------ QK-norm + RoPE
HQ, HKV, D, MP = 4, 2, 128, 64
QKV, QW, KW, CS, POS = X, W, R, S, SC


def VR(B, qkv=QKV, qw=QW, kw=KW, cs=CS, pos=POS, eps=1e-6, t=T, hq=HQ, hkv=HKV, d=D, mp=MP,
       f=0):
    return B.rmsq_qk_norm_rope_validate(qkv, qw, kw, cs, pos, eps, t, hq, hkv, d, mp, f)


def test_rope_valid_calls(B):
    assert VR(B) == B.RMSQ_OK
    for d in (64, 256):
        assert VR(B, d=d) == B.RMSQ_OK
    assert VR(B, qw=KW) == B.RMSQ_OK                     # q and k may share one weight
    assert VR(B, t=0, qkv=None, pos=None) == B.RMSQ_OK
    assert VR(B, hq=64, hkv=8, d=128) == B.RMSQ_OK
    # qkv spans T * (Hq + 2 Hkv) * D * 2 bytes: a neighbour just past it is fine
    assert VR(B, pos=QKV + T * (HQ + 2 * HKV) * D * 2) == B.RMSQ_OK


@pytest.mark.parametrize("kw,status", [
    (dict(d=96), "EINVAL"), (dict(d=32), "EINVAL"), (dict(d=512), "EINVAL"),
    (dict(hq=0), "EINVAL"), (dict(hkv=0), "EINVAL"), (dict(hq=4096, d=256), "EINVAL"),
    (dict(mp=0), "EINVAL"), (dict(eps=0.0), "EINVAL"), (dict(eps=float("nan")), "EINVAL"),
    (dict(t=-1), "EINVAL"), (dict(t=1 << 31), "EINVAL"),
    (dict(qkv=None), "EINVAL"), (dict(qw=None), "EINVAL"), (dict(kw=None), "EINVAL"),
    (dict(cs=None), "EINVAL"), (dict(pos=None), "EINVAL"),
    (dict(qkv=QKV + 8), "EALIGN"), (dict(qw=QW + 2), "EALIGN"), (dict(cs=CS + 4), "EALIGN"),
    (dict(pos=POS + 4), "EALIGN"),
    (dict(qw=QKV), "EALIAS"), (dict(cs=QKV + 16), "EALIAS"), (dict(pos=QKV + 256), "EALIAS"),
    (dict(pos=QKV + T * (HQ + 2 * HKV) * D * 2 - 8), "EALIAS"),
    (dict(kw=QKV - 16), "EALIAS"),
])
def test_rope_bad_arguments(B, kw, status):
    code = getattr(B, "RMSQ_" + status)
    assert VR(B, **kw) == code
    a = dict(qkv=QKV, qw=QW, kw=KW, cs=CS, pos=POS, eps=1e-6, t=T, hq=HQ, hkv=HKV, d=D, mp=MP)
    a.update(kw)
    assert B.lib().rmsq_qk_norm_rope(a["qkv"], a["qw"], a["kw"], a["cs"], a["pos"], a["eps"],
                                     a["t"], a["hq"], a["hkv"], a["d"], a["mp"], 1, 0,
                                     None) == code


def test_rope_launch_shape_is_checked(B):
    """Bad explicit shapes are rejected before any device call."""
    def ex(hpb, hpl):
        return B.lib().rmsq_qk_norm_rope_ex(QKV, QW, KW, CS, POS, 1e-6, T, HQ, HKV, D, MP, 1, 0,
                                            hpb, hpl, None, None, None)
    L = D // 16
    for hpb, hpl in ((1024 // L + 1, 1), (6, 4), (-1, 1), (4, -1), (0, 2), (2, 0), (7, 7),
                     (16, 8), (2 * (1024 // L + 1), 2)):
        assert ex(hpb, hpl) == B.RMSQ_EINVAL, (hpb, hpl)


@pytest.mark.parametrize("hq,hkv,d", [(32, 8, 128), (64, 8, 128), (16, 8, 64), (8, 1, 256),
                                      (40, 8, 128), (1, 1, 128), (28, 4, 128), (12, 4, 64)])
def test_rope_query_launch(B, hq, hkv, d):
    hpb, hpl, grid = B.rmsq_qk_norm_rope_query_launch(1000, hq, hkv, d)
    nh, L = hq + hkv, d // 16
    groups = hpb // hpl
    assert 1 <= hpl <= 6 and hpb % hpl == 0 and groups * L <= 1024
    assert (groups * L) % 64 == 0 or hpb >= nh   # whole waves unless one workgroup per token
    assert hpb - hpl < nh                          # every lane group has a head
    assert grid == 1000 * -(-nh // hpb)
    with pytest.raises(B.RmsqError):
        B.rmsq_qk_norm_rope_query_launch(1000, hq, hkv, 96)


def test_rope_default_shape_follows_the_batch(B):
    """Small batches get one head per lane (more, shorter waves), batches that fill the chip
    once the most heads per lane that fit, larger ones two heads per lane in single-wave
    workgroups -- for the 32 q + 8 kv heads of size 128 layout."""
    assert B.rmsq_qk_norm_rope_query_launch(1, 32, 8, 128)[:2] == (40, 1)
    assert B.rmsq_qk_norm_rope_query_launch(256, 32, 8, 128)[:2] == (40, 1)
    assert B.rmsq_qk_norm_rope_query_launch(4096, 32, 8, 128)[:2] == (40, 5)
    assert B.rmsq_qk_norm_rope_query_launch(16384, 32, 8, 128)[:2] == (16, 2)


# ------------------------------------------------------------------ measurement probe library
def test_probe_library_exports_and_checks_arguments():
    """librmsq_probe.so (include/rmsq_probe.h) exports exactly its entry point and rejects bad
    shapes on the host before any device call."""
    import ctypes

    from rmsnorm_quantization_amd import build

    if build.probe_is_stale():
        build.build_probe_library()
    out = subprocess.run(["nm", "-D", "--defined-only", build.PROBE_LIB], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(\w+)$", out, flags=re.M))
    assert {e for e in exported if "rmsq" in e} == {"rmsq_probe_stream"}
    L = ctypes.CDLL(build.PROBE_LIB)
    p = ctypes.c_void_p
    i32 = ctypes.c_int
    L.rmsq_probe_stream.argtypes = [p, p, p, p, p, ctypes.c_int64, ctypes.c_int64, i32, i32, i32,
                                    i32, i32, p, p, p]

    def call(rows=4, hidden=4096, out1=8, tpr=256, vpt=2, a=X, b=R, c=RO, d=Q, e=None, shift=0,
             eb=4):
        return L.rmsq_probe_stream(a, b, c, d, e, rows, hidden, out1, shift, eb, tpr, vpt, None,
                                   None, None)

    assert call(rows=0) == 0
    assert call(rows=0, e=SC, shift=4) == 0 and call(rows=0, e=SC, shift=-1) == 0
    for kw in (dict(hidden=4000), dict(tpr=96), dict(tpr=2048, vpt=1, hidden=16384),
               dict(vpt=9), dict(tpr=256, vpt=3), dict(out1=2), dict(rows=-1), dict(a=None),
               dict(e=SC, shift=7), dict(e=SC, shift=-2), dict(e=SC, eb=2)):
        assert call(**kw) == -1, kw
    assert call(a=X + 8) == -2 and call(d=Q + 4) == -2 and call(e=SC + 2, shift=3) == -2
    assert call(rows=0, e=SC + 1, eb=1) == 0  # a byte stream needs no alignment


def test_input_f16_flag_is_accepted_by_the_quantizing_ops(B):
    F = B.RMSQ_INPUT_F16
    assert V(B, mode=B.RMSQ_FP8_TOKEN, f=F) == B.RMSQ_OK
    assert V(B, mode=B.RMSQ_FP8_STATIC, sc=SC, s=None, f=F) == B.RMSQ_OK
    assert V(B, mode=B.RMSQ_FP8_GROUP, g=128, f=F | B.RMSQ_SCALE_COLMAJOR) == B.RMSQ_OK
    assert V(B, mode=B.RMSQ_FP4_BLOCK16, sc=SC, g=16, f=F) == B.RMSQ_OK
    assert V(B, mode=B.RMSQ_FP8_TOKEN, f=F | (1 << 9)) == B.RMSQ_EUNSUPPORTED
    assert VA(B, f=F) == B.RMSQ_OK
    assert VA(B, mode=B.RMSQ_FP8_GROUP, g=128, f=F | B.RMSQ_SCALE_E8M0) == B.RMSQ_OK
    assert VA(B, f=F | (1 << 9)) == B.RMSQ_EUNSUPPORTED


def test_input_f16_flag_for_padding_and_rope(B):
    """The padded-output and QK-norm + RoPE ops take RMSQ_INPUT_F16 (binary16 activations and
    weights); any other flag bit is refused before any device call, by the entry points too."""
    F = B.RMSQ_INPUT_F16
    assert VP(B, f=F) == B.RMSQ_OK and VP(B, r=None, ro=None, f=F) == B.RMSQ_OK
    assert VR(B, f=F) == B.RMSQ_OK
    for bad in (1, 1 << 9, F | 2):
        assert VP(B, f=bad) == B.RMSQ_EUNSUPPORTED
        assert VR(B, f=bad) == B.RMSQ_EUNSUPPORTED
        assert B.lib().rmsq_rms_norm_pad(X, R, W, 1e-6, Q, RO, T, H, H + 64, bad,
                                         None) == B.RMSQ_EUNSUPPORTED
        assert B.lib().rmsq_qk_norm_rope(QKV, QW, KW, CS, POS, 1e-6, T, HQ, HKV, D, MP, 1, bad,
                                         None) == B.RMSQ_EUNSUPPORTED


# ------------------------------------------------------------------ FP4 with a batch global scale
GSO = SC  # the global scale output


def VD(B, x=X, r=R, w=W, eps=1e-6, q=Q, s=S, ro=RO, gs=GSO, t=T, h=H, f=0):
    return B.rmsq_fused_fp4_dynamic_validate(x, r, w, eps, q, s, ro, gs, t, h, f)


def test_fp4_dynamic_valid_calls(B):
    assert VD(B) == B.RMSQ_OK
    assert VD(B, r=None, ro=None) == B.RMSQ_OK
    assert VD(B, ro=R) == B.RMSQ_OK                          # new residual in place
    assert VD(B, f=B.RMSQ_INPUT_F16) == B.RMSQ_OK
    assert VD(B, t=0, x=None, q=None, s=None, gs=None) == B.RMSQ_OK
    assert VD(B, gs=X + T * H * 2) == B.RMSQ_OK              # just past x


@pytest.mark.parametrize("kw,status", [
    (dict(h=264), "EINVAL"), (dict(h=8), "EINVAL"), (dict(t=-1), "EINVAL"),
    (dict(eps=0.0), "EINVAL"), (dict(gs=None), "EINVAL"), (dict(s=None), "EINVAL"),
    (dict(q=None), "EINVAL"), (dict(ro=None), "EINVAL"), (dict(x=None), "EINVAL"),
    (dict(f=1), "EUNSUPPORTED"), (dict(f=4), "EUNSUPPORTED"), (dict(f=1 << 9), "EUNSUPPORTED"),
    (dict(gs=GSO + 2), "EALIGN"), (dict(q=Q + 2), "EALIGN"), (dict(x=X + 8), "EALIGN"),
    (dict(gs=X + 64), "EALIAS"), (dict(gs=W), "EALIAS"), (dict(gs=R + 4), "EALIAS"),
    (dict(gs=Q + 8), "EALIAS"), (dict(gs=S), "EALIAS"), (dict(gs=RO + 4), "EALIAS"),
    (dict(q=X), "EALIAS"), (dict(s=R), "EALIAS"), (dict(ro=W), "EALIAS"),
])
def test_fp4_dynamic_bad_arguments(B, kw, status):
    code = getattr(B, "RMSQ_" + status)
    assert VD(B, **kw) == code
    a = dict(x=X, r=R, w=W, eps=1e-6, q=Q, s=S, ro=RO, gs=GSO, t=T, h=H, f=0)
    a.update(kw)
    assert B.lib().rmsq_fused_fp4_dynamic(a["x"], a["r"], a["w"], a["eps"], a["q"], a["s"],
                                          a["ro"], a["gs"], a["t"], a["h"], a["f"],
                                          None) == code
    shape = B.rmsq_launch(64, 1, 1, 0)  # a valid shape: the status is the argument check's
    assert B.lib().rmsq_fused_fp4_dynamic_ex(a["x"], a["r"], a["w"], a["eps"], a["q"], a["s"],
                                             a["ro"], a["gs"], a["t"], a["h"], a["f"],
                                             C.byref(shape), None, None, None) == code


def test_fp4_dynamic_launch_shape_is_checked(B):
    short = B.rmsq_launch(64, 1, 1, 0)  # 512 elements: too few for H = 1024
    assert B.lib().rmsq_fused_fp4_dynamic_ex(X, R, W, 1e-6, Q, S, RO, GSO, T, 1024, 0,
                                             C.byref(short), None, None,
                                             None) == B.RMSQ_EINVAL
