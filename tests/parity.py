"""GPU-vs-oracle comparison rule for fused RMSNorm + quantization (test infrastructure).

The bar, per output:
  residual_out   bit-exact.
  codes          equal, or the adjacent magnitude with the same sign (+0 and -0 count as
                 equal); a mismatch is only accepted where the value it was encoded from lies
                 within 1e-5 (relative) of the rounding midpoint between the two codes.
  scales         f32 scales within 1e-6 relative.  An E8M0 scale may differ by a factor 2 only
                 where the unrounded scale absmax/448 lies within 1e-6 (relative) of a power of
                 two; an FP4 e4m3 block scale may differ by one code only where its unrounded
                 value (absmax * gs) / 6 lies within 1e-6 (relative) of the rounding midpoint
                 between the two codes.  The codes of such a group or block are compared, by the
                 code rule above, with the oracle's y re-quantized at the GPU's scale.
  budget         code mismatches plus scale flips at most 0.01% of the elements.
  dequantized    FP8: per row, ||dq_gpu - dq_ref||_2 <= 1e-2 * ||dq_ref||_2 (a relative error
                 of the dequantized row; a per-element bound cannot hold, since an allowed
                 one-code tie flip near 448 is a ~7% change of that element).  FP4: per element
                 within one e2m1 step * d / gs.
Why ties can differ at all: the GPU sums squares in a different order than the oracle, so
inv_rms may differ in its last bit (and SiLU uses a short exp, a few ulp from the exactly rounded
activation), and a value sitting on a rounding midpoint can then land on either neighbour.
For the norm path the binary64 sums agree after rounding to f32 and the counts come out zero;
the rule is what is asserted.
"""
from dataclasses import dataclass, field

import numpy as np

import oracle as O

MAX_MISMATCH_FRAC = 1e-4
MID_REL = 1e-5
SCALE_REL = 1e-6
DEQ_REL = 1e-2

_E4 = None
_E2 = None


def e4_table():
    global _E4
    if _E4 is None:
        _E4 = O.e4m3_table().astype(np.float64)
    return _E4


def e2_table():
    global _E2
    if _E2 is None:
        _E2 = O.e2m1_table().astype(np.float64)
    return _E2


@dataclass
class Report:
    elements: int = 0
    code_mismatch: int = 0
    scale_mismatch: int = 0   # f32 scales that differ (within 1e-6), E8M0 / e4m3 scale flips
    scale_flips: int = 0      # E8M0 factor-2 flips and FP4 one-code block-scale flips
    residual_mismatch: int = 0
    max_dequant_rel: float = 0.0
    notes: list = field(default_factory=list)

    def __str__(self):
        return (f"elements={self.elements} code_mismatch={self.code_mismatch} "
                f"scale_mismatch={self.scale_mismatch} scale_flips={self.scale_flips} "
                f"residual_mismatch={self.residual_mismatch} "
                f"max_dequant_rel={self.max_dequant_rel:.3g}")


def _codes_ok(qg, qr, pre, fmt, rep: Report):
    """Rule 2 on code arrays of one shape (FP4 as nibbles); pre: the value each reference code
    was encoded from."""
    if np.array_equal(qg, qr):
        return
    signbit = 0x80 if fmt == "e4m3" else 0x8
    magmask = 0x7F if fmt == "e4m3" else 0x7
    tab = e4_table() if fmt == "e4m3" else e2_table()
    qg = qg.astype(np.int64)
    qr = qr.astype(np.int64)
    mg, mr = qg & magmask, qr & magmask
    same = (qg == qr) | ((mg == 0) & (mr == 0))
    bad = ~same
    n = int(bad.sum())
    rep.code_mismatch += n
    if n == 0:
        return
    sg, sr = qg[bad] & signbit, qr[bad] & signbit
    assert np.all((sg == sr) | (mg[bad] == 0) | (mr[bad] == 0)), "code mismatch with sign flip"
    assert np.all(np.abs(mg[bad] - mr[bad]) == 1), "code mismatch by more than one code"
    lo = np.minimum(mg[bad], mr[bad])
    mid = (tab[lo] + tab[lo + 1]) / 2
    p = np.abs(pre[bad].astype(np.float64))
    assert np.all(np.abs(p - mid) <= MID_REL * mid), "code mismatch away from a rounding midpoint"


def _scaled(y, mul):
    """The value a code is encoded from (the oracle's rule): y * mul in f32, a zero y staying
    the zero it is."""
    y = np.asarray(y, np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        v = (y * np.float32(mul)).astype(np.float32)
    return np.where(y == 0, y, v)


def _requant_fp8(y_group, s):
    """The oracle's FP8 encoding of one group's y at scale s (a zero scale gives zero codes)."""
    if s == 0:
        return np.zeros(y_group.shape, np.uint8), np.zeros(y_group.shape, np.float32)
    with np.errstate(divide="ignore", over="ignore"):
        r = np.float32(1) / np.float32(s)
    v = _scaled(y_group, r)
    return O.e4m3_encode(v), v


def _requant_fp4(y_block, sf, gs):
    """The oracle's e2m1 encoding of one 16-block's y at block scale byte sf and global gs."""
    d = np.float32(e4_table()[sf])
    if not d > 0:
        return np.zeros(16, np.uint8), np.zeros(16, np.float32)
    with np.errstate(divide="ignore", over="ignore"):
        m = np.float32(gs) / d
    v = _scaled(y_block, m)
    return O.e2m1_encode(v), v


def compare(mode, gpu, ref, *, T, H, group_size=0, flags=0, scale_in=0.0, rows=None,
            raw_group_scales=None, y_ref=None) -> Report:
    """Assert the rule above.  gpu/ref are dicts with q, scales, residual_out (numpy, as the
    oracle lays them out); ref also has pre.  rows: which of the T rows were computed (the
    arrays are then already restricted to them; col-major scales are [H/G, len(rows)]).
    raw_group_scales: the oracle's unrounded per-group scales absmax/448 (E8M0 modes).
    y_ref(rows): the oracle's normalized f32 rows y for the given row indices (into the compared
    arrays); needed only where a scale flipped."""
    rep = Report(elements=T * H)
    if ref.get("residual_out") is not None:
        rb = int((gpu["residual_out"] != ref["residual_out"]).sum())
        rep.residual_mismatch = rb
        assert rb == 0, f"residual_out differs in {rb} elements"

    pre = ref["pre"]
    qr_cmp = None  # the reference codes after re-quantizing flipped groups at the GPU's scale

    if mode == O.FP4_BLOCK16:
        sg, sr = gpu["scales"].astype(np.int64), ref["scales"].astype(np.int64)  # [T, H/16]
        ng, nr = O.unpack_fp4(gpu["q"]), O.unpack_fp4(ref["q"])
        diff = sg != sr
        rep.scale_mismatch = rep.scale_flips = int(diff.sum())
        nr_cmp, pre_cmp = nr.copy(), pre.copy()
        if rep.scale_flips:
            assert np.all(np.abs(sg[diff] - sr[diff]) == 1), "FP4 block scale off by > 1 code"
            assert y_ref is not None, "FP4 block-scale flip: the oracle's y is needed"
            gs = np.float32(scale_in)
            ts, bs = np.nonzero(diff)
            ys = y_ref(np.unique(ts))
            row_of = {t: i for i, t in enumerate(np.unique(ts))}
            for t, b in zip(ts, bs):
                yb = ys[row_of[t], 16 * b:16 * b + 16]
                u = np.float64((np.float32(np.abs(yb).max()) * gs) / np.float32(6))
                lo = min(sg[t, b], sr[t, b]) & 0x7F
                mid = (e4_table()[lo] + e4_table()[lo + 1]) / 2
                assert abs(u - mid) <= SCALE_REL * mid, "FP4 block scale flip off a midpoint"
                codes, v = _requant_fp4(yb, int(sg[t, b]), gs)
                nr_cmp[t, 16 * b:16 * b + 16] = codes
                pre_cmp[t, 16 * b:16 * b + 16] = v
        _codes_ok(ng, nr_cmp, pre_cmp, "e2m1", rep)
        if rep.scale_mismatch == 0 and np.array_equal(gpu["q"], ref["q"]):
            return _budget(rep)  # identical codes and scales: rule 4 holds trivially
        # rule 4: per element within one e2m1 step * d / gs
        gs = np.float64(np.float32(scale_in))
        dg = np.repeat(e4_table()[sg] / gs, 16, axis=1)
        dr = np.repeat(e4_table()[sr] / gs, 16, axis=1)
        vg = e2_table()[ng] * dg
        vr = e2_table()[nr] * dr
        gap = np.array([0.5, 0.5, 0.5, 0.5, 1.0, 1.0, 2.0, 2.0])
        step = gap[nr & 7] * np.maximum(dg, dr)
        assert np.all(np.abs(vg - vr) <= step + 1e-30), "FP4 dequantized value off by > one step"
        rel = np.abs(vg - vr) / np.maximum(np.abs(vr).max(), 1e-30)
        rep.max_dequant_rel = float(rel.max()) if rel.size else 0.0
    else:
        qg, qr = gpu["q"], ref["q"]
        qr_cmp, pre_cmp = qr, pre
        if mode == O.FP8_STATIC:
            s_g = s_r = np.full((T, 1), np.float32(scale_in), np.float64)
            G = H
        elif mode == O.FP8_TOKEN:
            s_g = gpu["scales"].astype(np.float64)[:, None]
            s_r = ref["scales"].astype(np.float64)[:, None]
            G = H
        else:
            G = group_size
            sg, sr = gpu["scales"], ref["scales"]
            if flags & O.SCALE_COLMAJOR:
                sg, sr = sg.T, sr.T
            if flags & O.SCALE_E8M0_U8:
                s_g = np.ldexp(1.0, sg.astype(np.int64) - 127)
                s_r = np.ldexp(1.0, sr.astype(np.int64) - 127)
            else:
                s_g, s_r = sg.astype(np.float64), sr.astype(np.float64)
        if mode != O.FP8_STATIC:
            e8 = mode == O.FP8_GROUP and bool(flags & (O.SCALE_E8M0 | O.SCALE_E8M0_U8))
            if e8:
                diff = s_g != s_r
                rep.scale_flips = int(diff.sum())
                if rep.scale_flips:
                    assert raw_group_scales is not None, "E8M0 scale flip: unrounded scale needed"
                    assert y_ref is not None, "E8M0 scale flip: the oracle's y is needed"
                    raw = np.asarray(raw_group_scales, np.float64)
                    if flags & O.SCALE_COLMAJOR:
                        raw = raw.T
                    ratio = np.maximum(s_g[diff], s_r[diff]) / np.minimum(s_g[diff], s_r[diff])
                    assert np.all(ratio == 2.0), "E8M0 scale differs by more than a factor 2"
                    p2 = np.ldexp(1.0, np.round(np.log2(raw[diff])).astype(np.int64))
                    assert np.all(np.abs(raw[diff] - p2) <= SCALE_REL * p2), \
                        "E8M0 flip off a power of two"
                    qr_cmp, pre_cmp = qr.copy(), pre.copy()
                    ts, gsel = np.nonzero(diff)
                    ys = y_ref(np.unique(ts))
                    row_of = {t: i for i, t in enumerate(np.unique(ts))}
                    for t, g in zip(ts, gsel):
                        codes, v = _requant_fp8(ys[row_of[t], G * g:G * g + G], s_g[t, g])
                        qr_cmp[t, G * g:G * g + G] = codes
                        pre_cmp[t, G * g:G * g + G] = v
            else:
                rel = np.abs(s_g - s_r) / np.maximum(np.abs(s_r), 1e-38)
                diff = rel > 0
                assert np.all(rel <= SCALE_REL), f"scale off by {rel.max():.3g} relative"
            rep.scale_mismatch = int(diff.sum())
        _codes_ok(qg, qr_cmp, pre_cmp, "e4m3", rep)
        if np.array_equal(qg, qr) and np.array_equal(s_g, s_r):
            return _budget(rep)  # identical codes and scales: rule 4 holds trivially
        # rule 4: relative L2 error of each dequantized row
        dqg = (e4_table()[qg].reshape(T, H // G, G) * s_g[:, :, None]).reshape(T, H)
        dqr = (e4_table()[qr].reshape(T, H // G, G) * s_r[:, :, None]).reshape(T, H)
        err = np.sqrt(((dqg - dqr) ** 2).sum(axis=1))
        ref_norm = np.sqrt((dqr ** 2).sum(axis=1))
        assert np.all((err <= DEQ_REL * ref_norm) | ((ref_norm == 0) & (err == 0))), \
            "dequantized row off by > 1e-2 relative"
        rel = err / np.maximum(ref_norm, 1e-38)
        rep.max_dequant_rel = float(rel.max()) if rel.size else 0.0

    return _budget(rep)


def _budget(rep: Report) -> Report:
    assert rep.code_mismatch + rep.scale_flips <= MAX_MISMATCH_FRAC * rep.elements, \
        f"{rep.code_mismatch} code mismatches and {rep.scale_flips} scale flips exceed 0.01% " \
        f"of {rep.elements}"
    return rep
