"""Helpers for the GPU tests: run librmsq through its C ABI with guard bands around every
output, and hand back numpy arrays in the oracle's layout.  Test infrastructure only."""
import functools

import numpy as np
import torch

import oracle as O
from rmsnorm_quantization_amd import binding as B
from rmsnorm_quantization_amd import synth

PAD = 256        # guard band on each side of every output (keeps 16-byte alignment)
GUARD = 0xA5     # guard byte
FILL = 0xCD      # initial content of output data (an unwritten element shows up as a mismatch)


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU test run without a visible GPU")
    B.lib()  # fail loudly if librmsq.so is missing


class Guarded:
    def __init__(self, nbytes, dev="cuda"):
        self.n = int(nbytes)
        self.buf = torch.full((self.n + 2 * PAD,), GUARD, dtype=torch.uint8, device=dev)
        self.buf[PAD:PAD + self.n].fill_(FILL)
        self.data = self.buf[PAD:PAD + self.n]

    def check(self, what):
        lo = self.buf[:PAD]
        hi = self.buf[PAD + self.n:]
        assert bool((lo == GUARD).all()) and bool((hi == GUARD).all()), f"{what}: guard band overwritten"


def to_dev(t):
    return None if t is None else t.contiguous().to("cuda")


def scale_bytes(mode, T, H, G, flags, ld):
    shp, dt = O.scale_shape(mode, T, H, G, flags, ld)
    if shp is None:
        return 0, None, None
    return int(np.prod(shp)) * np.dtype(dt).itemsize, shp, dt


def run(mode, x, r, w, eps, scale_in=None, group_size=0, flags=0, scale_ld=0, launch=None,
        inplace=False, stream=None, rows=None):
    """Run one launch on device tensors x, r, w (r may be None).  Returns the outputs as numpy
    arrays (restricted to `rows` when given) plus the raw device tensors."""
    T, H = x.shape
    qb = T * H // 2 if mode == O.FP4_BLOCK16 else T * H
    gq = Guarded(qb)
    sb, sshape, sdt = scale_bytes(mode, T, H, group_size, flags, scale_ld)
    gs = Guarded(sb) if sshape is not None else None
    if r is not None:
        if inplace:
            rout_t = r
            grs = None
        else:
            grs = Guarded(T * H * 2)
            rout_t = grs.data.view(torch.bfloat16)
    else:
        rout_t, grs = None, None
    sc = None
    if scale_in is not None:
        sc = torch.tensor([float(np.float32(scale_in))], dtype=torch.float32, device="cuda")
    sview = None
    if gs is not None:
        sview = gs.data if sdt == np.uint8 else gs.data.view(torch.float32)
    B.rmsq_fused(x, r, w, eps, mode, sc, gq.data, sview, rout_t, group_size=group_size,
                 flags=flags, scale_ld=scale_ld, launch=launch, stream=stream)
    torch.cuda.synchronize()
    gq.check("out_q")
    if gs is not None:
        gs.check("out_scales")
    if grs is not None:
        grs.check("residual_out")

    qcols = H // 2 if mode == O.FP4_BLOCK16 else H
    q = gq.data.view(T, qcols)
    out = {}
    sel = None if rows is None else torch.as_tensor(np.asarray(rows), device="cuda")
    out["q"] = (q if sel is None else q[sel]).cpu().numpy()
    if gs is not None:
        s = sview.view(*sshape)
        if sel is not None:
            if mode == O.FP8_GROUP and flags & O.SCALE_COLMAJOR:
                s = s[:, sel]
            elif s.dim() == 1:
                s = s[sel]
            else:
                s = s[sel]
        out["scales"] = s.cpu().numpy()
        out["scales_full"] = sview
    else:
        out["scales"] = None
    if rout_t is not None:
        ro = rout_t.view(T, H)
        out["residual_out"] = synth.bits(ro if sel is None else ro[sel])
    else:
        out["residual_out"] = None
    return out


@functools.lru_cache(maxsize=8)
def workload_inputs(workload, T, H):
    """Seeded inputs of one workload shape, on the GPU and as bf16 bit arrays (cached)."""
    x, r, w = synth.make_inputs(workload, T, H)
    return (to_dev(x), to_dev(r), to_dev(w), synth.bits(x), None if r is None else synth.bits(r),
            synth.bits(w))


def sample_rows(T, n=48, seed=0):
    """A spread of rows including the first, last and a few in the middle."""
    if T <= n:
        return np.arange(T)
    rng = np.random.default_rng(seed + T)
    pick = set(rng.choice(T, n, replace=False).tolist()) | {0, 1, T // 2, T - 2, T - 1}
    return np.array(sorted(pick))


def host_threads():
    """Threads for the oracle on the host: the CPUs this process may use, at most 16 (one GPU's
    share of a GPU host)."""
    import os

    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _spans(T, nthr):
    step = max(1, -(-T // (4 * nthr)))
    return [(lo, min(lo + step, T)) for lo in range(0, T, step)]


def _join(parts, key, axis=0):
    vals = [p[key] for p in parts]
    if vals[0] is None:
        return None
    return np.concatenate(vals, axis=axis)


def oracle_threaded(mode, xb, rb, wb, eps, scale_in=0.0, group_size=0, flags=0, want_pre=True):
    """The oracle over every row of a batch, rows split over host_threads() threads (the oracle
    is C called through ctypes, which releases the GIL).  Rows are independent, so the result is
    the whole-batch call's; column-major scales come back [H/G, T]."""
    from concurrent.futures import ThreadPoolExecutor

    T = xb.shape[0]
    spans = _spans(T, host_threads())

    def run_span(sp):
        lo, hi = sp
        return O.fused(xb[lo:hi], None if rb is None else rb[lo:hi], wb, eps, mode,
                       scale_in=scale_in, group_size=group_size, flags=flags, want_pre=want_pre)

    with ThreadPoolExecutor(max_workers=host_threads()) as ex:
        parts = list(ex.map(run_span, spans))
    col = mode == O.FP8_GROUP and bool(flags & O.SCALE_COLMAJOR)
    return {"q": _join(parts, "q"), "scales": _join(parts, "scales", axis=1 if col else 0),
            "residual_out": _join(parts, "residual_out"), "pre": _join(parts, "pre")}


def oracle_act_threaded(mode, xb, scale_in=0.0, group_size=0, flags=0, want_pre=True):
    """SiLU+Mul -> quant by the oracle over every row, split over host threads."""
    from concurrent.futures import ThreadPoolExecutor

    T = xb.shape[0]

    def run_span(sp):
        lo, hi = sp
        return O.silu_mul_quant(xb[lo:hi], mode, scale_in=scale_in, group_size=group_size,
                                flags=flags, want_pre=want_pre)

    with ThreadPoolExecutor(max_workers=host_threads()) as ex:
        parts = list(ex.map(run_span, _spans(T, host_threads())))
    col = mode == O.FP8_GROUP and bool(flags & O.SCALE_COLMAJOR)
    return {"q": _join(parts, "q"), "scales": _join(parts, "scales", axis=1 if col else 0),
            "residual_out": None, "pre": _join(parts, "pre")}


def rms_y_threaded(xb, rb, wb, eps, f16=False):
    """The oracle's normalized rows y over every row, split over host threads."""
    from concurrent.futures import ThreadPoolExecutor

    T = xb.shape[0]

    def run_span(sp):
        lo, hi = sp
        return O.rms_y(xb[lo:hi], None if rb is None else rb[lo:hi], wb, eps, f16=f16)

    with ThreadPoolExecutor(max_workers=host_threads()) as ex:
        return np.concatenate(list(ex.map(run_span, _spans(T, host_threads()))), axis=0)


def oracle_on_rows(mode, xb, rb, wb, eps, rows, scale_in=0.0, group_size=0, flags=0):
    """Oracle outputs for the given rows (col-major scales come back [H/G, len(rows)])."""
    xs = xb if rows is None else xb[rows]
    rs = None if rb is None else (rb if rows is None else rb[rows])
    return O.fused(xs, rs, wb, eps, mode, scale_in=scale_in, group_size=group_size,
                   flags=flags, want_pre=True)


def y_ref_norm(xb, rb, wb, eps, rows=None, f16=False):
    """The y_ref callback of tests.parity.compare for a norm launch: the oracle's normalized f32
    rows for row indices into the compared arrays (into `rows` when only those were compared)."""
    def f(idx):
        sel = np.asarray(idx) if rows is None else np.asarray(rows)[np.asarray(idx)]
        return O.rms_y(xb[sel], None if rb is None else rb[sel], wb, eps, f16=f16)
    return f


def y_ref_act(xb, rows=None, f16=False):
    """The y_ref callback of tests.parity.compare for SiLU+Mul: the oracle's activation rows."""
    def f(idx):
        sel = np.asarray(idx) if rows is None else np.asarray(rows)[np.asarray(idx)]
        return O.silu_mul(xb[sel], f16=f16)
    return f


def run_act(mode, x, scale_in=None, group_size=0, flags=0, scale_ld=0, launch=None, rows=None):
    """SiLU+Mul -> quant on device x [T, 2I], outputs guarded like run()."""
    T, I = x.shape[0], x.shape[1] // 2
    qb = T * I // 2 if mode == O.FP4_BLOCK16 else T * I
    gq = Guarded(qb)
    sb, sshape, sdt = scale_bytes(mode, T, I, group_size, flags, scale_ld)
    gs = Guarded(sb) if sshape is not None else None
    sc = None
    if scale_in is not None:
        sc = torch.tensor([float(np.float32(scale_in))], dtype=torch.float32, device="cuda")
    sview = None
    if gs is not None:
        sview = gs.data if sdt == np.uint8 else gs.data.view(torch.float32)
    B.rmsq_silu_mul_quant(x, mode, sc, gq.data, sview, group_size=group_size, flags=flags,
                          scale_ld=scale_ld, launch=launch)
    torch.cuda.synchronize()
    gq.check("out_q")
    if gs is not None:
        gs.check("out_scales")
    qcols = I // 2 if mode == O.FP4_BLOCK16 else I
    q = gq.data.view(T, qcols)
    sel = None if rows is None else torch.as_tensor(np.asarray(rows), device="cuda")
    out = {"q": (q if sel is None else q[sel]).cpu().numpy(), "residual_out": None}
    if gs is not None:
        s = sview.view(*sshape)
        if sel is not None:
            s = s[:, sel] if (mode == O.FP8_GROUP and flags & O.SCALE_COLMAJOR) else s[sel]
        out["scales"] = s.cpu().numpy()
    else:
        out["scales"] = None
    return out
