"""ctypes front end of the C oracle (TEST INFRASTRUCTURE ONLY).

All tensors are numpy arrays on the host: bf16 values travel as their uint16 bit patterns,
codes as uint8, scales as float32 (or uint8 for E8M0 bytes).  Nothing here computes any part
of the method; it marshals arguments and allocates outputs.
"""
import ctypes as C

import numpy as np

from .build import ensure_built

FP8_STATIC, FP8_TOKEN, FP8_GROUP, FP4_BLOCK16 = 0, 1, 2, 3
SCALE_COLMAJOR, SCALE_E8M0, SCALE_E8M0_U8 = 1, 2, 4
INPUT_F16 = 1 << 8  # x, residual, weight and residual_out are IEEE binary16 patterns

_lib = None


def lib():
    global _lib
    if _lib is None:
        L = C.CDLL(ensure_built())
        p = C.c_void_p
        i64 = C.c_int64
        L.orc_bf16_to_f32.argtypes = [C.c_uint16]
        L.orc_bf16_to_f32.restype = C.c_float
        L.orc_f32_to_bf16.argtypes = [C.c_float]
        L.orc_f32_to_bf16.restype = C.c_uint16
        L.orc_e4m3_decode.argtypes = [C.c_uint8]
        L.orc_e4m3_decode.restype = C.c_float
        L.orc_e4m3_encode.argtypes = [C.c_float]
        L.orc_e4m3_encode.restype = C.c_uint8
        L.orc_e2m1_decode.argtypes = [C.c_uint8]
        L.orc_e2m1_decode.restype = C.c_float
        L.orc_e2m1_encode.argtypes = [C.c_float]
        L.orc_e2m1_encode.restype = C.c_uint8
        L.orc_e8m0_ceil_exp.argtypes = [C.c_float]
        L.orc_e8m0_ceil_exp.restype = C.c_int
        for name in ("orc_e4m3_encode_n", "orc_e2m1_encode_n", "orc_f32_to_bf16_n",
                     "orc_e8m0_ceil_exp_n"):
            getattr(L, name).argtypes = [p, p, i64]
            getattr(L, name).restype = None
        L.orc_f16_to_f32.argtypes = [C.c_uint16]
        L.orc_f16_to_f32.restype = C.c_float
        L.orc_f32_to_f16.argtypes = [C.c_float]
        L.orc_f32_to_f16.restype = C.c_uint16
        L.orc_f32_to_f16_n.argtypes = [p, p, i64]
        L.orc_f32_to_f16_n.restype = None
        L.orc_residual_add_dt.argtypes = [p, p, p, i64, C.c_int]
        L.orc_residual_add_dt.restype = None
        L.orc_inv_rms_dt.argtypes = [p, i64, C.c_float, C.c_int]
        L.orc_inv_rms_dt.restype = C.c_float
        L.orc_normalize_dt.argtypes = [p, p, C.c_float, p, i64, C.c_int]
        L.orc_normalize_dt.restype = None
        L.orc_residual_add.argtypes = [p, p, p, i64]
        L.orc_residual_add.restype = None
        L.orc_inv_rms.argtypes = [p, i64, C.c_float]
        L.orc_inv_rms.restype = C.c_float
        L.orc_normalize.argtypes = [p, p, C.c_float, p, i64]
        L.orc_normalize.restype = None
        L.orc_quantize_row.argtypes = [p, i64, C.c_int, C.c_float, C.c_int, C.c_uint, p, p, p]
        L.orc_quantize_row.restype = C.c_int
        L.orc_silu_mul.argtypes = [C.c_uint16, C.c_uint16]
        L.orc_silu_mul.restype = C.c_float
        L.orc_silu_mul_row_dt.argtypes = [p, i64, p, C.c_int]
        L.orc_silu_mul_row_dt.restype = None
        L.orc_silu_mul_row.argtypes = [p, i64, p]
        L.orc_silu_mul_row.restype = None
        L.orc_silu_mul_quant.argtypes = [p, C.c_int, C.c_float, p, p, i64, i64, C.c_int,
                                         C.c_uint, i64, p]
        L.orc_silu_mul_quant.restype = C.c_int
        L.orc_rms_norm_pad.argtypes = [p, p, p, C.c_float, p, p, i64, i64, i64, C.c_uint]
        L.orc_rms_norm_pad.restype = C.c_int
        L.orc_rope_cache.argtypes = [p, i64, i64, C.c_double]
        L.orc_rope_cache.restype = None
        L.orc_qk_norm_rope.argtypes = [p, p, p, p, p, C.c_float, i64, i64, i64, i64, i64, C.c_int,
                                       C.c_uint]
        L.orc_qk_norm_rope.restype = C.c_int
        L.orc_fused.argtypes = [p, p, p, C.c_float, C.c_int, C.c_float, p, p, p,
                                i64, i64, C.c_int, C.c_uint, i64, p]
        L.orc_fused.restype = C.c_int
        L.orc_fp4_global_scale.argtypes = [C.c_float]
        L.orc_fp4_global_scale.restype = C.c_float
        L.orc_fused_fp4_dynamic.argtypes = [p, p, p, C.c_float, p, p, p, p, i64, i64, C.c_uint, p]
        L.orc_fused_fp4_dynamic.restype = C.c_int
        L.rmsq_ref_fused.argtypes = [p, p, p, C.c_float, C.c_int, p, p, p, p, i64, i64,
                                     C.c_int, C.c_uint, i64]
        L.rmsq_ref_fused.restype = C.c_int
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- converters
def bf16_to_f32(bits):
    bits = _c(bits, np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(v):
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint16)
    lib().orc_f32_to_bf16_n(_ptr(v), _ptr(out), v.size)
    return out


def f16_to_f32(bits):
    """binary16 bit patterns -> f32 values, decoded by the oracle."""
    bits = _c(bits, np.uint16)
    flat = bits.reshape(-1)
    out = np.array([lib().orc_f16_to_f32(int(b)) for b in flat], np.float32)
    return out.reshape(bits.shape)


def f32_to_f16(v):
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint16)
    lib().orc_f32_to_f16_n(_ptr(v), _ptr(out), v.size)
    return out


def e4m3_encode(v):
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().orc_e4m3_encode_n(_ptr(v), _ptr(out), v.size)
    return out


def e2m1_encode(v):
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().orc_e2m1_encode_n(_ptr(v), _ptr(out), v.size)
    return out


def e8m0_ceil_exp(s):
    s = _c(s, np.float32)
    out = np.empty(s.shape, np.int32)
    lib().orc_e8m0_ceil_exp_n(_ptr(s), _ptr(out), s.size)
    return out


def e4m3_table():
    """float32[256]: the oracle's decode of every e4m3fn byte."""
    return np.array([lib().orc_e4m3_decode(c) for c in range(256)], np.float32)


def e2m1_table():
    """float32[16]: the oracle's decode of every e2m1 nibble."""
    return np.array([lib().orc_e2m1_decode(c) for c in range(16)], np.float32)


def e4m3_decode(codes):
    return e4m3_table()[_c(codes, np.uint8)]


def e2m1_decode(codes):
    return e2m1_table()[_c(codes, np.uint8) & 0xF]


def unpack_fp4(packed):
    """[..., H/2] bytes -> [..., H] nibbles (element 2k from the low nibble)."""
    packed = _c(packed, np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


# ---------------------------------------------------------------- row steps
def residual_add(x, r):
    x = _c(x, np.uint16)
    r = _c(r, np.uint16)
    h = np.empty_like(x)
    lib().orc_residual_add(_ptr(x), _ptr(r), _ptr(h), x.size)
    return h


def inv_rms(h, eps):
    h = _c(h, np.uint16)
    return np.float32(lib().orc_inv_rms(_ptr(h), h.size, eps))


def normalize(h, w, inv):
    h = _c(h, np.uint16)
    w = _c(w, np.uint16)
    y = np.empty(h.shape, np.float32)
    lib().orc_normalize(_ptr(h), _ptr(w), float(inv), _ptr(y), h.size)
    return y


# ---------------------------------------------------------------- whole operation
def scale_shape(mode, T, H, group_size=0, flags=0, scale_ld=0):
    if mode == FP8_STATIC:
        return None, None
    if mode == FP8_TOKEN:
        return (T,), np.float32
    if mode == FP8_GROUP:
        ng = H // group_size
        dt = np.uint8 if flags & SCALE_E8M0_U8 else np.float32
        if flags & SCALE_COLMAJOR:
            return (ng, scale_ld or T), dt
        return (T, ng), dt
    if mode == FP4_BLOCK16:
        return (T, H // 16), np.uint8
    raise ValueError(mode)


def fused(x, residual, weight, eps, mode, scale_in=0.0, group_size=0, flags=0, scale_ld=0,
          want_pre=False):
    """Run the oracle on [T,H] bf16-bit arrays.  Returns a dict with q, scales,
    residual_out and (optionally) pre, the f32 value each code was encoded from."""
    x = _c(x, np.uint16)
    T, H = x.shape
    r = None if residual is None else _c(residual, np.uint16)
    w = _c(weight, np.uint16)
    q = np.zeros((T, H // 2 if mode == FP4_BLOCK16 else H), np.uint8)
    shp, dt = scale_shape(mode, T, H, group_size, flags, scale_ld)
    scales = None if shp is None else np.zeros(shp, dt)
    rout = None if r is None else np.zeros_like(r)
    pre = np.zeros((T, H), np.float32) if want_pre else None
    rc = lib().orc_fused(_ptr(x), _ptr(r), _ptr(w), float(eps), int(mode), float(scale_in),
                         _ptr(q), _ptr(scales), _ptr(rout), T, H, int(group_size),
                         int(flags), int(scale_ld), _ptr(pre))
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (rc={rc})")
    return {"q": q, "scales": scales, "residual_out": rout, "pre": pre}


def fp4_global_scale(amax):
    """(448 * 6) / amax in f32, FLT_MAX where that is not finite."""
    return np.float32(lib().orc_fp4_global_scale(float(amax)))


def fused_fp4_dynamic(x, residual, weight, eps, flags=0, want_pre=False):
    """FP4 block-16 with the global scale taken from the batch: dict with q, scales,
    residual_out, global_scale (np.float32) and optionally pre."""
    x = _c(x, np.uint16)
    T, H = x.shape
    r = None if residual is None else _c(residual, np.uint16)
    w = _c(weight, np.uint16)
    q = np.zeros((T, H // 2), np.uint8)
    scales = np.zeros((T, H // 16), np.uint8)
    rout = None if r is None else np.zeros_like(r)
    gs = np.zeros(1, np.float32)
    pre = np.zeros((T, H), np.float32) if want_pre else None
    rc = lib().orc_fused_fp4_dynamic(_ptr(x), _ptr(r), _ptr(w), float(eps), _ptr(q),
                                     _ptr(scales), _ptr(rout), _ptr(gs), T, H, int(flags),
                                     _ptr(pre))
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (rc={rc})")
    return {"q": q, "scales": scales, "residual_out": rout, "global_scale": gs[0], "pre": pre}


def quantize_row(y, mode, scale_in=0.0, group_size=0, flags=0):
    """Quantize one normalized f32 row.  Returns (q, row_scales, pre)."""
    y = _c(y, np.float32)
    H = y.size
    q = np.zeros(H // 2 if mode == FP4_BLOCK16 else H, np.uint8)
    if mode == FP8_TOKEN:
        sc = np.zeros(1, np.float32)
    elif mode == FP8_GROUP:
        sc = np.zeros(H // group_size, np.uint8 if flags & SCALE_E8M0_U8 else np.float32)
    elif mode == FP4_BLOCK16:
        sc = np.zeros(H // 16, np.uint8)
    else:
        sc = np.zeros(1, np.float32)
    pre = np.zeros(H, np.float32)
    rc = lib().orc_quantize_row(_ptr(y), H, int(mode), float(scale_in), int(group_size),
                                int(flags), _ptr(q), _ptr(sc), _ptr(pre))
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (rc={rc})")
    return q, (None if mode == FP8_STATIC else sc), pre


def rms_y(x, residual, weight, eps, f16=False):
    """The normalized f32 rows y (before quantization), built from the oracle's steps; f16: the
    16-bit inputs are IEEE binary16 rather than bf16."""
    x = _c(x, np.uint16)
    w = _c(weight, np.uint16)
    T, H = x.shape
    dt = int(bool(f16))
    y = np.empty((T, H), np.float32)
    h = np.empty(H, np.uint16)
    for t in range(T):
        if residual is None:
            h[:] = x[t]
        else:
            r = _c(residual[t], np.uint16)
            xt = _c(x[t], np.uint16)
            lib().orc_residual_add_dt(_ptr(xt), _ptr(r), _ptr(h), H, dt)
        inv = lib().orc_inv_rms_dt(_ptr(h), H, float(eps), dt)
        yt = np.empty(H, np.float32)
        lib().orc_normalize_dt(_ptr(h), _ptr(w), float(inv), _ptr(yt), H, dt)
        y[t] = yt
    return y


# ---------------------------------------------------------------- SiLU+Mul -> quant
def silu_mul(x, f16=False):
    """[T, 2I] bf16 bits (IEEE binary16 with f16) -> [T, I] f32 activation silu(gate) * up."""
    x = _c(x, np.uint16)
    T, I2 = x.shape
    I = I2 // 2
    a = np.empty((T, I), np.float32)
    for t in range(T):
        lib().orc_silu_mul_row_dt(_ptr(x[t]), I, a[t].ctypes.data_as(C.c_void_p),
                                  int(bool(f16)))
    return a


def silu_mul_quant(x, mode, scale_in=0.0, group_size=0, flags=0, scale_ld=0, want_pre=False):
    """Run the oracle's SiLU+Mul -> quant on [T, 2I] bf16 bits."""
    x = _c(x, np.uint16)
    T, I2 = x.shape
    I = I2 // 2
    q = np.zeros((T, I // 2 if mode == FP4_BLOCK16 else I), np.uint8)
    shp, dt = scale_shape(mode, T, I, group_size, flags, scale_ld)
    scales = None if shp is None else np.zeros(shp, dt)
    pre = np.zeros((T, I), np.float32) if want_pre else None
    rc = lib().orc_silu_mul_quant(_ptr(x), int(mode), float(scale_in), _ptr(q), _ptr(scales), T,
                                  I, int(group_size), int(flags), int(scale_ld), _ptr(pre))
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (rc={rc})")
    return {"q": q, "scales": scales, "pre": pre}


# ---------------------------------------------------------------- RMSNorm -> padded bf16
def rms_norm_pad(x, residual, weight, eps, out_ld, flags=0):
    """[T, H] bf16 bits -> (out [T, out_ld] bf16 bits, residual_out or None); with
    flags=INPUT_F16 every 16-bit array is IEEE binary16."""
    x = _c(x, np.uint16)
    T, H = x.shape
    r = None if residual is None else _c(residual, np.uint16)
    w = _c(weight, np.uint16)
    out = np.full((T, out_ld), 0xFFFF, np.uint16)
    rout = None if r is None else np.zeros_like(r)
    rc = lib().orc_rms_norm_pad(_ptr(x), _ptr(r), _ptr(w), float(eps), _ptr(out), _ptr(rout), T,
                                H, int(out_ld), int(flags))
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (rc={rc})")
    return out, rout


# ---------------------------------------------------------------- QK-norm + RoPE
def rope_cache(max_pos, D, base=1_000_000.0):
    """[max_pos, D] f32: cos | sin of p * base^(-2i/D)."""
    cache = np.empty((max_pos, D), np.float32)
    lib().orc_rope_cache(_ptr(cache), int(max_pos), int(D), float(base))
    return cache


def qk_norm_rope(qkv, qw, kw, cache, pos, eps, Hq, Hkv, D, neox=True, flags=0):
    """Returns a new [T, (Hq+2Hkv)*D] bf16-bit array (the input is not modified); with
    flags=INPUT_F16, qkv, qw, kw and the result are IEEE binary16."""
    out = np.array(qkv, np.uint16, copy=True, order="C")
    T = out.shape[0]
    qw = _c(qw, np.uint16)
    kw = _c(kw, np.uint16)
    cache = _c(cache, np.float32)
    pos = _c(pos, np.int64)
    rc = lib().orc_qk_norm_rope(_ptr(out), _ptr(qw), _ptr(kw), _ptr(cache), _ptr(pos), float(eps),
                                T, int(Hq), int(Hkv), int(D), cache.shape[0], int(bool(neox)),
                                int(flags))
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (rc={rc})")
    return out
