"""Thin ctypes binding of librmsq (include/rmsq.h), argument marshalling only.

torch supplies device memory and the stream; every step of the computation runs in the HIP
kernels of librmsq.so.  The library is loaded from this package directory; if it is missing
the binding raises -- there is no fallback path.

Function names match the C ABI (rmsq_fused, rmsq_fused_with_launch, rmsq_fused_timed,
rmsq_silu_mul_quant, rmsq_silu_mul_quant_ex, rmsq_silu_mul_quant_validate,
rmsq_silu_mul_query_launch, rmsq_fused_fp4_dynamic, rmsq_fused_fp4_dynamic_ex,
rmsq_fused_fp4_dynamic_validate, rmsq_rms_norm_pad, rmsq_rms_norm_pad_ex, rmsq_rms_norm_pad_validate,
rmsq_rms_norm_pad_query_launch,
rmsq_qk_norm_rope, rmsq_qk_norm_rope_ex, rmsq_qk_norm_rope_validate,
rmsq_qk_norm_rope_query_launch, rmsq_validate,
rmsq_query_launch, rmsq_block_to_rowblock, rmsq_convert, rmsq_status_string,
rmsq_abi_version).  A few allocating helpers named after the fused ops of the vLLM fusion
pages (rms_norm_static_fp8_quant, fused_add_rms_norm_static_fp8_quant,
rms_norm_dynamic_per_token_quant, rms_norm_per_block_quant, fused_add_rms_norm_fp4_quant)
sit on top for callers who want tensors back.
"""
import ctypes as C
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librmsq.so")

# ---- constants mirrored from include/rmsq.h ----
RMSQ_OK, RMSQ_EINVAL, RMSQ_EALIGN, RMSQ_EALIAS, RMSQ_EUNSUPPORTED, RMSQ_ELAUNCH, RMSQ_EDEVICE = (
    0, -1, -2, -3, -4, -5, -6)
RMSQ_FP8_STATIC, RMSQ_FP8_TOKEN, RMSQ_FP8_GROUP, RMSQ_FP4_BLOCK16 = 0, 1, 2, 3
RMSQ_SCALE_COLMAJOR, RMSQ_SCALE_E8M0, RMSQ_SCALE_E8M0_U8 = 1, 2, 4
RMSQ_INPUT_F16 = 1 << 8
RMSQ_CVT_E4M3, RMSQ_CVT_E2M1, RMSQ_CVT_BF16, RMSQ_CVT_INV_SQRT = 0, 1, 2, 3
RMSQ_CVT_E4M3_IN_RANGE = 4
RMSQ_LAUNCH_XCD_RANGES = 1
RMSQ_LAUNCH_ROW_TILES = 2
RMSQ_MAX_HIDDEN = 65536
RMSQ_ABI_VERSION = 5  # the argument lists below are those of this version


class RmsqError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {rmsq_status_string(status)} (status {status})")
        self.status = status


class rmsq_launch(C.Structure):
    _fields_ = [("threads_per_row", C.c_int32), ("chunks_per_thread", C.c_int32),
                ("rows_per_block", C.c_int32), ("options", C.c_int32)]

    def as_tuple(self):
        return (self.threads_per_row, self.chunks_per_thread, self.rows_per_block, self.options)


_lib = None


def lib():
    """The loaded librmsq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; "
                f"g.build()'` (or python rmsnorm_quantization_amd/build.py)")
        L = C.CDLL(LIB_PATH)
        p, i64, f32, i32, u32 = C.c_void_p, C.c_int64, C.c_float, C.c_int, C.c_uint
        fused_args = [p, p, p, f32, i32, p, p, p, p, i64, i64, i32, u32, i64]
        L.rmsq_fused.argtypes = fused_args + [p]
        L.rmsq_fused.restype = i32
        L.rmsq_fused_with_launch.argtypes = fused_args + [C.POINTER(rmsq_launch), p]
        L.rmsq_fused_with_launch.restype = i32
        L.rmsq_fused_timed.argtypes = fused_args + [C.POINTER(rmsq_launch), p, p, p]
        L.rmsq_fused_timed.restype = i32
        L.rmsq_validate.argtypes = fused_args
        L.rmsq_validate.restype = i32
        dyn_args = [p, p, p, f32, p, p, p, p, i64, i64, u32]
        L.rmsq_fused_fp4_dynamic.argtypes = dyn_args + [p]
        L.rmsq_fused_fp4_dynamic.restype = i32
        L.rmsq_fused_fp4_dynamic_ex.argtypes = dyn_args + [C.POINTER(rmsq_launch), p, p, p]
        L.rmsq_fused_fp4_dynamic_ex.restype = i32
        L.rmsq_fused_fp4_dynamic_validate.argtypes = dyn_args
        L.rmsq_fused_fp4_dynamic_validate.restype = i32
        pad_args = [p, p, p, f32, p, p, i64, i64, i64, u32]
        L.rmsq_rms_norm_pad.argtypes = pad_args + [p]
        L.rmsq_rms_norm_pad.restype = i32
        L.rmsq_rms_norm_pad_ex.argtypes = pad_args + [C.POINTER(rmsq_launch), p, p, p]
        L.rmsq_rms_norm_pad_ex.restype = i32
        L.rmsq_rms_norm_pad_validate.argtypes = pad_args
        L.rmsq_rms_norm_pad_validate.restype = i32
        act_args = [p, i32, p, p, p, i64, i64, i32, u32, i64]
        L.rmsq_silu_mul_quant.argtypes = act_args + [p]
        L.rmsq_silu_mul_quant.restype = i32
        L.rmsq_silu_mul_quant_ex.argtypes = act_args + [C.POINTER(rmsq_launch), p, p, p]
        L.rmsq_silu_mul_quant_ex.restype = i32
        L.rmsq_silu_mul_quant_validate.argtypes = act_args
        L.rmsq_silu_mul_quant_validate.restype = i32
        rope_args = [p, p, p, p, p, f32, i64, i32, i32, i32, i64]
        L.rmsq_qk_norm_rope.argtypes = rope_args + [i32, u32, p]
        L.rmsq_qk_norm_rope.restype = i32
        L.rmsq_qk_norm_rope_ex.argtypes = rope_args + [i32, u32, i32, i32, p, p, p]
        L.rmsq_qk_norm_rope_ex.restype = i32
        L.rmsq_qk_norm_rope_validate.argtypes = rope_args + [u32]
        L.rmsq_qk_norm_rope_validate.restype = i32
        L.rmsq_qk_norm_rope_query_launch.argtypes = [i64, i32, i32, i32, C.POINTER(i32),
                                                     C.POINTER(i32), C.POINTER(i64)]
        L.rmsq_qk_norm_rope_query_launch.restype = i32
        L.rmsq_query_launch.argtypes = [i32, i64, i64, i32, u32, C.POINTER(rmsq_launch),
                                        C.POINTER(i64)]
        L.rmsq_query_launch.restype = i32
        L.rmsq_rms_norm_pad_query_launch.argtypes = [i64, i64, i64, u32,
                                                     C.POINTER(rmsq_launch), C.POINTER(i64)]
        L.rmsq_rms_norm_pad_query_launch.restype = i32
        L.rmsq_silu_mul_query_launch.argtypes = [i32, i64, i64, i32, C.POINTER(rmsq_launch),
                                                 C.POINTER(i64)]
        L.rmsq_silu_mul_query_launch.restype = i32
        L.rmsq_block_to_rowblock.argtypes = [i64, i64]
        L.rmsq_block_to_rowblock.restype = i64
        L.rmsq_convert.argtypes = [i32, p, p, i64, p]
        L.rmsq_convert.restype = i32
        L.rmsq_status_string.argtypes = [i32]
        L.rmsq_status_string.restype = C.c_char_p
        L.rmsq_abi_version.argtypes = []
        L.rmsq_abi_version.restype = i32
        if L.rmsq_abi_version() != RMSQ_ABI_VERSION:
            raise RuntimeError(
                f"{LIB_PATH} has ABI version {L.rmsq_abi_version()}, this binding needs "
                f"{RMSQ_ABI_VERSION}: rebuild it")
        _lib = L
    return _lib


def _ptr(t) -> Optional[int]:
    """Device pointer of a tensor (or None); raw integers pass through."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("rmsq: tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("rmsq: tensors must be contiguous")
    return t.data_ptr()


# ---- argument checks on tensors (raw integer pointers are the caller's responsibility) --------
# Everything below runs before any pointer is taken: a tensor that cannot hold what the call
# reads or writes raises ValueError instead of becoming an out-of-bounds access on the GPU.
def _need(t, what: str, nbytes: int, kind: str):
    """t (a tensor; None and integers are not checked) must be of `kind` and hold nbytes:
    "act" 16-bit activations (any 2-byte type: the call's RMSQ_INPUT_F16 flag, not the tensor's
    dtype, says whether the bits are bf16 or binary16), "f32", "i64", "byte" (any 1-byte
    type)."""
    if not isinstance(t, torch.Tensor):
        return
    if kind == "act" and t.element_size() != 2:
        raise ValueError(f"rmsq: {what} must have 16-bit elements (bfloat16 or float16), "
                         f"not {t.dtype}")
    elif kind == "f32" and t.dtype != torch.float32:
        raise ValueError(f"rmsq: {what} must be float32, not {t.dtype}")
    elif kind == "i64" and t.dtype != torch.int64:
        raise ValueError(f"rmsq: {what} must be int64, not {t.dtype}")
    elif kind == "byte" and t.element_size() != 1:
        raise ValueError(f"rmsq: {what} must have 1-byte elements, not {t.dtype}")
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"rmsq: {what} holds {have} bytes, the call needs {nbytes}")


def _rows_cols(t, what: str, rows, cols, cols_of=lambda c: c):
    """(rows, cols) of a call whose sizes default to a 2-D tensor's shape."""
    if rows is not None and cols is not None:
        return int(rows), int(cols)
    if not isinstance(t, torch.Tensor) or t.dim() != 2:
        raise ValueError(f"rmsq: {what} must be a 2-D tensor, or pass the sizes explicitly")
    return int(t.shape[0] if rows is None else rows), int(cols_of(t.shape[1]) if cols is None
                                                         else cols)


def _scale_nbytes(mode, T, n, group_size, flags, ld) -> int:
    """Bytes of the scales output of a quantization of T rows of n values."""
    if mode == RMSQ_FP8_TOKEN:
        return 4 * T
    if mode == RMSQ_FP8_GROUP and group_size in (64, 128) and T > 0:
        ng = n // group_size
        el = 1 if flags & RMSQ_SCALE_E8M0_U8 else 4
        if flags & RMSQ_SCALE_COLMAJOR:
            return ((ng - 1) * (ld or T) + T) * el
        return T * ng * el
    if mode == RMSQ_FP4_BLOCK16:
        return T * (n // 16)
    return 0


def _check_quant_outputs(mode, scale_in, out_q, out_scales, T, n, group_size, flags, ld):
    _need(scale_in, "scale_in", 4, "f32")
    _need(out_q, "out_q", T * n // 2 if mode == RMSQ_FP4_BLOCK16 else T * n, "byte")
    sb = _scale_nbytes(mode, T, n, group_size, flags, ld)
    f32 = mode == RMSQ_FP8_TOKEN or (mode == RMSQ_FP8_GROUP and not flags & RMSQ_SCALE_E8M0_U8)
    _need(out_scales, "out_scales", sb, "f32" if f32 else "byte")


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str):
    if status != RMSQ_OK:
        raise RmsqError(status, where)


# ---------------------------------------------------------------- C ABI, same names
def rmsq_status_string(status: int) -> str:
    return lib().rmsq_status_string(int(status)).decode()


def rmsq_abi_version() -> int:
    return lib().rmsq_abi_version()


def rmsq_fused(x, residual, weight, eps, mode, scale_in, out_q, out_scales, residual_out,
               tokens=None, hidden=None, group_size=0, flags=0, scale_ld=0, stream=None,
               launch: Optional[rmsq_launch] = None, check=True) -> int:
    """Enqueue one fused launch.  Tensors are passed by device pointer; sizes default to x's
    shape ([T, H], 2-D).  Raises ValueError when a tensor cannot hold what the call reads or
    writes, and RmsqError on a non-zero status unless check=False."""
    T, H = _check_fused(x, residual, weight, mode, scale_in, out_q, out_scales, residual_out,
                        tokens, hidden, group_size, flags, scale_ld)
    args = (_ptr(x), _ptr(residual), _ptr(weight), float(eps), int(mode), _ptr(scale_in),
            _ptr(out_q), _ptr(out_scales), _ptr(residual_out), int(T), int(H), int(group_size),
            int(flags), int(scale_ld))
    if launch is None:
        st = lib().rmsq_fused(*args, _stream(stream))
    else:
        st = lib().rmsq_fused_with_launch(*args, C.byref(launch), _stream(stream))
    if check:
        _check(st, "rmsq_fused")
    return st


def _check_fused(x, residual, weight, mode, scale_in, out_q, out_scales, residual_out, tokens,
                 hidden, group_size, flags, scale_ld):
    T, H = _rows_cols(x, "x", tokens, hidden)
    act = 2 * T * H
    for t, what in ((x, "x"), (residual, "residual"), (residual_out, "residual_out")):
        _need(t, what, act, "act")
    _need(weight, "weight", 2 * H, "act")
    _check_quant_outputs(mode, scale_in, out_q, out_scales, T, H, group_size, flags, scale_ld)
    return T, H


def rmsq_fused_with_launch(x, residual, weight, eps, mode, scale_in, out_q, out_scales,
                           residual_out, tokens=None, hidden=None, group_size=0, flags=0,
                           scale_ld=0, launch=None, stream=None, check=True) -> int:
    return rmsq_fused(x, residual, weight, eps, mode, scale_in, out_q, out_scales, residual_out,
                      tokens, hidden, group_size, flags, scale_ld, stream, launch, check)


def rmsq_fused_timed(x, residual, weight, eps, mode, scale_in, out_q, out_scales, residual_out,
                     tokens=None, hidden=None, group_size=0, flags=0, scale_ld=0, launch=None,
                     start_event=None, stop_event=None, stream=None, check=True) -> int:
    """One launch whose start/stop events (raw hipEvent_t handles, e.g. a recorded
    torch.cuda.Event's .cuda_event) are stamped by the dispatch itself."""
    T, H = _check_fused(x, residual, weight, mode, scale_in, out_q, out_scales, residual_out,
                        tokens, hidden, group_size, flags, scale_ld)
    st = lib().rmsq_fused_timed(_ptr(x), _ptr(residual), _ptr(weight), float(eps), int(mode),
                                _ptr(scale_in), _ptr(out_q), _ptr(out_scales),
                                _ptr(residual_out), int(T), int(H), int(group_size), int(flags),
                                int(scale_ld), None if launch is None else C.byref(launch),
                                start_event, stop_event, _stream(stream))
    if check:
        _check(st, "rmsq_fused_timed")
    return st


def rmsq_fused_fp4_dynamic(x, residual, weight, eps, out_q, out_scales, residual_out,
                           global_scale, tokens=None, hidden=None, flags=0, stream=None,
                           launch=None, start_event=None, stop_event=None, check=True) -> int:
    """(Residual add ->) RMSNorm -> FP4 block-16 with the global scale taken from the batch
    (written to global_scale, one f32).  With a launch shape or events it goes through
    rmsq_fused_fp4_dynamic_ex."""
    T, H = _check_fused(x, residual, weight, RMSQ_FP4_BLOCK16, global_scale, out_q, out_scales,
                        residual_out, tokens, hidden, 16, flags, 0)
    args = (_ptr(x), _ptr(residual), _ptr(weight), float(eps), _ptr(out_q), _ptr(out_scales),
            _ptr(residual_out), _ptr(global_scale), int(T), int(H), int(flags))
    if launch is None and start_event is None and stop_event is None:
        st = lib().rmsq_fused_fp4_dynamic(*args, _stream(stream))
    else:
        st = lib().rmsq_fused_fp4_dynamic_ex(*args, None if launch is None else C.byref(launch),
                                             start_event, stop_event, _stream(stream))
    if check:
        _check(st, "rmsq_fused_fp4_dynamic")
    return st


def rmsq_fused_fp4_dynamic_validate(x, residual, weight, eps, out_q, out_scales, residual_out,
                                    global_scale, tokens, hidden, flags=0) -> int:
    """Host-only argument check; pointers are plain integers (or None)."""
    return lib().rmsq_fused_fp4_dynamic_validate(x, residual, weight, float(eps), out_q,
                                                 out_scales, residual_out, global_scale,
                                                 int(tokens), int(hidden), int(flags))


def rmsq_rms_norm_pad(x, residual, weight, eps, out, residual_out, tokens=None, hidden=None,
                      out_ld=None, stream=None, launch=None, start_event=None, stop_event=None,
                      check=True, flags=0) -> int:
    """(Residual add ->) RMSNorm -> out [T, out_ld] (bf16, or binary16 with RMSQ_INPUT_F16)
    with zero padding columns."""
    T, H = _rows_cols(x, "x", tokens, hidden)
    if out_ld is None:
        if not isinstance(out, torch.Tensor) or out.dim() != 2:
            raise ValueError("rmsq: out must be a 2-D tensor [T, out_ld], or pass out_ld")
        ld = int(out.shape[1])
    else:
        ld = int(out_ld)
    for t, what in ((x, "x"), (residual, "residual"), (residual_out, "residual_out")):
        _need(t, what, 2 * T * H, "act")
    _need(weight, "weight", 2 * H, "act")
    _need(out, "out", 2 * T * ld, "act")
    args = (_ptr(x), _ptr(residual), _ptr(weight), float(eps), _ptr(out), _ptr(residual_out),
            int(T), int(H), int(ld), int(flags))
    if launch is None and start_event is None and stop_event is None:
        st = lib().rmsq_rms_norm_pad(*args, _stream(stream))
    else:
        st = lib().rmsq_rms_norm_pad_ex(*args, None if launch is None else C.byref(launch),
                                        start_event, stop_event, _stream(stream))
    if check:
        _check(st, "rmsq_rms_norm_pad")
    return st


def rmsq_rms_norm_pad_validate(x, residual, weight, eps, out, residual_out, tokens, hidden,
                               out_ld, flags=0) -> int:
    """Host-only argument check; pointers are plain integers (or None)."""
    return lib().rmsq_rms_norm_pad_validate(x, residual, weight, float(eps), out, residual_out,
                                            int(tokens), int(hidden), int(out_ld), int(flags))


def rmsq_silu_mul_quant(x, mode, scale_in, out_q, out_scales, tokens=None, inter=None,
                        group_size=0, flags=0, scale_ld=0, stream=None, launch=None,
                        start_event=None, stop_event=None, check=True) -> int:
    """SiLU+Mul -> quant of x [T, 2I] (gate first).  With a launch shape or events it goes
    through rmsq_silu_mul_quant_ex."""
    T, I = _rows_cols(x, "x", tokens, inter, cols_of=lambda c: c // 2)
    _need(x, "x", 4 * T * I, "act")
    _check_quant_outputs(mode, scale_in, out_q, out_scales, T, I, group_size, flags, scale_ld)
    args = (_ptr(x), int(mode), _ptr(scale_in), _ptr(out_q), _ptr(out_scales), int(T), int(I),
            int(group_size), int(flags), int(scale_ld))
    if launch is None and start_event is None and stop_event is None:
        st = lib().rmsq_silu_mul_quant(*args, _stream(stream))
    else:
        st = lib().rmsq_silu_mul_quant_ex(*args, None if launch is None else C.byref(launch),
                                          start_event, stop_event, _stream(stream))
    if check:
        _check(st, "rmsq_silu_mul_quant")
    return st


def rmsq_silu_mul_quant_validate(x, mode, scale_in, out_q, out_scales, tokens, inter,
                                 group_size=0, flags=0, scale_ld=0) -> int:
    """Host-only argument check; pointers are plain integers (or None)."""
    return lib().rmsq_silu_mul_quant_validate(x, int(mode), scale_in, out_q, out_scales,
                                              int(tokens), int(inter), int(group_size),
                                              int(flags), int(scale_ld))


def rmsq_qk_norm_rope(qkv, q_weight, k_weight, cos_sin_cache, positions, eps, num_q_heads,
                      num_kv_heads, head_dim, is_neox=True, tokens=None, max_position=None,
                      stream=None, heads_per_block=0, heads_per_lane=0, start_event=None,
                      stop_event=None, check=True, flags=0) -> int:
    """In-place per-head RMSNorm + rotary embedding of the q and k heads of qkv
    [T, (Hq + 2 Hkv) * D] (bf16, or binary16 with flags=RMSQ_INPUT_F16); cos_sin_cache
    [max_position, D] f32, positions [T] int64.  With a launch shape (heads per workgroup and
    per lane group) or events it goes through rmsq_qk_norm_rope_ex."""
    D = int(head_dim)
    width = (int(num_q_heads) + 2 * int(num_kv_heads)) * D
    T, _ = _rows_cols(qkv, "qkv", tokens, width)
    if max_position is None:
        if not isinstance(cos_sin_cache, torch.Tensor) or cos_sin_cache.dim() != 2 \
                or cos_sin_cache.shape[1] != D:
            raise ValueError(f"rmsq: cos_sin_cache must be a 2-D tensor [max_position, {D}], "
                             f"or pass max_position")
        mp = int(cos_sin_cache.shape[0])
    else:
        mp = int(max_position)
    if isinstance(qkv, torch.Tensor) and tokens is None and qkv.shape[1] != width:
        raise ValueError(f"rmsq: qkv rows hold {qkv.shape[1]} values, the heads need {width}")
    _need(qkv, "qkv", 2 * T * width, "act")
    _need(q_weight, "q_weight", 2 * D, "act")
    _need(k_weight, "k_weight", 2 * D, "act")
    _need(cos_sin_cache, "cos_sin_cache", 4 * mp * D, "f32")
    _need(positions, "positions", 8 * T, "i64")
    args = (_ptr(qkv), _ptr(q_weight), _ptr(k_weight), _ptr(cos_sin_cache), _ptr(positions),
            float(eps), int(T), int(num_q_heads), int(num_kv_heads), int(head_dim), int(mp))
    if heads_per_block == 0 and heads_per_lane == 0 and start_event is None and \
            stop_event is None:
        st = lib().rmsq_qk_norm_rope(*args, int(bool(is_neox)), int(flags), _stream(stream))
    else:
        st = lib().rmsq_qk_norm_rope_ex(*args, int(bool(is_neox)), int(flags),
                                        int(heads_per_block), int(heads_per_lane), start_event,
                                        stop_event, _stream(stream))
    if check:
        _check(st, "rmsq_qk_norm_rope")
    return st


def rmsq_qk_norm_rope_validate(qkv, q_weight, k_weight, cos_sin_cache, positions, eps, tokens,
                               num_q_heads, num_kv_heads, head_dim, max_position,
                               flags=0) -> int:
    """Host-only argument check; pointers are plain integers (or None)."""
    return lib().rmsq_qk_norm_rope_validate(qkv, q_weight, k_weight, cos_sin_cache, positions,
                                            float(eps), int(tokens), int(num_q_heads),
                                            int(num_kv_heads), int(head_dim), int(max_position),
                                            int(flags))


def rmsq_qk_norm_rope_query_launch(tokens, num_q_heads, num_kv_heads, head_dim):
    """(heads per workgroup, heads per lane group, grid size) of the default launch."""
    hpb = C.c_int(0)
    hpl = C.c_int(0)
    grid = C.c_int64(0)
    _check(lib().rmsq_qk_norm_rope_query_launch(int(tokens), int(num_q_heads), int(num_kv_heads),
                                                int(head_dim), C.byref(hpb), C.byref(hpl),
                                                C.byref(grid)),
           "rmsq_qk_norm_rope_query_launch")
    return hpb.value, hpl.value, grid.value


def rmsq_validate(x, residual, weight, eps, mode, scale_in, out_q, out_scales, residual_out,
                  tokens, hidden, group_size=0, flags=0, scale_ld=0) -> int:
    """Host-only argument check; pointers are plain integers (or None) and never dereferenced."""
    return lib().rmsq_validate(x, residual, weight, float(eps), int(mode), scale_in, out_q,
                               out_scales, residual_out, int(tokens), int(hidden),
                               int(group_size), int(flags), int(scale_ld))


def rmsq_query_launch(mode, tokens, hidden, group_size=0, flags=0):
    """The default launch shape of rmsq_fused for these arguments, and its grid size."""
    l = rmsq_launch()
    grid = C.c_int64(0)
    _check(lib().rmsq_query_launch(int(mode), int(tokens), int(hidden), int(group_size),
                                   int(flags), C.byref(l), C.byref(grid)),
           "rmsq_query_launch")
    return l, grid.value


def rmsq_rms_norm_pad_query_launch(tokens, hidden, out_ld, flags=0):
    l = rmsq_launch()
    grid = C.c_int64(0)
    _check(lib().rmsq_rms_norm_pad_query_launch(int(tokens), int(hidden), int(out_ld), int(flags),
                                                C.byref(l), C.byref(grid)),
           "rmsq_rms_norm_pad_query_launch")
    return l, grid.value


def rmsq_silu_mul_query_launch(mode, tokens, inter, group_size=0):
    l = rmsq_launch()
    grid = C.c_int64(0)
    _check(lib().rmsq_silu_mul_query_launch(int(mode), int(tokens), int(inter), int(group_size),
                                            C.byref(l), C.byref(grid)),
           "rmsq_silu_mul_query_launch")
    return l, grid.value


def rmsq_block_to_rowblock(block: int, grid: int) -> int:
    return lib().rmsq_block_to_rowblock(int(block), int(grid))


def rmsq_convert(fmt, inp, out, n=None, stream=None, check=True) -> int:
    n = inp.numel() if n is None else n
    st = lib().rmsq_convert(int(fmt), _ptr(inp), _ptr(out), int(n), _stream(stream))
    if check:
        _check(st, "rmsq_convert")
    return st


# ---------------------------------------------------------------- allocating helpers
def _act_flag(x, weight, residual=None) -> int:
    """RMSQ_INPUT_F16 for float16 activations, 0 for bfloat16; x, the weight and the residual
    must share the dtype (the pages' type check), anything else is refused."""
    if x.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError(f"rmsq: activations must be bfloat16 or float16, not {x.dtype}")
    for t in (weight, residual):
        if t is not None and t.dtype != x.dtype:
            raise TypeError(f"rmsq: x is {x.dtype} but another input is {t.dtype}")
    return RMSQ_INPUT_F16 if x.dtype == torch.float16 else 0


def _scalar(v, dev) -> torch.Tensor:
    if isinstance(v, torch.Tensor):
        return v.to(device=dev, dtype=torch.float32).reshape(1).contiguous()
    return torch.tensor([float(v)], dtype=torch.float32, device=dev)


def rms_norm_static_fp8_quant(x, weight, scale, eps, residual=None, inplace=True):
    """(q [T,H] float8_e4m3fn, residual_out or None).  With a residual, the new residual is
    written into `residual` itself when inplace=True (as the fused-add op does)."""
    q = torch.empty(x.shape, dtype=torch.float8_e4m3fn, device=x.device)
    rout = None if residual is None else (residual if inplace else torch.empty_like(residual))
    rmsq_fused(x, residual, weight, eps, RMSQ_FP8_STATIC, _scalar(scale, x.device),
               q.view(torch.uint8), None, rout, flags=_act_flag(x, weight, residual))
    return q, rout


def fused_add_rms_norm_static_fp8_quant(x, residual, weight, scale, eps):
    """Fused add + RMSNorm + FP8 static quant; `residual` is updated in place.  Returns q."""
    return rms_norm_static_fp8_quant(x, weight, scale, eps, residual=residual, inplace=True)[0]


def rms_norm_dynamic_per_token_quant(x, weight, eps, residual=None, inplace=True):
    """(q float8_e4m3fn [T,H], scales f32 [T], residual_out or None)."""
    T = x.shape[0]
    q = torch.empty(x.shape, dtype=torch.float8_e4m3fn, device=x.device)
    s = torch.empty((T,), dtype=torch.float32, device=x.device)
    rout = None if residual is None else (residual if inplace else torch.empty_like(residual))
    rmsq_fused(x, residual, weight, eps, RMSQ_FP8_TOKEN, None, q.view(torch.uint8), s, rout,
               flags=_act_flag(x, weight, residual))
    return q, s, rout


def rms_norm_per_block_quant(x, weight, eps, group_size=128, residual=None, inplace=True,
                             col_major=False, e8m0=False, e8m0_bytes=False, scale_ld=0):
    """(q float8_e4m3fn [T,H], scales, residual_out or None).  Scales are [T,H/G] f32, or
    [H/G, ld] with col_major, or uint8 E8M0 bytes with e8m0_bytes."""
    T, H = x.shape
    ng = H // group_size
    flags = (RMSQ_SCALE_COLMAJOR if col_major else 0) | (RMSQ_SCALE_E8M0 if e8m0 else 0) | (
        RMSQ_SCALE_E8M0_U8 if e8m0_bytes else 0) | _act_flag(x, weight, residual)
    ld = scale_ld or T
    shape = (ng, ld) if col_major else (T, ng)
    s = torch.empty(shape, dtype=torch.uint8 if e8m0_bytes else torch.float32, device=x.device)
    q = torch.empty(x.shape, dtype=torch.float8_e4m3fn, device=x.device)
    rout = None if residual is None else (residual if inplace else torch.empty_like(residual))
    rmsq_fused(x, residual, weight, eps, RMSQ_FP8_GROUP, None, q.view(torch.uint8), s, rout,
               group_size=group_size, flags=flags, scale_ld=scale_ld if col_major else 0)
    return q, s, rout


def fused_add_rms_norm_fp4_quant(x, residual, weight, global_scale, eps, inplace=True):
    """(packed e2m1 uint8 [T,H/2], e4m3 block scales uint8 [T,H/16], residual_out).
    global_scale is the encode multiplier gs (dequant value = e2m1 * decode(sf) / gs)."""
    T, H = x.shape
    q = torch.empty((T, H // 2), dtype=torch.uint8, device=x.device)
    sf = torch.empty((T, H // 16), dtype=torch.uint8, device=x.device)
    rout = residual if inplace else torch.empty_like(residual)
    rmsq_fused(x, residual, weight, eps, RMSQ_FP4_BLOCK16, _scalar(global_scale, x.device), q,
               sf, rout, group_size=16, flags=_act_flag(x, weight, residual))
    return q, sf, rout


def fused_add_rms_norm_fp4_quant_dynamic(x, residual, weight, eps, inplace=True):
    """(packed e2m1 uint8 [T,H/2], e4m3 block scales uint8 [T,H/16], global scale f32 [1],
    residual_out or None): FP4 with the global encode scale gs = 448 * 6 / max|y| of the batch
    (dequant value = e2m1 * decode(sf) / gs).  residual may be None (plain RMSNorm)."""
    T, H = x.shape
    q = torch.empty((T, H // 2), dtype=torch.uint8, device=x.device)
    sf = torch.empty((T, H // 16), dtype=torch.uint8, device=x.device)
    gs = torch.empty((1,), dtype=torch.float32, device=x.device)
    rout = None if residual is None else (residual if inplace else torch.empty_like(residual))
    rmsq_fused_fp4_dynamic(x, residual, weight, eps, q, sf, rout, gs,
                           flags=_act_flag(x, weight, residual))
    return q, sf, gs, rout


def silu_and_mul_quant(x, mode, scale=None, group_size=0, col_major=False, e8m0=False,
                       e8m0_bytes=False, scale_ld=0):
    """(codes, scales or None) for SiLU+Mul -> quant of x [T, 2I]: FP8 codes as
    float8_e4m3fn [T, I], FP4 as packed uint8 [T, I/2]; scale is the static per-tensor scale
    (FP8 static) or the global encode scale (FP4)."""
    T, I = x.shape[0], x.shape[-1] // 2
    flags = (RMSQ_SCALE_COLMAJOR if col_major else 0) | (RMSQ_SCALE_E8M0 if e8m0 else 0) | (
        RMSQ_SCALE_E8M0_U8 if e8m0_bytes else 0) | _act_flag(x, x)
    if mode == RMSQ_FP4_BLOCK16:
        q = torch.empty((T, I // 2), dtype=torch.uint8, device=x.device)
        s = torch.empty((T, I // 16), dtype=torch.uint8, device=x.device)
        group_size = 16
    else:
        q = torch.empty((T, I), dtype=torch.float8_e4m3fn, device=x.device)
        if mode == RMSQ_FP8_STATIC:
            s = None
        elif mode == RMSQ_FP8_TOKEN:
            s = torch.empty((T,), dtype=torch.float32, device=x.device)
        else:
            ng, ld = I // group_size, scale_ld or T
            s = torch.empty((ng, ld) if col_major else (T, ng),
                            dtype=torch.uint8 if e8m0_bytes else torch.float32, device=x.device)
    sc = _scalar(scale, x.device) if mode in (RMSQ_FP8_STATIC, RMSQ_FP4_BLOCK16) else None
    rmsq_silu_mul_quant(x, mode, sc, q.view(torch.uint8) if q.dtype != torch.uint8 else q, s,
                        group_size=group_size, flags=flags,
                        scale_ld=scale_ld if col_major else 0)
    return q, s


def fused_add_rms_norm_pad(x, residual, weight, eps, multiple=256, inplace=True):
    """(out [T, H padded up to `multiple`] in x's dtype with zero padding, residual_out):
    residual add + RMSNorm with the hidden dimension padded for a downstream GEMM."""
    T, H = x.shape
    flags = _act_flag(x, weight, residual)
    ld = -(-H // multiple) * multiple
    out = torch.empty((T, ld), dtype=x.dtype, device=x.device)
    rout = None if residual is None else (residual if inplace else torch.empty_like(residual))
    rmsq_rms_norm_pad(x, residual, weight, eps, out, rout, flags=flags)
    return out, rout


def qk_norm_rope(qkv, positions, q_weight, k_weight, cos_sin_cache, eps, num_q_heads,
                 num_kv_heads, is_neox=True):
    """The fused QK-norm + RoPE op on qkv [T, (Hq + 2 Hkv) * D] (bf16 or float16, the weights
    of the same dtype), in place; returns qkv."""
    D = q_weight.shape[0]
    flags = _act_flag(qkv, q_weight, k_weight)
    rmsq_qk_norm_rope(qkv, q_weight, k_weight, cos_sin_cache, positions, eps, num_q_heads,
                      num_kv_heads, D, is_neox, flags=flags)
    return qkv
