"""Fused (residual add ->) RMSNorm -> FP8/FP4 quantization for AMD MI355X (gfx950).

The compute path is the HIP library librmsq.so behind the C ABI in include/rmsq.h; the Python
binding only marshals torch tensors (device memory and streams) into that ABI.  The binding is
imported lazily so that the input generators can be used without a built library.
"""

__all__ = ["binding", "synth"]


def __getattr__(name):
    if name == "binding":
        from . import binding as _b

        return _b
    raise AttributeError(name)
