"""Fused (residual add ->) RMSNorm -> FP8/FP4 quantization for AMD MI355X (gfx950).

The compute path is the HIP library librmsq.so behind the C ABI in include/rmsq.h;
`rmsnorm_quantization_amd.binding` marshals torch tensors (device memory and streams) into that
ABI.  Submodules are imported on demand, so the input generators (`synth`) work without a
built library.
"""
