"""MI355X-native per-row symmetric weight quantization (int6 / int8 / fp16 passthrough,
percentile clip, STE fake quantization, AWQ column scaling, SQWA averaging).

The compute path is libpgq.so (HIP kernels for gfx950 behind the C ABI in include/pgq.h).
`int6_weight_export_amd.pgq` is the ctypes binding; `int6_weight_export_amd.ops` adds
torch-allocated convenience wrappers.  Importing either loads the library and raises if
it has not been built.
"""
__all__ = ["pgq", "ops", "build"]
