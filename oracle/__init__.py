"""CPU oracle for per-row symmetric weight quantization (test infrastructure only).

Only the tests, the smoke check and the bench's CPU-baseline leg may import this
package.  The arithmetic lives in orc.c (plain single-threaded C, IEEE binary32 basic
operations, its own fp16/bf16 converters); this module loads it with ctypes and adds
the per-tensor export policy and the snapshot averaging loop in plain Python.
Nothing here is shared with, or imported by, the GPU library.
"""
from .lib import (  # noqa: F401
    ORC_NONFINITE, ORC_SCALE_OVF, ORC_F16_OVF, ORC_BAD_AWQ,
    load, build, f32_to_f16, f16_to_f32, f32_to_bf16, bf16_to_f32, percentile_rank,
    quantize_rows, quantize_tensor, awq_multipliers, fakequant_rows, f16_passthrough, sqwa_update, ema_update, swa_update,
    pack6_row_bytes, pack6, unpack6, dequant, qgemm_bf16,
)
from .policy import (  # noqa: F401
    Policy, DEFAULT_INT8_PATTERNS, KIND_F16, KIND_INT6, KIND_INT8,
    tensor_kind, as_rows, export, qdq_tensor, sqwa_run, ema_run, swa_run,
)
