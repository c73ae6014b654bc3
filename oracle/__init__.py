"""Plain float64 CPU oracle for the H2O decode path.

TEST INFRASTRUCTURE: imported only by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library or its binding."""
from .h2o_ref import (  # noqa: F401
    StepResult,
    causal_attention,
    prefill_column_sums,
    prefill_keep,
    prefill_output,
    prefill_scores,
    POLICIES,
    prefill,
    decode_step,
    run_trace,
    members_from_slots,
    e4m3_value,
    e4m3_encode,
    quantize_row_e4m3,
    dequantize_row_e4m3,
)
