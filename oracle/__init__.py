"""CPU oracle for the MFA decode path (test infrastructure).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. The library itself never calls it, and it never calls the
library: the two share no code.
"""

from .mfa_oracle import (  # noqa: F401
    decode_bf16,
    e4m3fn_table,
    decode_e4m3fn,
    to_f64,
    rms_norm,
    q_path,
    kv_project,
    attend_one,
    decode_attn,
    out_proj,
    decode_layer,
    SOFTMAX_SCALE,
)
