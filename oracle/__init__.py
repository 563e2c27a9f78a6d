"""CPU oracle for scaled dot-product attention (float64, numpy).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the package smoke check and
by the benchmark's CPU-baseline leg, never by the product path. It shares no
code with the HIP library. Parity status of each function is stated in
``sdpa_oracle``'s docstrings and pinned by ``tests/test_oracle.py``.
"""
from .sdpa_oracle import (  # noqa: F401
    alibi_slopes,
    attention_backward,
    attention_forward,
    attention_probs,
    dropout_keep_threshold,
    dropout_mask,
    fp8_dequantize,
    fp8_e4m3_decode,
    fp8_e5m2_decode,
    philox4x32_10,
)
