"""CPU oracle for the LLM.int8() vector-wise mixed-precision linear.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The product path (the
HIP library and its Python binding) never imports it and shares no code with it.
"""

from .llm_int8 import (  # noqa: F401
    INT32_SAFE_K,
    outlier_columns,
    outlier_bitmap,
    bitmap_to_columns,
    row_absmax,
    quantize_rows,
    vectorwise_quant,
    quantize_weight,
    vectorwise_dequant,
    outlier_extract,
    int8_linear_matmul,
    outlier_matmul,
    mm_dequant,
    linear_forward,
    QuantResult,
    ForwardResult,
)
from .backward import (  # noqa: F401
    colwise_absmax,
    colwise_quant,
    grad_input,
    grad_weight,
    linear_backward,
    BackwardResult,
)
