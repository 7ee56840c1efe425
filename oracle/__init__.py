"""CPU oracle for ART paged decode attention (test infrastructure only).

This package is the checker, not the product.  Only the test suite, the
package-level ``smoke()`` entry and the CPU-baseline leg of the benchmark may
import it.  It shares no code with the HIP path: it decodes the stored bytes
itself, works in float64 NumPy, and follows the method step by step.

Source of the method: "ART: Attention Run-time Termination for Efficient Large
Language Model Decoding" (the gist.science explainer page), Technical Summary
section 2 (Methodology) and its subsections 2.1-2.4.
"""

from .art_oracle import (  # noqa: F401
    decode_bf16,
    decode_e4m3fn,
    decode_f32,
    art_reference,
    art_head,
    head_stats_trajectory,
    prefix_output,
    full_attention,
    stop_rule,
    direction_magnitude,
)
from .bruteforce import prefix_attention_bruteforce  # noqa: F401
from .feasible import classify_tests, feasible_stop, compare_with_oracle  # noqa: F401
from .importance import block_key_summary, block_scores, importance_order  # noqa: F401
from .inputs_check import check_inputs  # noqa: F401
