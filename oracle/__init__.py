"""CPU oracle for exact attention: test infrastructure, not part of the product.

Only the test suite, the smoke entry and the benchmark's CPU-baseline leg may
import this package.  The GPU library never calls it, and nothing here uses
the GPU library.

The oracle is the plain definition of attention written out in float64 numpy
(FlashAttention, NeurIPS 2022, as explained on the vibeengines.com page
"FlashAttention, explained", sections "The math, worked with real numbers" and
"Solve it yourself"): scores, a safe softmax per row, and the weighted sum of
values.  The backward pass is the analytic gradient of that definition.

Module map:
  attention  - forward (O and per-row log-sum-exp) and backward (dQ, dK, dV).
  fp8        - E4M3 decoding and attention of dequantized FP8 inputs.
  online     - the pages' block-by-block update rule (running max, running sum,
               rescaled output accumulator) in float64.  Tests use it only to
               check the pages' own assertions; it is not the parity target.
"""

from .attention import (  # noqa: F401
    attention_forward,
    attention_forward_head,
    attention_backward,
    attention_backward_head,
    attention_decode_head,
    safe_softmax,
    default_scale,
)
from .fp8 import (  # noqa: F401
    e4m3_to_float64,
    dequantize,
    attention_forward_fp8_head,
    attention_weights_fp8_head,
)
from .online import blockwise_softmax, merge_states, tiled_attention  # noqa: F401
