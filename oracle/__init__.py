"""CPU oracle for the fused block-wise 8-bit AdamW step with a stochastically
rounded bf16 parameter write.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this package: only the test suite, the smoke check of the build entry point
and the CPU-baseline leg of the benchmark do.  It shares no code, table or
constant generator with the HIP library; the two are independent
implementations of the same definitions, compared element by element.

Plain, slow, single-threaded numpy.  Floating point follows the precision the
pages fix for this path: state is dequantised to 32-bit, updated and
requantised in fp32 ("8-bit Optimizers via Block-wise Quantization", method
bullets on in-register dequantise/update/requantise; "[Feat]: Stochastic
rounding of AdamW momentums", the request to do the Adam arithmetic in
float32).  Every numpy ufunc on float32 arrays rounds once to nearest-even, so
no operation is contracted into a fused multiply-add.

Modules
  codebook  dynamic-tree signed/unsigned 256-entry codebooks and midpoints
  philox    Philox4x32-10 counter-based generator (Salmon et al., SC'11)
  rounding  bf16 decode, stochastic rounding and round-to-nearest-even
  adamw     host scalars, block quantiser and the per-tensor AdamW step
  onestate  Lion and SGD with momentum on the same state machinery
  state_sr  stochastic rounding of the 8-bit state between neighbouring entries

Parity status of each function is stated in its module header.
"""

from . import codebook, philox, rounding, adamw, onestate, state_sr  # noqa: F401
from .adamw import (  # noqa: F401
    Hparams,
    Scalars,
    host_scalars,
    dequantize_blockwise,
    quantize_blockwise,
    adamw_param_update,
    step_tensor,
    MODE_8BIT,
    MODE_BF16_SR,
    MODE_FP32,
    ROUND_STOCHASTIC,
    ROUND_NEAREST,
    BLOCK,
    FP32_STATE_THRESHOLD,
    default_mode,
)
from .onestate import ALGO_LION, ALGO_MOMENTUM, step_tensor_1state  # noqa: F401
from .state_sr import STATE_ROUND_NEAREST, STATE_ROUND_STOCHASTIC  # noqa: F401
