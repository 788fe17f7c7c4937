"""Fused block-wise 8-bit optimizer steps (AdamW; Lion and SGD with momentum on
the same machinery) with a stochastically rounded bf16 parameter write, for
AMD Instinct MI355X (gfx950).

The step runs in libopt8.so (hand-written HIP kernels behind a C ABI, declared
in include/opt8.h); `opt8` is its ctypes binding (argument marshalling only).
torch supplies device memory and streams only.
"""
from .opt8 import (  # noqa: F401
    OPT8_BLOCK, OPT8_FP32_STATE_THRESHOLD, OPT8_STATE_8BIT, OPT8_STATE_BF16_SR, OPT8_STATE_FP32,
    OPT8_ROUND_STOCHASTIC, OPT8_ROUND_NEAREST, OPT8_STATE_ROUND_NEAREST, OPT8_STATE_ROUND_STOCHASTIC,
    Opt8Error, opt8_tensor, opt8_hparams, opt8_init_codebooks, opt8_default_mode, opt8_adamw_step,
    opt8_adamw_step_noalloc,
    opt8_lion_step, opt8_momentum_step, opt8_last_error, make_hparams, make_tensor, tensor_array,
)
