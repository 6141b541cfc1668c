"""Float64 CPU oracle for the Gated Delta Rule-2 token mixer.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the benchmark's
CPU-baseline leg, never by the library. It shares no code with the HIP path.
"""
from .gdn2_oracle import (gdn2_backward, gdn2_decode_steps, gdn2_decode_tokens, gdn2_forward,
                          gdn2_step, gdn2_step_backward)

from .gdn2_block import epilogue as block_epilogue
from .gdn2_block import prologue as block_prologue

__all__ = ["gdn2_step", "gdn2_forward", "gdn2_decode_steps", "gdn2_decode_tokens",
           "gdn2_step_backward", "gdn2_backward", "block_prologue", "block_epilogue"]
