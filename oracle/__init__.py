"""CPU oracle for fused attention: forward (decode and causal prefill) and backward.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or run
anything in this package: only the test suite, the package smoke check and the
benchmark's CPU-baseline leg use it. It shares no code with the HIP kernels,
their headers or the Python binding.

Pages cited (by title and section):
  [FA4-decode]   "Optimization diaries: S/P ping-pong for FlashAttention-4 decode"
  [FA4-bwd]      "Optimization diaries: Improving FlashAttention-4 backward pass
                  kernel design for head dimension 64"
  [GQA-SM100]    "Building a Faster GQA Decode Kernel for Blackwell SM100"
  [FA4-edges]    "Flash Attention 4 — warp-role choreography and the edges"

Every function is parity-pinned by tests in ``tests/test_oracle_pins.py``.
"""
from .attention import (  # noqa: F401
    bf16_bits_to_f64,
    f16_bits_to_f64,
    to_f64,
    attention,
    attention_rows,
    attention_varlen,
    probabilities,
    split_partials,
    combine_partials,
    decode_row_counts,
)
from .backward import (  # noqa: F401
    attention_backward,
    attention_backward_varlen,
    backward_error_scales,
    backward_error_scales_varlen,
    backward_f64,
    backward_kv_head,
)
from .brute import brute_attention  # noqa: F401
