"""CPU oracle for scaled dot-product attention (test infrastructure only).

This package is the checker, not the product. Only the test suite, the
``smoke()`` entry point and the ``cpu_baseline`` leg of the benchmark may
import it. The GPU library never imports, links or calls anything in here, and
nothing in here imports the GPU library: the two share no code.

Source of the method: the codelab "Accelerate attention on GPU with cuDNN and
TransformerEngine" (JAX on GPU, lab 5), cited below as [Attention codelab §n]
where n is the codelab step:

* §1 "How attention works": the formula softmax(Q K^T / sqrt(d_k)) V and its
  four steps (score, scale + softmax whose weights sum to 1, attend, output
  shaped like Q).
* §3 "Create Q, K, V test arrays": the (B, T, N, H) / (B, S, K, H) layout.
* §4 "Implement attention from scratch": the unfused reference computation.
* §7 "Add a causal mask": each position attends only to itself and earlier
  positions (a lower-triangular mask); with fewer queries than keys it is
  applied top-left (query i at position i) or, for the key-value-cache form
  of the inference use §9 motivates, bottom-right (query i at position
  Skv - Sq + i).
* §9 "Compare MHA, GQA and MQA": K/V heads are broadcast over query heads when
  there are fewer of them; GQA with 2 KV heads each serving 4 query heads.
* §10 "TransformerEngine and FP8": E4M3 (4 exponent, 3 mantissa bits) for the
  forward pass with per-tensor amax scaling; E5M2 for the backward pass.
* §1 also motivates the scale by the softmax's gradients: ``backward.py``
  holds the row log-sum-exp and the chain-rule gradients dQ, dK, dV.

Every function is pinned by tests in ``tests/test_oracle.py`` and
``tests/test_codecs.py`` (``tests/test_oracle_backward.py`` for the
backward) to facts that do not come from the oracle itself
(closed forms, invariants, brute force, library routines, hand-derived golden
values). No function here is "parity unpinned".
"""

from .attention import attention_weights, sdpa, sdpa_rows, sdpa_one_row, brute_sdpa, kv_head_of, query_shift
from .backward import sdpa_lse, sdpa_backward
from .fp8_scaling import AMAX_HISTORY_LEN, DelayedScalingState, quantize_with_scale
from .codecs import (
    bf16_bits_to_f64,
    f16_bits_to_f64,
    e4m3_bits_to_f64,
    f64_to_bf16_bits,
    f64_to_e4m3_bits,
    e4m3_amax_scale,
    e5m2_bits_to_f64,
    f64_to_e5m2_bits,
    e5m2_amax_scale,
)

__all__ = [
    "attention_weights",
    "sdpa",
    "sdpa_rows",
    "sdpa_one_row",
    "brute_sdpa",
    "kv_head_of",
    "query_shift",
    "sdpa_lse",
    "sdpa_backward",
    "AMAX_HISTORY_LEN",
    "DelayedScalingState",
    "quantize_with_scale",
    "bf16_bits_to_f64",
    "f16_bits_to_f64",
    "e4m3_bits_to_f64",
    "f64_to_bf16_bits",
    "f64_to_e4m3_bits",
    "e4m3_amax_scale",
    "e5m2_bits_to_f64",
    "f64_to_e5m2_bits",
    "e5m2_amax_scale",
]
