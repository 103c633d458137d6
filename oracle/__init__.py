"""CPU oracle for the W4A8 mixture-of-experts layer and the block-FP8 dense linear.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The library under
``w4a8_moe_amd/`` never imports it and shares no code with it; the two meet only
through the seeded inputs of the ``synth`` module.

The oracle is plain, slow and obviously correct: NumPy (and SciPy's ``erf``), fp64
for all floating point except at the quantization points, where the method fixes
fp32 (scales, the quotients that are rounded to a code) or a code (int4, e4m3, bf16).
Each function names the passage of the source pages it follows:

* page A = "ROCm: enable trillion-parameter MoE models with INT4-FP8 single node"
  (sglang pull request 4152): the Grok-1 W4A8KV8 ``config.json`` and its
  ``quantization_config`` (``int4_experts``: bits 4, sym, group column;
  ``activation_scheme`` static; ``pack_method`` reorder), the routing constants
  ``num_local_experts`` 8 / ``num_experts_per_tok`` 2, the router gate kept out of
  quantization (``ignored_layers``), and the heading "INT4 MoE weights, FP8 compute".
* page B = "[AMD][Quantization] Add int4fp8_moe online quantization on ROCm"
  (sglang pull request 7392): experts quantized online to int4, int4 weights upcast
  to float8 for fp8 math; the highlight "Core Quantization Utilities" (tensor-wise
  FP8 quantization, column-wise INT4 quantization, packing INT4 into INT32).
* page C = "qwen4_exp: serve the block-FP8 dense projections natively (+25% decode)"
  (FreeToken pull request 392): block-FP8 (FP8_PB_WO) weight-only projections with
  per-128x128-block scales ``weight_scale_inv``, shapes [16384,2560] with scales
  [128,20] and [13312,2560] with scales [104,20].
* the per-tensor FP8 dense linear (``fp8_linear``) follows page A's ``quant_method``
  "fp8" with static activations (everything but the router gates and ``lm_head``) and
  page B's tensor-wise FP8 quantization.
* the FP8 KV cache store (``kv_cache_store``) follows page A's ``kv_cache_scheme``
  static, ``kv_cache_group`` (k_proj, v_proj) and ``min_kv_scale`` 1.0.

Where the pages leave a step open, the reading taken is stated at the function.
Parity pins for every function live in ``tests/test_oracle_*.py``.
"""
from .fp8 import E4M3_MAX, e4m3_decode, e4m3_encode, e4m3_table
from .bf16 import bf16_to_f32, bf16_to_f64, f64_to_bf16_bits
from .int4 import w4_quantize, w4_pack_codes, w4_unpack_codes, w4_pack, w4_dequant
from .route import route_top2, route_sort
from .moe import (ACT_SILU, ACT_GELU_ERF, ACT_GELU_TANH, activation, act_lipschitz,
                  quantize_static, static_scale, moe_forward, moe_reference_unquantized,
                  expert_gate_up, expert_down,
                  moe_error_bound)
from .block_fp8 import fp8_block_quantize, fp8_block_linear, fp8_block_linear_bruteforce
from .fp8_linear import fp8_tensor_quantize, fp8_quantize_activations, fp8_linear, fp8_linear_bruteforce
from .kv_cache import MIN_KV_SCALE, kv_scale, kv_cache_store

__all__ = [
    "E4M3_MAX", "e4m3_decode", "e4m3_encode", "e4m3_table",
    "bf16_to_f32", "bf16_to_f64", "f64_to_bf16_bits",
    "w4_quantize", "w4_pack_codes", "w4_unpack_codes", "w4_pack", "w4_dequant",
    "route_top2", "route_sort",
    "ACT_SILU", "ACT_GELU_ERF", "ACT_GELU_TANH", "activation", "act_lipschitz",
    "quantize_static", "static_scale", "moe_forward", "moe_reference_unquantized",
    "moe_error_bound", "expert_gate_up", "expert_down",
    "fp8_block_quantize", "fp8_block_linear", "fp8_block_linear_bruteforce",
    "fp8_tensor_quantize", "fp8_quantize_activations", "fp8_linear", "fp8_linear_bruteforce",
    "MIN_KV_SCALE", "kv_scale", "kv_cache_store",
]
