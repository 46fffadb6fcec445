"""CPU oracle for the quantized-GEMV hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only the test suite, the smoke check and the bench's
CPU-baseline leg use it.  It shares no code with the HIP library and imports
nothing from it; it takes plain numpy arrays and returns plain numpy arrays.

It is deliberately slow and literal: each function writes out the definition
from the pages it cites, with numpy as the only helper (a max, a sum, a
matrix product).  Float references are fp64; integer results are exact;
quantization steps use IEEE fp32 operations in the order the definition
states (numpy float32 arithmetic is correctly rounded).

Sources (cited by short tag throughout)
  [SEP]  "1-bit quantization is not magic" -- blog on separated quantization,
         m.lqnn.cn/news/241359 (sections 1-6).
  [VG]   "A Visual Guide to LLM Quantization" (Chinese translation),
         puppylpg.github.io (sections on linear quantization, activations,
         BitNet, BitNet b1.58; figures 15-60).
  [OVR]  LLM quantization overview, 2048ai.net/68d1f9e38867235e13877cac.html
         (sections 1-6).
  [DQ]   news report on ISTA-DASLab's quantization split by inference
         phase (prefill / decode), ai4snews.wisdomeyes.cn/zh/news/786ff1c6c728dd1806bd2871.
  [T158] "1.58 bits vs FP8: what ternary weights actually buy",
         feinterview.poetries.top.

Parity status: every function here is pinned by the ``not gpu`` tests in
``tests/test_oracle_*.py`` against worked examples, closed forms, exact
rational arithmetic or brute force.  The method-error diagnostic
``relative_method_error`` is reported only and is "parity unpinned".
"""
from .numerics import (bf16_bits_to_f32, f32_to_bf16_bits, round_rational_to_f32,
                       exact_abs_sum_units, mean_abs_f32, mean_abs_rows_f32)
from .quant import (absmax_scale, quantize_with_scale, quantize_absmax,
                    ternary_absmean, sign_residual_split, outlier_split_quantize,
                    gather_outlier_weights, dequantize, detect_outlier_channels,
                    asym_params, quantize_with_zero_point, quantize_asym, dequantize_asym,
                    sign_residual_split_zp)
from .packing import (pack, unpack, pack_loops, unpack_loops)
from .products import (int_dot_exact, int_gemm_exact, int_dot_bruteforce,
                       y_w8a8, y_w8a16, y_w8a16_batch, y_ternary, y_sign_residual, y_sign_residual_zp, y_prefill,
                       relative_method_error, normwise_error)

__all__ = [n for n in dir() if not n.startswith("_")]
