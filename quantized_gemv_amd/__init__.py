"""quantized_gemv_amd -- MI355X (gfx950) quantized GEMV library.

Python side of the C ABI in include/qgemv.h: symmetric absmax / absmean
quantization to int8, ternary, sign + int8-residual, thresholded separated
and group-wise 4-bit formats, bit packing, quantized GEMV for decode (batch 1
and small batches), the W8A8 prefill GEMM with an activation outlier split,
and an MXFP4 prefill on the FP4 matrix cores.  All arithmetic runs in the HIP kernels of
libqgemv.so; this package only marshals arguments (see _binding.py).
"""
from ._binding import (QgError, QWeight, CWeight, EXPORTED, LIB_PATH, lib, status_str,
                       quantize_absmax, quantize_absmax_split, detect_outliers, gather_columns_bf16, quantize_ternary,
                       split_sign_residual, split_sign_residual_zp, quantize_asym, quantize_q4k, SepWeight, sep_resid_ld, quantize_mxfp4, gemm_mxfp4, prefill_mxfp4, split_sep_threshold, qgemv_sep, qgemv_sep_grouped, SepGroupLaunch, CSepMatrix, pack, unpack, base3_row_bytes, pack_base3, unpack_base3, pack_tiles16, tiled16, qgemv, qgemv_grouped, qgemv_batch, qgemv_batch_grouped, batch_workspace_bytes, GroupLaunch, qgemv_launch_raw,
                       ChainStep, CChainStage, chain_plan_image, QG_CHAIN_MAX_STAGES, QG_CHAIN_MIN_K, QG_CHAIN_MAX_K,
                       QG_CHAIN_ERROR_OFFSET, QG_CHAIN_TIMEOUT_TICKS,
                       qgemm_w8a8_outlier, qgemm_w8a8, out_ld, QG_MAX_GROUP, QG_OUT_LD_ALIGN, QG_MAX_OUT_LD,
                       QG_F32, QG_BF16, QG_PER_TENSOR, QG_PER_ROW, QG_WFMT_INT8, QG_WFMT_TERNARY2,
                       QG_WFMT_SIGN1_RES8, QG_WFMT_Q4K, QG_WFMT_SIGN1_RES8Z, QG_WFMT_TERNARY3, QG_WFMT_INT8_T16, QG_ACT_INT8, QG_ACT_FLOAT, QG_MAX_OUTLIERS, QG_QGEMV_MAX_K,
                       QG_SEP_MAX_K, QG_BATCH_MAX_M, QG_BATCH_MAX_K, QG_MX_BLOCK, QG_QGEMM_MAX_K,
                       QG_ABSMAX_SCRATCH_PARTS, QG_ERR_DEVICE_CHECK)

__all__ = [n for n in dir() if not n.startswith("_")]
