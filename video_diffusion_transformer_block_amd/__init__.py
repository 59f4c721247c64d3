"""vdtq: MI355X (gfx950) hot path of 6Bit-Diffusion's inference-time
mixed-precision quantization for video diffusion transformers.

Calls implemented in libvdtq.so (hand-written HIP for CDNA4) and
exposed through the C ABI in include/vdtq.h:

  hadamard_quantize  block Hadamard + NVFP4 / per-token INT8 / MXFP4 / MXFP8
                     quantization (or bf16 rounding for the fallback)
  qgemm_w4a4         NVFP4 activations x NVFP4 weights
  qgemm_w4a8         INT8 activations x NVFP4 weights
  qgemm_w4a16        bf16 activations x NVFP4 weights (fallback)
  qgemm_mx           MXFP4 / MXFP8 activations x MXFP4 weights (MX-native
                     variant on the block-scaled matrix instructions)
  qgemm_mx_quant     qgemm_mx whose epilogue emits the next linear's MX
                     activation (bias, GELU, Hadamard, MX encoding)
  block_stats        Gamma / delta-similarity / outlier reductions of a block
  block_stats_mx8    the same with the delta cache stored in MXFP8
  dmpq_step          host scheduler: SKIP / NVFP4 / INT8 / BF16 per block
  dmpq_budget_gamma  host: the step's Gamma threshold in bit-budget mode
  dmpq_depth_params  host: a block's skip thresholds under a depth profile

This module only marshals torch tensors into those calls.
"""
from ._lib import (ACT_BF16, ACT_INT8, ACT_NVFP4, ACT_SKIP, DmpqParams, DmpqState,  # noqa: F401
                   VdtqError, lib)
from .ops import (BF16Tensor, INT8Tensor, MXTensor, NVFP4Tensor, block_stats, block_stats_mx8,  # noqa: F401
                  dmpq_budget_gamma, dmpq_depth_params, dmpq_params, dmpq_state, dmpq_step, hadamard_quantize, outlier_ratio,
                  qgemm_mx, qgemm_mx_quant, qgemm_w4a4, qgemm_w4a8, qgemm_w4a16, workspace)

__all__ = ["hadamard_quantize", "qgemm_w4a4", "qgemm_w4a8", "qgemm_w4a16", "qgemm_mx", "qgemm_mx_quant", "block_stats",
           "block_stats_mx8", "dmpq_step", "dmpq_budget_gamma", "dmpq_depth_params", "dmpq_params", "dmpq_state", "outlier_ratio",
           "NVFP4Tensor", "INT8Tensor", "BF16Tensor", "MXTensor", "VdtqError", "lib"]
