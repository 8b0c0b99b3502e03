"""MI355X-native NF4 dequant-GEMM: the data-parallel hot path of QLoRA.

Block-wise NF4 quantization of a frozen weight, double quantization of its
block constants, and the fused dequantize-to-bf16 matmuls of one QLoRA linear
(forward with the LoRA term, backward to the input), as hand-written gfx950
HIP kernels behind the C ABI declared in include/qlora_nf4.h.
"""
from .ops import (NF4Weight, Workspace, bwd_dx, bwd_dx_batched, codebook, dequant, dq_scales,  # noqa: F401
                  lora_fwd, lora_fwd_batched, lora_fwd_grouped, lora_fwd_noalloc, quantize, quantize_dq,
                  quantize_weight, workspace_bytes)
