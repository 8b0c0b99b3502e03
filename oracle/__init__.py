"""CPU oracle for the QLoRA NF4 hot path -- TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, obviously-correct reference written from the
pages on QLoRA (NF4 storage, double quantization of the block constants,
dequantize-to-bf16 matmul with LoRA adapters). It exists so that the HIP path
can be checked against something independent of it.

Rules that keep it independent:
  * It shares no code, tables or constants with ``qlora_dequant_gemm_amd``
    and imports nothing from it; the product package never imports this one.
  * Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
    of ``bench.py`` may import or call anything in here.
  * Floating point is fp64 unless a step is defined in fp32 (the 32-bit block
    constants and the fp32 value that decides a 4-bit code), in which case the
    fp32 operation is written out with numpy float32 IEEE arithmetic.

Modules:
  nf4      -- codebook, nearest-code rule, block quantization, packing,
              double quantization of the constants, dequantization to bf16.
  gemm     -- forward y = x.deq(W)^T + (alpha/r).(x.A^T).B^T and
              backward dX = dY.deq(W) [+ LoRA term], in fp64.
  storage  -- bits/parameter and memory arithmetic from buffer byte counts.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
(closed forms, brute force, invariants, the pages' printed figures); none is
"parity unpinned".
"""
from . import nf4, gemm, storage  # noqa: F401
