"""CPU oracle for the quantized GEMM hot path.  TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct numpy float64 implementations of what the library
computes: value decoders for the storage formats, dequantization, the dense and
MoE products, the MoE routing sort/pad, and the reference for the prepared-weight
byte layout.  Nothing here shares code with the HIP library, and nothing in the
library imports this package: only the tests, the smoke check and the benchmark's
CPU-baseline leg use it.

Sources followed (web pages on the Humming quantized-GEMM library):
* "Humming" (project README) -- "Key Features" and "Support Matrix": the weight,
  activation and scale types (int4, e2m1, e4m3, UE8M0, f16, bf16).
* "Humming: Fast, Flexible Kernels for Quantized Inference" -- the paragraphs on the
  standard format (weights, scales, zero points as separate parameters, groupwise
  INT4 with BF16 activations) and on the zero-exponent integer formats.
* "Humming" (wiki article) -- "Quantization representation" (channel / group / block
  scales, zero points, expert dimension) and "Device and workload selection" (the
  indexed MoE path that gathers rows through routing indices).
"""
