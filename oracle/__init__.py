"""CPU oracle for the int8-weight MoE feed-forward layer (test infrastructure).

A plain, slow, fp64 NumPy statement of what the layer computes, written from
the Jamba-1.5 paper ("Model Architecture": top K=2 of n=16 experts per token,
MoE in place of the MLP; "Serving Considerations and Improvements": the
ExpertsInt8 scheme -- expert weights stored as INT8 and turned back into BF16
values before the contraction, no calibration, BF16 activations).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. The product path (the HIP library and its binding) never
calls it, and it imports nothing from the product path.

Modules:
  quant -- per-output-channel symmetric int8 quantizer and bf16 rounding.
  fp8   -- OCP e4m3 encoding and the per-output-channel fp8 quantizer of the
           FP8 weight comparator (the paper compares ExpertsInt8 with FP8).
  moe   -- router, top-K gate, permutation, SwiGLU experts, combine (the
           expert FFN takes any codes and per-row scales: int8, e4m3 values,
           or bf16 weights with unit scales).

Readings taken where the paper is silent:
  * gate = softmax over all n logits, keep the K largest, renormalise;
  * expert = SwiGLU: down(silu(gate x) * (up x)), no biases;
  * int8 = symmetric, per output channel, scale = absmax/127 rounded once
    (RNE) to the scale dtype, codes = RNE(w / stored scale) clamped to +-127;
  * the expert contraction is exact (fp64 here); the GPU's bf16 rounding of
    activations and intermediates is covered by the tolerance.

Every function's parity is pinned by tests that do not reuse its own formula:
see tests/test_oracle_*.py.
"""
from . import quant, fp8, moe  # noqa: F401
