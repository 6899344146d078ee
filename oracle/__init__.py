"""CPU oracle for single-forward speculative verification.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the bench's
CPU-baseline leg may import or run anything in this package; the product path
never does.  It shares no code with the HIP path.

It is plain NumPy in fp64, deliberately slow and direct.  Two numeric modes:

  EXACT  every value in fp64, no intermediate rounding: the mathematical
         definition.  Reference for fp32 models and for all property pins.
  BF16   fp64 arithmetic that rounds to bf16 (nearest-even) exactly where a
         bf16 model stores bf16 values (normed activations, q/k/v after RoPE,
         attention output, SwiGLU output) and to fp32 where it keeps the fp32
         residual stream.  Reference for bf16 models.

Modules:
  numerics      bf16 / fp32 rounding, bf16 bit patterns to fp64
  decoder       the verify forward (and single-row decoding built on it)
  accept        greedy acceptance on a chain or a tree, commit plan, rollback
  spec_sampling speculative-sampling acceptance with residual resampling
  cfg           codebook heads and per-codebook classifier-free-guidance merge

Pins: every function here is checked in tests/ against something other than
itself (the pages' worked example and printed numbers, closed forms, brute
force on tiny inputs, invariants such as verify == token-by-token decoding).
"""
EXACT = "exact"
BF16 = "bf16"
