"""CPU oracle for single-forward speculative verification.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the bench's
CPU-baseline leg may import or run anything in this package; the product path
never does.  It shares no code with the HIP path.

It is plain NumPy in fp64, deliberately slow and direct.  Three numeric modes:

  EXACT    every value in fp64, no intermediate rounding: the mathematical
           definition.  Reference for fp32 models and for all property pins.
  BF16_KV  fp64 arithmetic on bf16 weights; the only rounding is of keys (after
           RoPE) and values to bf16 when they are written to the cache.
           Reference for bf16 models, whose kernels store weights and the KV cache
           in bf16 and carry activations at fp32 precision.
  BF16     additionally rounds every stored activation to bf16 (normed rows, q,
           attention output, SwiGLU output) and keeps an fp32 residual: a model
           that stores all activations in bf16.  Used to measure how far such
           rounding alone moves the logits.

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
BF16_KV = "bf16-kv"
