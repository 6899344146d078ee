"""MI355X-native single-forward speculative verification.

The compute path is libsdv.so (hand-written HIP kernels for gfx950, C ABI in
include/sdv.h); `binding` marshals PyTorch device tensors into its calls.
"""
from .binding import (DeviceModel, PagedKV, Verifier, Sampler, accept_greedy, kv_rollback, prefill, pack_weights,  # noqa: F401
                      philox_uniforms, Drafter, tree_parent, HypothesisPool, Streams, lib, SdvError, LIB_PATH, PAGE, MAX_T, HEAD_LM, HEAD_CODEBOOK,
                      SAMPLE_NEAR_ACCEPT, SAMPLE_NEAR_DRAW, SAMPLE_BAD_DRAFT)
