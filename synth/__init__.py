"""Seeded synthetic inputs (shapes, weights, KV contents, tokens, logits, uniforms).

Shared by the oracle-side tests, the GPU tests and the bench; holds no part of
the verify method's arithmetic.
"""
from .configs import *  # noqa: F401,F403
from .gen import *  # noqa: F401,F403
