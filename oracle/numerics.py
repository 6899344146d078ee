"""Rounding helpers of the oracle (test infrastructure only)."""
import numpy as np


def bits_to_f64(u: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) or fp32 values to fp64 (exact)."""
    u = np.asarray(u)
    if u.dtype == np.uint16:
        return (u.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return u.astype(np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest bf16 value (8 significant bits), ties to even.

    frexp gives x = m * 2^e with 0.5 <= |m| < 1; m * 256 carries exactly the 8
    significant bits in its integer part, and rint rounds half to even.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0), e - 8)


def round_f32(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest fp32 value (ties to even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
