"""Storage-precision helpers of the CPU reference (float64 arithmetic, rounded storage).

The LoopSpec page runs its models in BF16 (section 3.1).  The reference computes in
float64 and rounds to the model's storage type wherever a tensor is materialised in that
type: weights, the activations that enter a matrix product, and the KV cache.  The
residual stream, queries, products and probabilities are float32 tensors.
"""

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> exact float64 values."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), returned as float64.

    Done on the float64 value directly: the result is the bfloat16 number nearest to x,
    found by rounding the float64 significand to 8 bits.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)              # x = m * 2**e, 0.5 <= |m| < 1
    scaled = m * 256.0              # 8 significant bits (1 implicit + 7 stored)
    r = np.round(scaled)            # numpy rounds half to even
    return np.ldexp(r / 256.0, e)


def round_f32(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def store(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round to the model's storage type ("bf16", "f32", or "f64" = no rounding)."""
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f32":
        return round_f32(x)
    if dtype == "f64":          # unrounded: used only to pin the arithmetic itself
        return np.asarray(x, dtype=np.float64)
    raise ValueError(dtype)


def weight_f64(w: np.ndarray) -> np.ndarray:
    if w.dtype == np.uint16:
        return bf16_bits_to_f64(w)
    return w.astype(np.float64)
