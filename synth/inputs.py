"""Seeded synthetic inputs: prompts and random operands for kernel-level parity cases.

Nothing here computes any step of the decoding method; these are the data both the GPU
path and the CPU reference are fed.
"""

import numpy as np


def prompt(V: int, length: int, seed: int = 1, kind: str = "uniform") -> np.ndarray:
    """Prompt token ids (int32).

    kind="uniform": i.i.d. uniform over the vocabulary.
    kind="segments": seeded random 64-token segments, each repeated 3-6 times (uniform),
    concatenated until `length`, then 10% of positions replaced by uniform noise tokens.
    This mimics the repetitive contexts copy-suffix proposals feed on.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    if kind == "uniform":
        return rng.integers(0, V, size=length, dtype=np.int64).astype(np.int32)
    if kind != "segments":
        raise ValueError(kind)
    seg_len = 64 if length >= 256 else 16
    out = []
    while sum(len(s) for s in out) < length:
        seg = rng.integers(0, V, size=seg_len, dtype=np.int64)
        reps = int(rng.integers(3, 7))
        out.extend([seg] * reps)
    toks = np.concatenate(out)[:length].copy()
    noise = rng.random(length) < 0.10
    toks[noise] = rng.integers(0, V, size=int(noise.sum()), dtype=np.int64)
    return toks.astype(np.int32)


def hidden_rows(n: int, d: int, seed: int, scale: float = 1.0) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    return (rng.standard_normal((n, d), dtype=np.float32) * np.float32(scale)).astype(np.float32)


def bf16_bits_normal(shape, seed: int, scale: float = 1.0) -> np.ndarray:
    """Normal values rounded to bfloat16 (bit patterns, uint16)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal(size=shape, dtype=np.float32) * np.float32(scale)
    u = x.view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def distributions(n: int, V: int, seed: int, sparsity: float = 0.0, peaked: float = 1.0) -> np.ndarray:
    """n random probability vectors (float32 rows summing to ~1).

    Entries are exp(peaked * N(0,1)); a fraction `sparsity` of entries is zeroed (as
    top-p truncation does), keeping at least one nonzero entry per row.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    w = np.exp(peaked * rng.standard_normal((n, V)))
    if sparsity > 0:
        mask = rng.random((n, V)) < sparsity
        keep = rng.integers(0, V, size=n)
        mask[np.arange(n), keep] = False
        w[mask] = 0.0
    p = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
    return p


def uniforms_u32(shape, seed: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(0, 2**32, size=shape, dtype=np.uint64).astype(np.uint32)
