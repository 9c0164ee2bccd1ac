"""Shared set-up for the GPU parity tests: seeded inputs, engines, and the CPU reference
evaluated on exactly the same inputs (never on values produced by the GPU path)."""

import numpy as np
import torch

from oracle import numerics
from oracle.model import KV, Model
from synth import inputs, weights


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def tol(cfg):
    """Per-row relative L2 bound: 1e-5 for the fp32 model, 2e-2 for bf16 models."""
    return 1e-5 if cfg.dtype == "f32" else 2e-2


def kv_values(cfg, n_blocks, S, seed):
    """Random cache contents [n_blocks][S][2][d] in the storage dtype (bf16 bits / fp32)."""
    shape = (n_blocks, S, 2, cfg.d)
    if cfg.dtype == "bf16":
        return inputs.bf16_bits_normal(shape, seed)
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.standard_normal(shape, dtype=np.float32)


def as_f64(arr, cfg):
    return numerics.bf16_bits_to_f64(arr) if cfg.dtype == "bf16" else arr.astype(np.float64)


def to_dev(arr):
    if arr.dtype == np.uint16:
        arr = arr.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def oracle_row_block(m, layers, h, pos, key_slots, cache_blocks, cfg):
    """Apply `layers` (list of oracle layer dicts) to one hidden row at position pos whose
    earlier keys are the cache entries key_slots of cache_blocks[l] (float64 arrays
    [S][2][d]).  Returns the new row and the (k, v) it appended per layer."""
    kvs = []
    for l, lw in enumerate(layers):
        kv = KV(cfg.d, cap=len(key_slots) + 1)
        blk = cache_blocks[l]
        if key_slots:
            kv.append(blk[key_slots, 0, :], blk[key_slots, 1, :])
        h = m.layer(lw, h, pos, kv)
        kvs.append((kv.K[pos].copy(), kv.Vv[pos].copy()))
    return h, kvs


def branch_rows(n_rows, n_fin, depth_of_row, rng, S, max_anc=3):
    """Random branch rows: distinct slots; row i has a random ancestor path (slots of other
    speculative positions) of length <= max_anc; keys = finished prefix + path + self."""
    perm = rng.permutation(S)
    fin = perm[:n_fin].tolist()
    rest = perm[n_fin:].tolist()
    slots, anc = [], []
    for i in range(n_rows):
        na = int(rng.integers(0, max_anc + 1))
        a = [rest.pop() for _ in range(na)]
        anc.append(a)
        slots.append(rest.pop())
    pos = [n_fin + len(a) for a in anc]
    depth = [depth_of_row(i) for i in range(n_rows)]
    return fin, slots, anc, pos, depth
