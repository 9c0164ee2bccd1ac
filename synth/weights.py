"""Seeded synthetic weights for a looped decoder (random init, no trained checkpoint).

Every matrix has a PCG64 stream of its own, seeded by (seed, tensor index) through NumPy's
SeedSequence, and is filled with standard normals scaled by init_std (float32).  Tensor
indices follow a fixed order: 0 the embedding; then, for each prelude layer, each layer of
the shared block and each coda layer, Wq, Wk, Wv, Wo, Wgate, Wup, Wdown.  Independent
streams let the matrices be drawn in parallel threads (NumPy releases the GIL while it
fills an array) without changing any value.  RMSNorm gains are ones.  The LM head is tied
to the embedding.  For bf16 models every matrix is rounded to bfloat16
(round-to-nearest-even) and returned as uint16 bit patterns; both the GPU path and the
CPU reference consume exactly these arrays.

Matrices follow the y = x @ W.T convention: W has shape [out_features, in_features].
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

LAYER_KEYS = ("Wq", "Wk", "Wv", "Wo", "Wg", "Wu", "Wd")
_ROWS_PER_PIECE = 1024          # rows drawn and rounded per piece of a large matrix


def _round_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even; inputs are finite."""
    u = x32.view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def _layer_shapes(cfg):
    d, F = cfg.d, cfg.F
    return {"Wq": (d, d), "Wk": (d, d), "Wv": (d, d), "Wo": (d, d), "Wg": (F, d), "Wu": (F, d), "Wd": (d, F)}


def _draw(seed, index, shape, std, bf16):
    """Tensor `index`: standard normals from its own stream, scaled, optionally rounded.
    Drawn in row pieces so that the float32 temporary of a large matrix stays small."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(index)])))
    out = np.empty(shape, np.uint16 if bf16 else np.float32)
    for r0 in range(0, shape[0], _ROWS_PER_PIECE):
        r1 = min(shape[0], r0 + _ROWS_PER_PIECE)
        x = rng.standard_normal(size=(r1 - r0,) + tuple(shape[1:]), dtype=np.float32)
        x *= std
        out[r0:r1] = _round_bf16_bits(x) if bf16 else x
    return out


def make_weights(cfg, seed: int = 0, zero=(), threads=None):
    """Return {"emb": [V,d], "pre": [layer dicts], "core": [...], "coda": [...], gains...}.

    `zero` names layer matrices (e.g. ("Wo", "Wd")) to replace by zeros after drawing,
    which turns every layer into the identity map on the residual stream (a special case
    used by tests).
    """
    std = np.float32(cfg.init_std)
    bf16 = cfg.dtype == "bf16"
    shapes = _layer_shapes(cfg)
    jobs = [("emb", None, None, (cfg.V, cfg.d))]
    for part, n in (("pre", cfg.L_pre), ("core", cfg.L), ("coda", cfg.L_coda)):
        for li in range(n):
            for k in LAYER_KEYS:
                jobs.append((part, li, k, shapes[k]))
    threads = threads or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(threads) as ex:
        arrs = list(ex.map(lambda ij: _draw(seed, ij[0], ij[1][3], std, bf16), enumerate(jobs)))
    out = {"emb": arrs[0]}
    for part, n in (("pre", cfg.L_pre), ("core", cfg.L), ("coda", cfg.L_coda)):
        out[part] = [dict() for _ in range(n)]
    for (part, li, k, _), a in zip(jobs[1:], arrs[1:]):
        lw = out[part][li]
        if k in zero:
            a[...] = 0
        lw[k] = a
    for part in ("pre", "core", "coda"):
        for lw in out[part]:
            lw["g1"] = np.ones(cfg.d, np.float32)
            lw["g2"] = np.ones(cfg.d, np.float32)
    out["g_final"] = np.ones(cfg.d, np.float32)
    return out


def weight_bytes(cfg):
    """Bytes of one application of the shared block B, of the head, and of prelude/coda."""
    es = 2 if cfg.dtype == "bf16" else 4
    per_layer = (4 * cfg.d * cfg.d + 3 * cfg.F * cfg.d) * es
    return {"block": cfg.L * per_layer, "head": cfg.V * cfg.d * es,
            "pre": cfg.L_pre * per_layer, "coda": cfg.L_coda * per_layer, "layer": per_layer}
