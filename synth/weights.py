"""Seeded synthetic weights for a looped decoder (random init, no trained checkpoint).

Order of generation (NumPy PCG64(seed), standard normal scaled by init_std, float32):
embedding; then, for each prelude layer, each layer of the shared block and each coda
layer: Wq, Wk, Wv, Wo, Wgate, Wup, Wdown.  RMSNorm gains are ones.  The LM head is tied
to the embedding.  For bf16 models every matrix is rounded to bfloat16
(round-to-nearest-even) and returned as uint16 bit patterns; both the GPU path and the
CPU reference consume exactly these arrays.

Matrices follow the y = x @ W.T convention: W has shape [out_features, in_features].
"""

import numpy as np

LAYER_KEYS = ("Wq", "Wk", "Wv", "Wo", "Wg", "Wu", "Wd")


def _round_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even; inputs are finite."""
    u = x32.view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def _layer_shapes(cfg):
    d, F = cfg.d, cfg.F
    return {"Wq": (d, d), "Wk": (d, d), "Wv": (d, d), "Wo": (d, d), "Wg": (F, d), "Wu": (F, d), "Wd": (d, F)}


def make_weights(cfg, seed: int = 0, zero=()):
    """Return {"emb": [V,d], "pre": [layer dicts], "core": [...], "coda": [...], gains...}.

    `zero` names layer matrices (e.g. ("Wo", "Wd")) to replace by zeros after drawing,
    which turns every layer into the identity map on the residual stream (a special case
    used by tests).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    std = np.float32(cfg.init_std)
    bf16 = cfg.dtype == "bf16"

    def draw(shape):
        x = rng.standard_normal(size=shape, dtype=np.float32)
        x *= std
        return _round_bf16_bits(x) if bf16 else x

    out = {"emb": draw((cfg.V, cfg.d))}
    shapes = _layer_shapes(cfg)
    for part, n in (("pre", cfg.L_pre), ("core", cfg.L), ("coda", cfg.L_coda)):
        layers = []
        for _ in range(n):
            lw = {}
            for k in LAYER_KEYS:
                lw[k] = draw(shapes[k])
                if k in zero:
                    lw[k][...] = 0
            lw["g1"] = np.ones(cfg.d, np.float32)
            lw["g2"] = np.ones(cfg.d, np.float32)
            layers.append(lw)
        out[part] = layers
    out["g_final"] = np.ones(cfg.d, np.float32)
    return out


def weight_bytes(cfg):
    """Bytes of one application of the shared block B, of the head, and of prelude/coda."""
    es = 2 if cfg.dtype == "bf16" else 4
    per_layer = (4 * cfg.d * cfg.d + 3 * cfg.F * cfg.d) * es
    return {"block": cfg.L * per_layer, "head": cfg.V * cfg.d * es,
            "pre": cfg.L_pre * per_layer, "coda": cfg.L_coda * per_layer, "layer": per_layer}
