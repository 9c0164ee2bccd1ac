"""Pins of the CPU reference's looped model (eq. 1 of the LoopSpec page, section 2.1).

* Against an independent formulation built from PyTorch library primitives (scaled dot
  product attention with a causal mask, rms_norm, silu, rotary embedding as complex
  multiplication), float64, whole-sequence recomputation of every depth.
* Cached token-by-token decoding equals full recomputation (depth-indexed caches).
* Special cases: zero output projections make every block the identity, so all readout
  depths agree; rotary embedding at position 0 is the identity and preserves norms;
  attention over one key returns its value.
"""

from dataclasses import replace

import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

from oracle.model import KV, Model
from synth import configs, inputs, weights


def _torch_reference(cfg, w, tokens):
    """Whole-sequence forward of P, B^r (r = 1..R) and C at every readout depth, float64,
    from library primitives.  Returns {r: logits[T, V]}."""
    t = lambda a: torch.tensor(np.asarray(a, np.float64))
    T = len(tokens)
    H, hd = cfg.n_heads, cfg.head_dim
    half = hd // 2
    pos = torch.arange(T, dtype=torch.float64)
    inv = cfg.rope_theta ** (-torch.arange(0, half, dtype=torch.float64) * 2.0 / hd)
    rot = torch.polar(torch.ones(T, half, dtype=torch.float64), pos[:, None] * inv[None, :])   # e^{i pos f}

    def rope(x):                                   # [T, H, hd]; pair (j, j+half) as a complex number
        z = torch.complex(x[..., :half], x[..., half:]) * rot[:, None, :]
        return torch.cat([z.real, z.imag], dim=-1)

    def block(lw, h):
        a = Fn.rms_norm(h, (cfg.d,), weight=t(lw["g1"]), eps=cfg.norm_eps)
        q = (a @ t(lw["Wq"]).T).view(T, H, hd)
        k = (a @ t(lw["Wk"]).T).view(T, H, hd)
        v = (a @ t(lw["Wv"]).T).view(T, H, hd)
        q, k = rope(q), rope(k)
        o = Fn.scaled_dot_product_attention(q.transpose(0, 1), k.transpose(0, 1), v.transpose(0, 1),
                                            is_causal=True).transpose(0, 1).reshape(T, cfg.d)
        h = h + o @ t(lw["Wo"]).T
        b = Fn.rms_norm(h, (cfg.d,), weight=t(lw["g2"]), eps=cfg.norm_eps)
        return h + (Fn.silu(b @ t(lw["Wg"]).T) * (b @ t(lw["Wu"]).T)) @ t(lw["Wd"]).T

    E = t(w["emb"])
    h = E[torch.tensor(tokens)]
    for lw in w["pre"]:
        h = block(lw, h)
    out = {}
    for r in range(1, cfg.R + 1):
        for lw in w["core"]:
            h = block(lw, h)
        if r in cfg.readout_depths:
            hc = h
            for lw in w["coda"]:
                hc = block(lw, hc)
            out[r] = (Fn.rms_norm(hc, (cfg.d,), weight=t(w["g_final"]), eps=cfg.norm_eps) @ E.T).numpy()
    return out


F64_TINY = replace(configs.TINY, name="tiny-f64", dtype="f64")
F64_HUG = replace(configs.MINI_HUGINN, name="mini-huginn-f64", dtype="f64", V=256)


@pytest.mark.parametrize("cfg", [F64_TINY, F64_HUG], ids=lambda c: c.name)
def test_model_matches_library_formulation(cfg):
    w = weights.make_weights(cfg, seed=0)
    toks = list(inputs.prompt(cfg.V, 12, seed=3))
    m = Model(cfg, w)
    got = m.new_seq().extend(toks, last_only=False)
    ref = _torch_reference(cfg, w, toks)
    for r in cfg.readout_depths:
        err = np.abs(got[r] - ref[r]).max() / np.abs(ref[r]).max()
        assert err < 1e-12, (r, err)


@pytest.mark.parametrize("cfg", [configs.TINY, replace(configs.MINI_HUGINN, dtype="f32", V=256)],
                         ids=lambda c: c.name)
def test_cached_decode_equals_recompute(cfg):
    w = weights.make_weights(cfg, seed=0)
    toks = list(inputs.prompt(cfg.V, 10, seed=4))
    m = Model(cfg, w)
    full = m.new_seq().extend(toks, last_only=False)
    seq = m.new_seq()
    seq.extend(toks[:4], last_only=False)
    for i in range(4, len(toks)):
        step = seq.extend([toks[i]])
        for r in cfg.readout_depths:
            ref = full[r][i]
            assert np.abs(step[r] - ref).max() <= 1e-5 * np.abs(ref).max(), (i, r)


def test_identity_block_makes_depths_agree():
    cfg = configs.TINY
    w = weights.make_weights(cfg, seed=0, zero=("Wo", "Wd"))
    m = Model(cfg, w)
    lg, hid = m.new_seq().extend(list(inputs.prompt(cfg.V, 6, seed=5)), keep_hidden=True)
    for r in range(1, cfg.R + 1):
        assert np.array_equal(hid[r], hid[0])
    assert np.array_equal(lg[2], lg[4])


def test_rope_special_cases():
    cfg = F64_TINY
    m = Model(cfg, weights.make_weights(cfg, seed=0))
    x = np.random.Generator(np.random.PCG64(0)).standard_normal((3, cfg.d))
    assert np.array_equal(m.rope(x, [0, 0, 0]), x)
    y = m.rope(x, [5, 17, 1000])
    nh = lambda a: np.linalg.norm(a.reshape(3, cfg.n_heads, cfg.head_dim), axis=-1)
    assert np.allclose(nh(y), nh(x), rtol=1e-13)
    # relative-position property: <rope(q, m), rope(k, n)> depends on m - n only
    q, k = x[:1], x[1:2]
    s = lambda a, b: (m.rope(q, [a]).reshape(cfg.n_heads, -1) * m.rope(k, [b]).reshape(cfg.n_heads, -1)).sum(-1)
    assert np.allclose(s(9, 4), s(105, 100), rtol=1e-10)


def test_single_key_attention_returns_value():
    cfg = F64_TINY
    m = Model(cfg, weights.make_weights(cfg, seed=0))
    kv = KV(cfg.d)
    rng = np.random.Generator(np.random.PCG64(1))
    k, v, q = rng.standard_normal((3, 1, cfg.d))
    kv.append(k, v)
    assert np.allclose(m.attention(q, kv, 0), v, rtol=1e-14)
