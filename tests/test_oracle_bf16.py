"""Pins of the CPU reference's storage rounding (LoopSpec page, section 3.1: the models run in
BF16).  The reference computes in float64 and rounds to bfloat16 where a tensor is stored in
that type (weights, GEMM inputs, the KV cache) and to float32 elsewhere.

* `round_bf16` against PyTorch's float32 -> bfloat16 conversion (round to nearest, ties to
  even) on random values, exact ties, values next to ties and powers of two; and against the
  nearest bfloat16 number found by exact rational arithmetic for float64 inputs that float32
  cannot hold (where rounding through float32 first would round twice).
* The looped model at dtype "bf16" against a formulation from PyTorch library primitives
  (scaled dot product attention, rms_norm, silu, rotary embedding as complex
  multiplication) with the same bfloat16 / float32 casts at the same points.  The comparison
  is fine enough that rounding the queries to bfloat16 instead of float32, or a significand
  one bit short, is detected (both planted here on the CPU).
"""

from dataclasses import replace
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

from oracle import numerics
from oracle.model import Model
from synth import configs, inputs, weights


def _torch_bf16(x32):
    return torch.from_numpy(np.asarray(x32, np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def test_round_bf16_matches_torch_on_float32_values():
    rng = np.random.Generator(np.random.PCG64(7))
    vals = [rng.standard_normal(200_000).astype(np.float32),
            (rng.standard_normal(50_000) * 1e-30).astype(np.float32),
            (rng.standard_normal(50_000) * 1e30).astype(np.float32)]
    # exact ties: bfloat16 value + half an ulp (low 16 bits 0x8000), both parities of the kept bit
    hi = rng.integers(0x0080, 0x7F00, size=20_000, dtype=np.uint32)
    ties = ((hi << np.uint32(16)) | np.uint32(0x8000)).view(np.float32)
    vals += [ties, -ties]
    # next to ties, and powers of two with their neighbours
    for delta in (1, 0xFFFF - 0x8000, 0x7FFF):
        vals.append(((hi << np.uint32(16)) | np.uint32(0x8000 + delta if delta < 0x8000 else delta)).view(np.float32))
    p2 = np.ldexp(np.float32(1.0), np.arange(-120, 120)).astype(np.float32)
    vals += [p2, np.nextafter(p2, np.float32(0)), np.nextafter(p2, np.float32(np.inf)), -p2, np.zeros(3, np.float32)]
    x = np.concatenate(vals).astype(np.float32)
    got = numerics.round_bf16(x.astype(np.float64))
    want = _torch_bf16(x)
    assert np.array_equal(got, want), np.nonzero(got != want)[0][:10]


def _nearest_bf16_exact(x):
    """The bfloat16 number nearest to the float64 x (ties to an even significand), by exact
    rational arithmetic over the candidates m * 2^k with 128 <= |m| < 256."""
    if x == 0:
        return 0.0
    fx = Fraction(x)
    e = int(np.floor(np.log2(abs(x))))
    best = None
    for k in (e - 8, e - 7, e - 6):
        for m in range(128, 257):
            for s in (1, -1):
                c = Fraction(s * m) * Fraction(2) ** k
                dist = abs(c - fx)
                key = (dist, (m % 2) if m < 256 else 0)
                if best is None or key < best[0]:
                    best = (key, c)
    return float(best[1])


def test_round_bf16_is_the_nearest_bfloat16_for_float64_inputs():
    rng = np.random.Generator(np.random.PCG64(8))
    xs = list(rng.standard_normal(300) * 10.0 ** rng.integers(-20, 20, 300))
    # float64 values a hair above / below a tie: rounding through float32 first would land on the tie
    for m in rng.integers(128, 256, 60):
        for k in rng.integers(-30, 30, 2):
            tie = (float(m) + 0.5) * 2.0 ** int(k)
            xs += [tie, np.nextafter(tie, np.inf), np.nextafter(tie, -np.inf), -tie, tie * (1 + 2 ** -40),
                   tie * (1 - 2 ** -40)]
    x = np.asarray(xs, np.float64)
    got = numerics.round_bf16(x)
    want = np.asarray([_nearest_bf16_exact(v) for v in x])
    assert np.array_equal(got, want), [(v, g, w) for v, g, w in zip(x, got, want) if g != w][:5]


def _bf16_once(x):
    """float64 -> bfloat16 -> float64 with ONE rounding, from PyTorch's conversions.  torch
    converts float64 to bfloat16 through float32, which rounds twice: a float64 value a hair
    above a bfloat16 tie becomes the tie in float32 and then rounds to even.  Such values are
    moved one float32 ulp back towards the float64 value before the second conversion, so it
    sees which side of the tie they were on."""
    y = x.to(torch.float32)
    bits = y.view(torch.int32)
    on_tie = ((bits & 0xFFFF) == 0x8000) & (y.to(torch.float64) != x)
    toward_x = y + (x - y.to(torch.float64)).sign().to(torch.float32) * y.abs()
    y = torch.where(on_tie, torch.nextafter(y, toward_x), y)
    return y.to(torch.bfloat16).to(torch.float64)


def _torch_reference_rounded(cfg, w, tokens, q_bf16=False):
    """Whole-sequence forward from library primitives in float64, rounding where the model
    stores a tensor: bfloat16 for weights (already), normalised activations, keys, values,
    attention outputs and SwiGLU outputs; float32 for hidden rows, queries and products.
    q_bf16 rounds the queries to bfloat16 instead (a variant the reference must NOT match).
    Returns {r: logits[T, V]}."""
    t = lambda a: torch.tensor(np.asarray(a, np.float64))
    bf = _bf16_once
    f32 = lambda x: x.to(torch.float32).to(torch.float64)
    W = lambda a: t(numerics.weight_f64(a))
    T = len(tokens)
    H, hd = cfg.n_heads, cfg.head_dim
    half = hd // 2
    pos = torch.arange(T, dtype=torch.float64)
    inv = cfg.rope_theta ** (-torch.arange(0, half, dtype=torch.float64) * 2.0 / hd)
    rot = torch.polar(torch.ones(T, half, dtype=torch.float64), pos[:, None] * inv[None, :])

    def rope(x):
        xv = x.view(T, H, hd)
        z = torch.complex(xv[..., :half], xv[..., half:]) * rot[:, None, :]
        return torch.cat([z.real, z.imag], dim=-1).reshape(T, cfg.d)

    def block(lw, h):
        a = bf(Fn.rms_norm(h, (cfg.d,), weight=t(lw["g1"]), eps=cfg.norm_eps))
        q = f32(a @ W(lw["Wq"]).T)
        k = f32(a @ W(lw["Wk"]).T)
        v = bf(f32(a @ W(lw["Wv"]).T))
        q = bf(rope(q)) if q_bf16 else f32(rope(q))
        k = bf(rope(k))
        o = Fn.scaled_dot_product_attention(q.view(T, H, hd).transpose(0, 1), k.view(T, H, hd).transpose(0, 1),
                                            v.view(T, H, hd).transpose(0, 1), is_causal=True)
        o = bf(o.transpose(0, 1).reshape(T, cfg.d))
        h = f32(h + f32(o @ W(lw["Wo"]).T))
        b = bf(Fn.rms_norm(h, (cfg.d,), weight=t(lw["g2"]), eps=cfg.norm_eps))
        act = bf(Fn.silu(f32(b @ W(lw["Wg"]).T)) * f32(b @ W(lw["Wu"]).T))
        return f32(h + f32(act @ W(lw["Wd"]).T))

    E = W(w["emb"])
    h = f32(E[torch.tensor(tokens)])
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
            a = bf(Fn.rms_norm(hc, (cfg.d,), weight=t(w["g_final"]), eps=cfg.norm_eps))
            out[r] = f32(a @ E.T).numpy()
    return out


BF16_CFGS = [replace(configs.MINI_OURO, V=512), replace(configs.MINI_HUGINN, V=256, R=4, readout_depths=(2, 4))]
TOL = 2e-6          # max |difference| / max |logit|


def _max_rel(got, ref, cfg):
    return max(np.abs(got[r] - ref[r]).max() / np.abs(ref[r]).max() for r in cfg.readout_depths)


@pytest.fixture(scope="module", params=BF16_CFGS, ids=lambda c: c.name)
def bf16_case(request):
    cfg = request.param
    w = weights.make_weights(cfg, seed=0)
    toks = list(inputs.prompt(cfg.V, 12, seed=3))
    ref = _torch_reference_rounded(cfg, w, toks)
    return cfg, w, toks, ref


def test_bf16_model_matches_library_formulation(bf16_case):
    cfg, w, toks, ref = bf16_case
    got = Model(cfg, w).new_seq().extend(toks, last_only=False)
    err = _max_rel(got, ref, cfg)
    assert err < TOL, err
    # the comparison resolves a query rounding mistake: the reference is far from that variant
    var = _torch_reference_rounded(cfg, w, toks, q_bf16=True)
    assert _max_rel(got, var, cfg) > 10 * TOL


def test_bf16_pin_catches_a_short_significand(bf16_case, monkeypatch):
    """A planted mistake in the reference (7 significant bits instead of 8) fails the pin."""
    cfg, w, toks, ref = bf16_case

    def round7(x):
        x = np.asarray(x, dtype=np.float64)
        m, e = np.frexp(x)
        return np.ldexp(np.round(m * 128.0) / 128.0, e)

    monkeypatch.setattr(numerics, "round_bf16", round7)
    got = Model(cfg, w).new_seq().extend(toks, last_only=False)
    assert _max_rel(got, ref, cfg) > 10 * TOL


def test_bf16_cached_decode_equals_recompute():
    """Token-by-token decoding with the depth-indexed caches gives the whole-sequence result
    at dtype bf16 too (storage rounding happens per position, so the two agree up to float64
    summation order, which can move a rounding decision only in a rare last bit)."""
    cfg = BF16_CFGS[1]
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
            assert np.abs(step[r] - ref).max() <= 1e-4 * np.abs(ref).max(), (i, r)
