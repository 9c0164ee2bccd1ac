"""Pins of the CPU reference's readout processing and decoders.

Readout (LoopSpec page, section 2.1: temperature, optional truncation, normalisation):
sums to one; top_p = 1 is the plain softmax (library softmax); temperature to zero
tends to the argmax; top-p equals a brute-force search over token subsets on tiny
vocabularies.

Decoders (section 2.2-2.3 and eq. 9): greedy speculative decoding commits exactly the
greedy tokens of plain full-depth decoding; with identity blocks every proposal is
accepted and gamma reaches R/d1; gamma never exceeds R/d1; on a tiny-vocabulary model a
chi-square test over 10^5 seeds shows the first two committed tokens distributed as the
chain of p_R.
"""

import itertools
from dataclasses import replace

import numpy as np
import pytest
from scipy.special import softmax as sp_softmax
from scipy.stats import chi2

from oracle import copyprop, decode, philox, readout, sampler
from oracle.model import Model
from synth import configs, inputs, weights


def test_readout_sums_to_one_and_top_p_one_is_softmax():
    rng = np.random.Generator(np.random.PCG64(0))
    for T in (0.7, 1.0, 1.7):
        lg = rng.standard_normal(300).astype(np.float32) * 3
        p = readout.distribution(lg, greedy=False, T=T, top_p=1.0)
        assert abs(p.astype(np.float64).sum() - 1) < 1e-6
        assert np.allclose(p, sp_softmax(lg.astype(np.float64) / T), rtol=1e-6, atol=1e-12)
        q = readout.distribution(lg, greedy=False, T=T, top_p=0.8)
        assert abs(q.astype(np.float64).sum() - 1) < 1e-6


def test_low_temperature_tends_to_argmax():
    lg = np.array([0.1, 2.0, 1.99, -3.0], np.float32)
    p = readout.distribution(lg, greedy=False, T=1e-4, top_p=1.0)
    assert p[1] > 0.99999
    assert np.array_equal(readout.distribution(lg, greedy=True), np.array([0, 1, 0, 0], np.float32))
    # ties: lowest id wins
    assert readout.distribution(np.array([1.0, 3.0, 3.0], np.float32), greedy=True)[1] == 1.0


def _brute_top_p(p, top_p):
    """Smallest set of tokens whose mass reaches top_p; among sets of that size the one of
    largest mass, then the one whose sorted ids are smallest."""
    V = len(p)
    for k in range(1, V + 1):
        best = None
        for S in itertools.combinations(range(V), k):
            m = sum(p[i] for i in S)
            key = (m, tuple(-i for i in S))
            if best is None or key > best[0]:
                best = (key, S, m)
        if best[2] >= top_p:
            return set(best[1])
    return set(range(V))


def test_top_p_matches_brute_force():
    rng = np.random.Generator(np.random.PCG64(2))
    for trial in range(300):
        V = int(rng.integers(2, 9))
        lg = rng.standard_normal(V) * 2
        if trial % 5 == 0:
            lg[1] = lg[0]                                  # a tie
        p = readout.softmax_t(lg, 1.0)
        tp = float(rng.uniform(0.05, 0.99))
        got = set(np.nonzero(readout.top_p_keep(p, tp))[0].tolist())
        assert got == _brute_top_p(p, tp), (trial, p, tp)


@pytest.mark.parametrize("key", ["tiny", "mini-ouro-greedy", "mini-huginn"])
def test_greedy_speculative_equals_greedy_autoregressive(key):
    wl = configs.get(key)
    cfg, dec = wl.model, replace(wl.decode, new_tokens=10)
    m = Model(cfg, weights.make_weights(cfg, seed=0))
    prompt = inputs.prompt(cfg.V, dec.prompt_len, seed=dec.seed_p)
    ar = decode.ar_decode(m, prompt, dec.new_tokens, dec)
    sp, recs = decode.spec_decode_serial(m, prompt, dec.new_tokens, dec)
    assert sp == ar
    assert decode.gamma(recs[1:], cfg, dec) <= cfg.R / dec.d1 + 1e-12


def test_identity_blocks_accept_everything():
    cfg = replace(configs.TINY, readout_depths=(2, 3, 4))
    dec = configs.DecodeCfg(greedy=False, T=1.0, top_p=0.9, d1=2, d2=3, new_tokens=12, prompt_len=8)
    m = Model(cfg, weights.make_weights(cfg, seed=0, zero=("Wo", "Wd")))
    prompt = inputs.prompt(cfg.V, 8, seed=1)
    toks, recs = decode.spec_decode_serial(m, prompt, 12, dec)
    assert all(r["outcome"] == sampler.ACC1 for r in recs[1:])
    assert abs(decode.gamma(recs[1:], cfg, dec) - cfg.R / dec.d1) < 1e-12


@pytest.mark.parametrize("mode", ["single", "gated", "ungated"])
def test_chi_square_first_two_tokens_tiny_vocab(mode):
    """10^5 seeds on a V=8 looped model: the joint law of the first two committed tokens
    equals p_R(a | prompt) * p_R(b | prompt, a)."""
    cfg = configs.TINY_V8
    dec = configs.DecodeCfg(greedy=False, T=0.25, top_p=1.0, d1=2, d2=None if mode == "single" else 3,
                            gate=(mode != "ungated"), prompt_len=6)
    cfg = replace(cfg, readout_depths=(2, 3, 4))
    m = Model(cfg, weights.make_weights(cfg, seed=0))
    prompt = list(inputs.prompt(cfg.V, 6, seed=1))
    seq = m.new_seq()
    base = seq.extend(prompt)
    nxt = {}
    for a in range(cfg.V):
        s2 = m.new_seq()
        s2.extend(prompt)
        nxt[a] = s2.extend([a])
    dist = lambda lg: readout.distribution(lg, dec.greedy, dec.T, dec.top_p)
    P0 = sampler.fixed(dist(base[cfg.R]))
    T0 = len(prompt)
    N = 100_000
    counts = np.zeros((cfg.V, cfg.V))
    outcomes = np.zeros(6)
    for s in range(N):
        d = replace(dec, seed_s=s)
        a = sampler.sample(P0, philox.uniform(s, T0, philox.P_AR))
        rec = decode.decide(cfg, d, T0 + 1, nxt[a], prompt + [a])
        counts[a, rec["token"]] += 1
        outcomes[rec["outcome"]] += 1
    exp = np.zeros((cfg.V, cfg.V))
    pa = np.array(P0, np.float64) / sum(P0)
    for a in range(cfg.V):
        PR = np.array(sampler.fixed(dist(nxt[a][cfg.R])), np.float64)
        exp[a] = pa[a] * PR / PR.sum() * N
    ok = exp > 0
    assert counts[~ok].sum() == 0
    stat = float(((counts[ok] - exp[ok]) ** 2 / exp[ok]).sum())
    assert chi2.sf(stat, ok.sum() - 1) > 1e-4, stat
    # the cascade's branches are all exercised
    assert outcomes[sampler.RESAMPLED] > 500
    if mode != "single":
        assert outcomes[sampler.ACC2] > 500


def test_copy_candidates_rule():
    assert copyprop.candidates([5, 6, 7, 1, 5, 6, 7, 2, 5, 6, 7]) == [2, 1]
    assert copyprop.candidates([1, 2, 3, 4]) == []
    assert copyprop.candidates([9, 4, 9, 5, 9]) == [5, 4]           # n=1 fallback, most recent first
    A = [0, 10, 50, 50, 3]
    assert copyprop.screen([4, 2, 3, 1], A, tau=5 / (1 << 40)) == [2, 3, 1]


def test_copy_mode_greedy_equals_autoregressive():
    wl = configs.get("mini-huginn-copy")
    cfg = wl.model
    dec = replace(wl.decode, greedy=True, new_tokens=12)
    m = Model(cfg, weights.make_weights(cfg, seed=0))
    prompt = inputs.prompt(cfg.V, dec.prompt_len, seed=dec.seed_p, kind="segments")
    ar = decode.ar_decode(m, prompt, dec.new_tokens, dec)
    sp, recs = decode.spec_decode_serial(m, prompt, dec.new_tokens, dec)
    assert sp == ar
    assert any(r["cands"] for r in recs)
