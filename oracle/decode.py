"""Plain full-depth autoregressive decoding and a serial speculative decoder (test
infrastructure only).

`ar_decode` is the plain definition the method must preserve (LoopSpec page,
section 1 and 2.2: every position runs all R loops before the next position starts; the
committed distribution is p_R).

`spec_decode_serial` makes, position by position, exactly the decisions of the pipelined
decoder of section 2.2-2.3: at depth d1 draw x~1 from q1 = p_d1; at d2 evaluate the gate
and draw the residual second proposal; at R run the cascade.  Because the KV caches are
depth-indexed, the hidden state of a position at depth r does not depend on how the
pipeline interleaved the work, so with the same position-keyed uniforms the pipelined
decoder commits the same tokens with the same outcomes.  With copy proposals (CopyLoop
page) the candidates of a position are screened at the shallow depth and verified by the
point-mass cascade; if none survive, a single self-speculative proposal is drawn at the
screening depth instead.

The branch cap of the pipelined decoder only decides which proposals get precomputed
rows; proposals are drawn and verified regardless, so it does not appear here.
"""

import numpy as np

from . import copyprop, philox, sampler
from .readout import distribution


def _dist(logits, dec):
    return distribution(logits, dec.greedy, dec.T, dec.top_p)


def ar_decode(model, prompt, n_new, dec, return_logits=False):
    """Full-depth autoregressive decoding; x_pos = SAMPLE(p_R, U(seed, pos, AR))."""
    cfg = model.cfg
    seq = model.new_seq()
    lg = seq.extend(list(prompt), depths=(cfg.R,))[cfg.R]
    toks, logits = [], []
    pos = len(prompt)
    for i in range(n_new):
        logits.append(lg)
        P = sampler.fixed(_dist(lg, dec))
        x = sampler.sample(P, philox.uniform(dec.seed_s, pos, philox.P_AR))
        toks.append(x)
        pos += 1
        if i + 1 < n_new:
            lg = seq.extend([x], depths=(cfg.R,))[cfg.R]
    return (toks, logits) if return_logits else toks


def distributions(cfg, dec, lg_by_depth):
    """Fixed-point readout distributions {depth: P} from logits {depth: logits}."""
    return {r: sampler.fixed(_dist(lg, dec)) for r, lg in lg_by_depth.items()}


def decide(cfg, dec, pos, lg_by_depth, prefix=None):
    """The decision at one position from its readouts {depth: logits}.

    Returns a record dict: token, outcome, x1, gate, x2 (and cands for copy mode).
    """
    return decide_fixed(cfg, dec, pos, distributions(cfg, dec, lg_by_depth), prefix)


def decide_fixed(cfg, dec, pos, P_by_depth, prefix=None, uniform=None):
    """The decision at one position from its fixed-point readout distributions
    {depth: P} (P(v) = floor(p(v) * 2^40)), with the position-keyed uniforms (or, for tests of
    how far a decision is from a boundary, uniform(purpose) in their place)."""
    R, d1, d2 = cfg.R, dec.d1, dec.d2
    seed = dec.seed_s
    residual = getattr(dec, "residual", True)
    U = uniform or (lambda purpose: philox.uniform(seed, pos, purpose))
    P_R = P_by_depth[R]
    rec = {"pos": pos, "x1": -1, "gate": False, "x2": -1, "cands": []}
    if dec.copy:
        s = dec.screen_depth
        P_s = P_by_depth[s]
        cands = copyprop.screen(copyprop.candidates(prefix, dec.copy_max_cands), P_s, dec.tau)
        rec["cands"] = cands
        if cands:
            Us = [U(philox.P_COPY0 + j) for j in range(len(cands))]
            tok, out, j = sampler.verify_copy(P_R, cands, Us, U(philox.P_RESAMPLE))
            rec.update(token=tok, outcome=out, j=j)
            return rec
        P_1 = P_s
    else:
        P_1 = P_by_depth[d1]
    x1 = sampler.draw1(P_1, U(philox.P_DRAW1))
    rec["x1"] = x1
    gate, x2, P_2 = False, -1, None
    if d2 is not None and not dec.copy:
        P_2 = P_by_depth[d2]
        gate, x2 = sampler.draw2(P_1, P_2, x1, U(philox.P_DRAW2), gated=dec.gate, residual=residual)
    rec["gate"], rec["x2"] = gate, x2
    tok, out = sampler.verify(P_R, P_1, x1, U(philox.P_ACC1), U(philox.P_RESAMPLE),
                              gate_open=gate, P_d2=P_2, x2=x2, U3=U(philox.P_ACC2), residual=residual)
    rec.update(token=tok, outcome=out)
    return rec


def forced_logits(model, prompt, forced, depths=None):
    """Logits along a teacher-forced stream, in one whole-sequence pass: returns a list whose
    entry i holds {r: logits} of the position that decides new token i (the last prompt
    position for i = 0, the position of forced[i - 1] after that).  Equal to the cached
    token-by-token decode of spec_decode_serial(forced=...) (pinned: cached decoding equals
    recomputation) at a fraction of its cost for large models."""
    cfg = model.cfg
    depths = cfg.readout_depths if depths is None else tuple(depths)
    toks = list(prompt) + list(forced[:-1])
    lg = model.new_seq().extend(toks, depths=depths, last_only=False)
    T0 = len(prompt)
    return [{r: lg[r][T0 - 1 + i] for r in depths} for i in range(len(forced))]


def spec_decode_serial(model, prompt, n_new, dec, forced=None, return_logits=False):
    """Serial speculative decoding.  The first new token comes from the prefill's p_R
    (as in plain decoding); every later position is decided by `decide`.

    forced: optional token list to teacher-force (the decisions are still computed at
    every position, but the prefix follows `forced`).
    """
    cfg = model.cfg
    seq = model.new_seq()
    depths = cfg.readout_depths
    lg = seq.extend(list(prompt), depths=depths)
    pos = len(prompt)
    P = sampler.fixed(_dist(lg[cfg.R], dec))
    x = sampler.sample(P, philox.uniform(dec.seed_s, pos, philox.P_AR))
    recs = [{"pos": pos, "token": x, "outcome": sampler.DRAWN, "x1": -1, "gate": False, "x2": -1, "cands": []}]
    logits = [lg]
    prefix = list(prompt)
    if forced is not None:
        x = forced[0]
    prefix.append(x)
    for i in range(1, n_new):
        pos += 1
        lg = seq.extend([x], depths=depths)
        logits.append(lg)
        rec = decide(cfg, dec, pos, lg, prefix)
        recs.append(rec)
        x = rec["token"] if forced is None else forced[i]
        prefix.append(x)
    toks = [r["token"] for r in recs]
    if return_logits:
        return toks, recs, logits
    return toks, recs


def gamma(recs, cfg, dec):
    """Mean acceptance length, LoopSpec eq. 9: N R / (N1 d1 + N2 d2 + (N - N1 - N2) R)."""
    N = len(recs)
    n1 = sum(1 for r in recs if r["outcome"] in (sampler.ACC1, sampler.ACC_COPY))
    n2 = sum(1 for r in recs if r["outcome"] == sampler.ACC2)
    d1 = dec.screen_depth if dec.copy else dec.d1
    d2 = dec.d2 if dec.d2 is not None else cfg.R
    return N * cfg.R / (n1 * d1 + n2 * d2 + (N - n1 - n2) * cfg.R)


def exact_commit_distribution(P_R, P_1, P_2=None, gated=True, residual=True):
    """Exact law of the committed token under the fixed-point sampler, by counting the
    uniform words that lead to each outcome (2^32 equally likely values per word).

    Returns a list of Fractions over the vocabulary.  Used to check losslessness
    (committed law == P_R / sum(P_R) up to quantisation) without sampling noise.
    """
    from fractions import Fraction
    V = len(P_R)
    W = 1 << 32

    def law_sample(A):
        # P(SAMPLE(A, U) = v) = #{U : cum_{v-1} <= floor(U Z / 2^32) < cum_v} / 2^32
        Z = sum(A)
        out, c = [], 0
        for a in A:
            lo = -(-c * W // Z)            # min U with floor(U Z / W) >= c  = ceil(c W / Z)
            c += a
            hi = -(-c * W // Z)
            out.append(Fraction(min(hi, W) - min(lo, W), W))
        return out

    def law_accept(num, den):
        # P(U * den < num * 2^32) = min(1, ceil(num W / den) / W)
        if den == 0:
            return Fraction(1)
        n_ok = min(W, -(-num * W // den))
        return Fraction(n_ok, W)

    res = [Fraction(0)] * V
    q1 = law_sample(P_1)
    r1 = sampler.resid(P_R, P_1)
    if sum(r1) == 0:
        r1 = list(P_R)
    for x1 in range(V):
        if q1[x1] == 0:
            continue
        a1 = law_accept(P_R[x1], P_1[x1])
        res[x1] += q1[x1] * a1
        rej = q1[x1] * (1 - a1)
        if rej == 0:
            continue
        r2 = sampler.proposal2(P_1, P_2, x1, residual) if P_2 is not None else None
        open_ = P_2 is not None and sum(r2) > 0 and (not gated or P_2[x1] < P_1[x1])
        if not open_:
            for v, pv in enumerate(law_sample(r1)):
                res[v] += rej * pv
            continue
        Z1, Z2 = sum(r1), sum(r2)
        r3 = [max(0, a * Z2 - b * Z1) for a, b in zip(r1, r2)]
        if sum(r3) == 0:
            r3 = r1
        l3 = law_sample(r3)
        for x2, q2 in enumerate(law_sample(r2)):
            if q2 == 0:
                continue
            a2 = law_accept(r1[x2] * Z2, Z1 * r2[x2])
            res[x2] += rej * q2 * a2
            rr = rej * q2 * (1 - a2)
            if rr:
                for v, pv in enumerate(l3):
                    res[v] += rr * pv
    return res
