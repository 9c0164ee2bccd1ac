"""Checks of a pipelined GPU decode against the CPU reference, position by position.

The GPU decoder runs with its readout trace on, so every committed position carries the
logits and distributions its branch read out at each readout depth.  For position i:

1. logits: the GPU's logits at every traced depth equal the reference's logits along the
   same (teacher-forced) token stream to the per-row relative L2 tolerance of the model's
   dtype (the reference computes the whole stream in one pass: cached decoding equals
   recomputation, a pinned property of the reference).  Where a second reference is given
   (the same model with float32-accumulated products), the tolerance at a position and
   depth is the larger of that and twice the second reference's own distance from the
   first: on random-init models many loop iterations amplify rounding-level differences
   (two correct implementations drift apart by ~2-4e-2 after 32 iterations of the
   Huginn-shaped block), while every single call stays within the tolerance (the loop-step
   and readout parity tests);
2. distribution: the GPU's distribution equals the reference readout processing (LoopSpec
   page, section 2.1: temperature, softmax, top-p, renormalisation) applied to the GPU's own
   logits: element by element to float32 rounding, with top-p membership allowed to differ
   only for tokens whose preceding mass lies within 1e-4 of top_p;
3. decision: (token, outcome, x1, gate, x2) equal the reference sampler's decision on the
   GPU's own distributions with the same position-keyed uniforms, exactly;
4. the reference's own decision (on its own logits) equals the GPU's wherever it is not
   within the measured error of a decision boundary.  Every comparison a decision makes is
   between a uniform word and a quantity of the distributions (an inverse-CDF position, an
   acceptance ratio), so a decision is robust to an error in the distributions that moves
   those quantities by less than d if it survives shifting each uniform by d: for a draw from
   p, any p' within L1 distance d samples like p with the uniform moved by at most d; ratios
   and residual draws move by at most the error divided by the smallest probability or
   residual mass involved.  d is set from the measured L1 and max differences between the
   GPU's and the reference's distributions at that position; positions where a shifted
   uniform changes the reference decision are counted and returned.  Greedy decisions
   compare argmaxes instead: their boundary is a top-2 tie of the logits at a depth the
   decision reads, within twice the measured elementwise logit error;
5. greedy: the committed token is the reference argmax wherever the reference's top-2 gap
   exceeds twice the largest elementwise logit difference measured at that position.
"""

import numpy as np

from oracle import decode as odecode
from oracle import philox
from oracle import readout as oreadout
from oracle import sampler as osampler


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def tol(cfg):
    return 1e-5 if cfg.dtype == "f32" else 2e-2


TOPP_SLACK = 1e-4        # preceding-mass window around top_p where membership may differ
P_REL = 2e-5             # elementwise relative tolerance of a renormalised probability
P_ABS = 1e-10


def check_distribution(p_gpu, logits_gpu, greedy, T, top_p):
    """Item 2 above for one row; returns the number of boundary tokens whose membership
    differs."""
    pg = np.asarray(p_gpu, np.float64)
    lg = np.asarray(logits_gpu, np.float32)
    if greedy:
        want = oreadout.greedy_onehot(lg).astype(np.float64)
        assert np.array_equal(pg, want), (int(np.argmax(pg)), int(np.argmax(lg)))
        return 0
    p = oreadout.softmax_t(lg, T)
    keep_ref = oreadout.top_p_keep(p, top_p)
    keep_gpu = pg > 0
    diff = np.nonzero(keep_ref != keep_gpu)[0]
    if len(diff):
        order = np.lexsort((np.arange(len(p)), -p))
        before = np.empty(len(p))
        before[order] = np.concatenate([[0.0], np.cumsum(p[order])[:-1]])
        assert np.all(np.abs(before[diff] - top_p) <= TOPP_SLACK), (len(diff), before[diff][:5])
    q = np.where(keep_gpu, p, 0.0)
    q /= q.sum()
    err = np.abs(pg - q) - (P_REL * q + P_ABS)
    assert err.max() <= 0, (float(np.max(np.abs(pg - q) / np.maximum(q, 1e-300))), int(np.argmax(err)))
    assert abs(pg.sum() - 1.0) < 1e-5
    return len(diff)


def _key(rec):
    return (int(rec["token"]), int(rec["outcome"]), int(rec["x1"]), bool(rec["gate"]), int(rec["x2"]))


def _decide(cfg, dec, pos, i, P, prefix, uniform=None):
    U = uniform or (lambda k: philox.uniform(dec.seed_s, pos, k))
    if i == 0:
        t = osampler.sample(P[cfg.R], U(philox.P_AR))
        return {"token": t, "outcome": osampler.DRAWN, "x1": -1, "gate": False, "x2": -1}
    return odecode.decide_fixed(cfg, dec, pos, P, prefix, uniform=U)


def _shift_robust(cfg, dec, pos, i, P, prefix, delta, key_of):
    """Whether the reference decision stays the same with each uniform word, and all of them
    together, shifted by +-delta (a fraction of 2^32)."""
    base = key_of(_decide(cfg, dec, pos, i, P, prefix))
    sh = int(min(1.0, delta) * 2.0 ** 32)
    purposes = [philox.P_DRAW1, philox.P_DRAW2, philox.P_ACC1, philox.P_ACC2, philox.P_RESAMPLE, philox.P_AR] + \
        [philox.P_COPY0 + j for j in range(dec.copy_max_cands if dec.copy else 0)]
    clamp = lambda u: min(max(u, 0), (1 << 32) - 1)
    orig = lambda k: philox.uniform(dec.seed_s, pos, k)
    trials = [(k, s) for k in purposes for s in (-1, 1)] + [(None, -1), (None, 1)]
    for k, sgn in trials:
        U = (lambda q, k=k, sgn=sgn: clamp(orig(q) + sgn * sh) if (k is None or q == k) else orig(q))
        if key_of(_decide(cfg, dec, pos, i, P, prefix, U)) != base:
            return False
    return True


def _residual_floor(cfg, dec, P):
    """Smallest normalised mass a decision at this position may divide by: 1, the residual
    masses of p_R (-) q1 and of the second proposal (when there is one)."""
    R = cfg.R
    one = float(1 << 40)
    zs = [1.0]
    q1 = P.get(dec.screen_depth if dec.copy else dec.d1)
    if q1 is not None:
        zs.append(sum(osampler.resid(P[R], q1)) / one)
        if dec.d2 is not None and not dec.copy and dec.d2 in P:
            zs.append(sum(osampler.resid(P[dec.d2], q1)) / one)
    return max(min(zs), 1e-3)


def check_stream(cfg, dec, model, prompt, toks, recs, mode="spec", lgs_alt=None):
    """Items 1-5 for a GPU decode (tokens and traced records).  lgs_alt: the stream's logits
    from the float32-product reference (forced_logits of Model(..., products="f32")), or
    None.  Returns a report dict."""
    T0 = len(prompt)
    lgs = odecode.forced_logits(model, prompt, toks)
    R = cfg.R
    rep = {"positions": len(toks), "max_rel_l2": 0.0, "max_rel_l2_alt": 0.0, "oracle_agree": 0, "near_boundary": 0,
           "greedy_checked": 0, "topp_boundary_tokens": 0}
    for i, rec in enumerate(recs):
        pos = T0 + i
        assert rec["pos"] == pos
        tr = rec["trace"]
        assert R in tr
        prefix = list(prompt) + list(toks[:i])
        worst = 0.0
        for r, (lg_g, p_g) in tr.items():
            e = rel_l2(lg_g, lgs[i][r])
            t = tol(cfg)
            if lgs_alt is not None:
                ea = rel_l2(lgs_alt[i][r], lgs[i][r])
                rep["max_rel_l2_alt"] = max(rep["max_rel_l2_alt"], ea)
                t = max(t, 2 * ea)
            assert e <= t, (i, r, e, t)
            worst = max(worst, e)
            rep["topp_boundary_tokens"] += check_distribution(p_g, lg_g, dec.greedy, dec.T, dec.top_p)
        rep["max_rel_l2"] = max(rep["max_rel_l2"], worst)
        # 3. the decision is the reference sampler's on the GPU's own distributions
        P = {r: osampler.fixed(p_g) for r, (lg_g, p_g) in tr.items()}
        if mode == "ar" and i > 0:
            want = {"token": osampler.sample(P[R], philox.uniform(dec.seed_s, pos, philox.P_AR)),
                    "outcome": osampler.DRAWN, "x1": -1, "gate": False, "x2": -1}
            assert int(rec["token"]) == want["token"], i
        else:
            want = _decide(cfg, dec, pos, i, P, prefix)
            assert _key(rec) == _key(want), (i, _key(rec), _key(want))
        # 4. the reference's own decision
        if mode == "spec" or i == 0:
            Pref = odecode.distributions(cfg, dec, {r: lgs[i][r] for r in tr})
            ref = _decide(cfg, dec, pos, i, Pref, prefix)
        else:
            ref = {"token": osampler.sample(odecode.distributions(cfg, dec, {R: lgs[i][R]})[R],
                                            philox.uniform(dec.seed_s, pos, philox.P_AR))}
        ar_step = mode == "ar" and i > 0
        same = int(rec["token"]) == int(ref["token"]) if ar_step else _key(rec) == _key(ref)
        if same:
            rep["oracle_agree"] += 1
        else:
            Pref = odecode.distributions(cfg, dec, {r: lgs[i][r] for r in tr})
            dp = [np.abs(np.asarray(tr[r][1], np.float64) - np.asarray(Pref[r], np.float64) / 2.0 ** 40) for r in tr]
            l1 = max(x.sum() for x in dp)
            linf = max(x.max() for x in dp)
            delta = 4 * max(l1, cfg.V * linf) / _residual_floor(cfg, dec, {r: Pref[r] for r in tr})
            if dec.greedy:
                # greedy decisions compare argmaxes: a boundary is a top-2 tie of the logits at a
                # depth the decision reads, within twice the measured elementwise logit error
                robust = True
                for r in tr:
                    lr = np.asarray(lgs[i][r], np.float64)
                    gap = np.diff(np.sort(lr)[-2:])[0]
                    if gap <= 2 * np.abs(np.asarray(tr[r][0], np.float64) - lr).max():
                        robust = False
            elif ar_step:
                key_of = lambda d: int(d["token"])
                Pd = {R: Pref[R]}
                robust = _shift_robust(cfg, dec, pos, 0, Pd, prefix, delta, key_of)
            else:
                robust = _shift_robust(cfg, dec, pos, i, Pref, prefix, delta, _key)
            assert not robust, (i, "GPU and reference decisions differ away from any boundary", _key(rec),
                                _key(ref), delta)
            rep["near_boundary"] += 1
        # 5. greedy tokens: wherever the measured logit errors cannot reorder the reference's
        # top token against any other (its logit minus its error above every other logit plus
        # that token's error), the committed token must be the reference's argmax
        if dec.greedy:
            lr = np.asarray(lgs[i][R], np.float64)
            err = np.abs(np.asarray(tr[R][0], np.float64) - lr)
            a = int(np.argmax(lr))
            if lr[a] - err[a] > np.delete(lr + err, a).max():
                assert int(rec["token"]) == a, i
                rep["greedy_checked"] += 1
    return rep


def run_gpu_decode(cfg, dec, w, prompt, n_new, mode="spec", max_jobs=256, fast_prefill=None):
    """Pipelined decode on the GPU with the readout trace on; the engine is closed after.
    fast_prefill: ls_prefill (True), the decode calls (False) or the decoder's default."""
    from looped_transformer_self_amd.decoder import Decoder
    from looped_transformer_self_amd.engine import Engine
    S = len(prompt) + n_new + 4 * dec.max_branches + 16
    e = Engine(cfg, w, slot_capacity=S, max_rows=max(16, min(128, dec.max_branches)), max_keys=S, max_jobs=max_jobs,
               prob_rows=4 * dec.max_branches + 16)
    try:
        d = Decoder(e, dec, mode, trace=True)
        d.prefill(prompt, fast=fast_prefill)
        toks = d.decode(n_new)
        recs = d.records[:n_new]
        st = d.stats()
    finally:
        e.close()
    return toks, recs, st
