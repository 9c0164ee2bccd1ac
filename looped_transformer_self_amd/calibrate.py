"""Depth calibration for pipelined self-speculative decoding (LoopSpec page, section 2.4).

The page bounds the error of an intermediate readout by an empirical power-law envelope,
E_X[TV(p_r, p_R)] <= beta * r^(-alpha) (eq. 7), bounds the expected number of serial loop
steps per committed token by d1 + beta d1^(-alpha) d2 + 2 beta d2^(-alpha) R (eq. 11), and
gives the bound's stationary point in closed form (eq. 8): with D = alpha^2 + alpha + 1,
d1* = (alpha beta)^((alpha+1)/D) (2 alpha R)^(1/D), d2* = (alpha beta)^(alpha/D) (2 alpha R)^((alpha+1)/D).
Section 3.1 measures the TV curve at ten depths, averaged over token positions, at T = 1.0
and top-p 0.7, and draws the envelope over it.

This module measures TV(p_r, p_R) through the library (ls_prelude, ls_loop_step and
ls_readout at a set of depths, teacher-forced over prompt positions), fits the envelope,
and evaluates eq. 8 and eq. 11.  Readings where the page is silent: the envelope is the
least-squares line in log-log coordinates over the depths r < R, lifted (beta raised) until
it lies on or above every measured point; integer depths are the pair 1 <= d1 < d2 < R that
minimises eq. 11, optionally restricted to d2 and R being multiples of d1 (the page's
implementation constraint).

Command line: python -m looped_transformer_self_amd.calibrate --workload C4 [--positions N]
"""

import argparse
import json
import math
from dataclasses import replace

import numpy as np

from . import _lib as L

MAX_DEPTHS = L.LS_MAX_READOUT_DEPTHS


def continuous_optimum(alpha, beta, R):
    """Eq. 8: the stationary point (d1*, d2*) of the commit-cost bound."""
    D = alpha * alpha + alpha + 1.0
    ab = alpha * beta
    t = 2.0 * alpha * R
    return ab ** ((alpha + 1.0) / D) * t ** (1.0 / D), ab ** (alpha / D) * t ** ((alpha + 1.0) / D)


def commit_cost_bound(d1, d2, alpha, beta, R):
    """Eq. 11: upper bound on the expected serial loop steps per committed token."""
    return d1 + beta * d1 ** (-alpha) * d2 + 2.0 * beta * d2 ** (-alpha) * R


def best_integer_depths(alpha, beta, R, multiples=False):
    """The integer pair 1 <= d1 < d2 < R minimising eq. 11 (with multiples=True only pairs where
    d1 divides d2 and R).  Returns (d1, d2, bound)."""
    best = None
    for d1 in range(1, R):
        for d2 in range(d1 + 1, R):
            if multiples and (d2 % d1 or R % d1):
                continue
            c = commit_cost_bound(d1, d2, alpha, beta, R)
            if best is None or c < best[2]:
                best = (d1, d2, c)
    return best


def fit_envelope(depths, tv):
    """Power-law upper envelope beta * r^(-alpha) over measured mean TV values (eq. 7): the
    least-squares slope in log-log coordinates, with beta the smallest value that keeps the
    curve on or above every point.  Depths with TV = 0 (the full depth) are left out."""
    r = np.asarray(depths, np.float64)
    y = np.asarray(tv, np.float64)
    keep = y > 0
    r, y = np.log(r[keep]), np.log(y[keep])
    if len(r) < 2:
        raise ValueError("the envelope needs TV at two or more depths below R")
    slope, _ = np.polyfit(r, y, 1)
    alpha = -float(slope)
    log_beta = float(np.max(y + alpha * r))
    return alpha, math.exp(log_beta)


def depth_passes(R, extra=()):
    """Depth sets of at most MAX_DEPTHS readout depths (each ending with R) that together cover
    the depths to measure: every depth for R <= MAX_DEPTHS, else a geometric spread."""
    if R <= MAX_DEPTHS:
        want = list(range(1, R))
    else:
        want = sorted({1, 2, 3, 4, 6, 8, 12, 16, 20, 24, 28, R - 1} | set(extra))
        want = [r for r in want if 1 <= r < R]
    per = MAX_DEPTHS - 1
    return [tuple(want[i:i + per]) + (R,) for i in range(0, len(want), per)]


def tv_by_depth(cfg, weights, prompt, greedy=False, T=1.0, top_p=0.7, chunk=16, depths=None, device="cuda"):
    """TV(p_r, p_R) at every prompt position (teacher-forced) and every measured depth r,
    computed from the library's readouts.  Returns {r: float64 array over positions}."""
    import torch

    from .engine import Engine

    prompt = [int(t) for t in prompt]
    n = len(prompt)
    passes = [tuple(sorted(set(depths) | {cfg.R}))] if depths else depth_passes(cfg.R)
    out = {}
    for dset in passes:
        c2 = replace(cfg, readout_depths=dset)
        nd = len(dset)
        e = Engine(c2, weights, slot_capacity=n + 8, max_rows=chunk, max_keys=n + 8, max_jobs=4,
                   prob_rows=chunk * nd, device=device)
        try:
            fin = torch.zeros(n + 8, dtype=torch.int32, device=device)
            import ctypes
            fin_ptr = ctypes.c_void_p(fin.data_ptr())
            tv = {r: np.zeros(n) for r in dset}
            for c0 in range(0, n, chunk):
                toks = prompt[c0:c0 + chunk]
                m = len(toks)
                slots = list(range(c0, c0 + m))
                pos = slots
                anc = [slots[:i] for i in range(m)]
                r0 = e.rows(slots, pos, [0] * m, c0, anc, fin_ptr, extra=[np.asarray(toks, np.int32)])
                e.prelude(r0, r0.extra[0])
                for k in range(1, cfg.R + 1):
                    e.loop_step(e.rows(slots, pos, [k] * m, c0, anc, fin_ptr))
                    if k in dset:
                        j = dset.index(k)
                        rr = e.rows(slots, pos, [j] * m, c0, anc, fin_ptr,
                                    extra=[np.arange(j * chunk, j * chunk + m, dtype=np.int32)])
                        e.readout(rr, greedy, T, top_p, rr.extra[0])
                st = e.sync_status()
                if st != L.LS_OK:
                    raise L.LoopSpecError(st, "tv_by_depth")
                P = e.probs.cpu().numpy().astype(np.float64)
                pR = P[(nd - 1) * chunk:(nd - 1) * chunk + m]
                for j, r in enumerate(dset):
                    tv[r][c0:c0 + m] = 0.5 * np.abs(P[j * chunk:j * chunk + m] - pR).sum(axis=1)
                fin[c0:c0 + m] = torch.tensor(slots, dtype=torch.int32, device=device)
            for r in dset:
                out[r] = tv[r]
        finally:
            e.close()
    return dict(sorted(out.items()))


def calibrate(cfg, weights, prompt, greedy=False, T=1.0, top_p=0.7, skip=1, **kw):
    """Measure the TV curve, fit eq. 7's envelope and evaluate eq. 8 and eq. 11.  Positions
    before `skip` (the first tokens of the prompt) are left out of the averages."""
    tv = tv_by_depth(cfg, weights, prompt, greedy, T, top_p, **kw)
    R = cfg.R
    mean = {r: float(v[skip:].mean()) for r, v in tv.items()}
    rs = [r for r in mean if r < R]
    alpha, beta = fit_envelope(rs, [mean[r] for r in rs])
    d1c, d2c = continuous_optimum(alpha, beta, R)
    bi = best_integer_depths(alpha, beta, R)
    bm = best_integer_depths(alpha, beta, R, multiples=True)
    return {"mean_tv": mean, "alpha": alpha, "beta": beta, "d_star": (d1c, d2c),
            "bound_at_d_star": commit_cost_bound(d1c, d2c, alpha, beta, R) if 1 <= d1c < d2c else None,
            "best_integer": bi, "best_integer_multiples": bm, "positions": len(prompt) - skip,
            "T": T, "top_p": top_p, "greedy": greedy}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workload", default="C4")
    ap.add_argument("--positions", type=int, default=128)
    ap.add_argument("--T", type=float, default=1.0)
    ap.add_argument("--top-p", type=float, default=0.7)
    a = ap.parse_args()
    from synth import configs, inputs, weights as W
    wl = configs.get(a.workload)
    cfg, dec = wl.model, wl.decode
    w = W.make_weights(cfg, seed=dec.seed_w)
    prompt = inputs.prompt(cfg.V, a.positions, seed=dec.seed_p, kind=dec.prompt_kind)
    res = calibrate(cfg, w, prompt, T=a.T, top_p=a.top_p)
    res["workload"] = wl.key
    print(json.dumps(res))


if __name__ == "__main__":
    main()
