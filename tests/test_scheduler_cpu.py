"""Branch scheduler against a scripted stand-in for the device (CPU only).

LoopSpec page, section 2.2 and Fig. 1: with R = 4, plain decoding of three tokens takes
12 batched loop steps; a single proposal at depth 1 whose first proposal is rejected once
takes 9; adding a second proposal at depth 2 takes 7.  Under continuous acceptance the
commit interval tends to d1, under continuous rejection to R.  Section 3.4 (Table 6 text):
forking unconditionally at depths (2, 8) with R = 32 yields up to 249 branches in one
batched forward.  The cap on branches never changes the committed tokens.
"""

import types
from dataclasses import replace

import numpy as np
import pytest
import torch

from looped_transformer_self_amd import _lib as L
from looped_transformer_self_amd import decoder as D
from synth.configs import DecodeCfg, ModelCfg


class FakeEngine:
    """Stands in for the device: records the rows of every call, returns scripted outcomes.

    verify_script(job_kind, node_pos, k) -> (token, outcome, gate) decides draws and
    verifications; the scheduler's own bookkeeping is what is under test."""

    def __init__(self, cfg, script, S=4096, prob_rows=4096):
        self.cfg = cfg
        self.S = S
        self.prob_rows = prob_rows
        self.max_rows = 128
        self.dev = torch.device("cpu")
        self.script = script
        self.loop_rows = []
        self.probs = torch.zeros(1, 1)

    def rows(self, slots, pos, depth, n_fin, anc, fin_ptr, extra=()):
        for p, a in zip(pos, anc):
            assert p == n_fin + len(a)
        r = types.SimpleNamespace(n=len(slots), slots=list(slots), pos=list(pos), depth=list(depth), extra=list(extra))
        return r

    def rows_set(self, specs, fin):
        assert len(fin) == specs[0][3]
        return [self.rows(sl, p, dp, nf, anc, None, extra) for sl, p, dp, nf, anc, extra in specs]

    def prelude(self, rows, tok):
        pass

    def loop_step(self, rows):
        assert len(set(rows.slots)) == len(rows.slots), "a slot appears twice in one step"
        self.loop_rows.append(rows.n)

    def readout(self, rows, greedy, T, top_p, out_rows):
        pass

    def verify(self, jobs, uniforms, cands=None):
        out = np.zeros((len(jobs), 4), np.int32)
        for i, j in enumerate(jobs):
            out[i] = self.script(int(j[0]), j)
        return out

    def sync_status(self):
        return L.LS_OK


def _run(cfg, dec, script, n_new, mode="spec"):
    e = FakeEngine(cfg, script)
    d = D.Decoder(e, dec, mode)
    # a one-token "prompt" whose prefill commits the first token
    d.prefill([1])
    n_prefill_steps = len(e.loop_rows)
    toks = d.decode(n_new + 1)
    return d, e, e.loop_rows[n_prefill_steps:]


def _fig1_script(second):
    """Token 1 is rejected at the first proposal (accepted as the second one if a second
    proposal exists); tokens 2 and 3 are accepted as first proposals.  The gate opens only
    at the first branch."""
    state = {"verify": 0, "draw2": 0}

    def script(op, j):
        if op == L.LS_JOB_DRAW1:
            return (100, L.LS_OUT_DRAWN, 0, 0)
        if op == L.LS_JOB_DRAW2:
            state["draw2"] += 1
            return (200, L.LS_OUT_DRAWN, 1, 0) if state["draw2"] == 1 else (-1, L.LS_OUT_DRAWN, 0, 0)
        if op == L.LS_JOB_VERIFY:
            state["verify"] += 1
            if state["verify"] == 1:
                return (200, L.LS_OUT_ACC2, 0, 0) if second else (200, L.LS_OUT_RESAMPLED, 0, 0)
            return (100, L.LS_OUT_ACC1, 0, 0)
        if op == L.LS_JOB_SAMPLE:
            return (7, L.LS_OUT_DRAWN, 0, 0)
        raise AssertionError(op)
    return script


FIG_CFG = ModelCfg("fig1", V=8, d=32, n_heads=2, head_dim=16, F=32, L=1, R=4, dtype="f32", readout_depths=(1, 2, 4))


def test_fig1_standard_decoding_takes_12_steps():
    dec = DecodeCfg(greedy=True, d1=1, d2=None)
    d, e, rows = _run(FIG_CFG, dec, _fig1_script(False), 3, mode="ar")
    assert len(rows) == 12


def test_fig1_single_proposal_takes_9_steps():
    dec = DecodeCfg(greedy=True, d1=1, d2=None)
    d, e, rows = _run(FIG_CFG, dec, _fig1_script(False), 3)
    assert len(rows) == 9
    assert [r["outcome"] for r in d.records[1:4]] == [L.LS_OUT_RESAMPLED, L.LS_OUT_ACC1, L.LS_OUT_ACC1]


def test_fig1_second_proposal_takes_7_steps():
    dec = DecodeCfg(greedy=True, d1=1, d2=2)
    d, e, rows = _run(FIG_CFG, dec, _fig1_script(True), 3)
    assert len(rows) == 7
    assert [r["outcome"] for r in d.records[1:4]] == [L.LS_OUT_ACC2, L.LS_OUT_ACC1, L.LS_OUT_ACC1]


def _always(outcome, gate=1):
    def script(op, j):
        if op == L.LS_JOB_DRAW1:
            return (3, L.LS_OUT_DRAWN, 0, 0)
        if op == L.LS_JOB_DRAW2:
            return (4, L.LS_OUT_DRAWN, gate, 0) if gate else (-1, L.LS_OUT_DRAWN, 0, 0)
        if op == L.LS_JOB_VERIFY:
            return (3 if outcome == L.LS_OUT_ACC1 else 5, outcome, 0, 0)
        return (7, L.LS_OUT_DRAWN, 0, 0)
    return script


def test_commit_interval_acceptance_and_rejection():
    cfg = replace(FIG_CFG, R=8, readout_depths=(2, 8))
    dec = DecodeCfg(greedy=True, d1=2, d2=None, max_branches=64)
    n = 40
    d, e, rows = _run(cfg, dec, _always(L.LS_OUT_ACC1), n)
    # steady state: one commit every d1 steps (plus the first R - d1 fill)
    assert len(rows) == (cfg.R - dec.d1) + n * dec.d1
    d, e, rows = _run(cfg, dec, _always(L.LS_OUT_RESAMPLED), n)
    assert len(rows) == n * cfg.R
    st = d.stats()
    assert st["gamma"] <= cfg.R / dec.d1


def test_unconditional_forks_reach_249_rows():
    cfg = replace(FIG_CFG, R=32, readout_depths=(2, 8, 32))
    dec = DecodeCfg(greedy=True, d1=2, d2=8, gate=False, max_branches=10_000)
    d, e, rows = _run(cfg, dec, _always(L.LS_OUT_ACC1, gate=1), 40)
    assert max(rows) == 249


def test_cap_limits_rows_but_not_tokens():
    cfg = replace(FIG_CFG, R=32, readout_depths=(2, 8, 32))
    script_tokens = []

    def script(op, j):
        if op == L.LS_JOB_DRAW1:
            return (3, L.LS_OUT_DRAWN, 0, 0)
        if op == L.LS_JOB_DRAW2:
            return (4, L.LS_OUT_DRAWN, 1, 0)
        if op == L.LS_JOB_VERIFY:
            k = len(script_tokens)
            script_tokens.append(k)
            return [(3, L.LS_OUT_ACC1, 0, 0), (4, L.LS_OUT_ACC2, 0, 0), (6, L.LS_OUT_RESAMPLED, 0, 0)][k % 3]
        return (7, L.LS_OUT_DRAWN, 0, 0)

    outs = []
    for cap in (10_000, 16, 3, 1):
        script_tokens.clear()
        dec = DecodeCfg(greedy=True, d1=2, d2=8, gate=False, max_branches=cap)
        d, e, rows = _run(cfg, dec, script, 30)
        assert max(rows) <= max(cap, 1)
        outs.append(d.tokens)
    assert all(o == outs[0] for o in outs)
