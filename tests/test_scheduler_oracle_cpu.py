"""The pipelined branch scheduler against the serial reference decoder, on the CPU.

LoopSpec page, section 2.2-2.3: because the KV caches are depth-indexed, the hidden state
of a position at a given depth does not depend on how the pipeline interleaves the work, so
with the same position-keyed uniforms the pipelined decoder must commit exactly the tokens,
with exactly the outcomes, that the serial decoder commits one position at a time.  The
same holds for the copy-suffix proposals screened at a shallow depth (CopyLoop page) and
for the ablations of Table 3 (non-residual second proposal, ungated forking).

`OracleEngine` stands in for the device: its readouts are the reference model's
distributions for each row's token path (float64, recomputed per path), its verification
jobs follow the job contract of include/loopspec.h on the reference sampler.  Everything the
scheduler decides (spawns, prunes, re-roots, slot and probability-row reuse, job building,
screening thresholds, the branch cap) is what is under test.
"""

import ctypes
import types
from dataclasses import replace

import numpy as np
import pytest
import torch

from looped_transformer_self_amd import _lib as L
from looped_transformer_self_amd import decoder as D
from oracle import decode as odecode
from oracle import readout as oreadout
from oracle import sampler as osampler
from oracle.model import Model
from synth import configs, inputs, weights


class OracleEngine:
    def __init__(self, cfg, w, S=2048, prob_rows=256, max_rows=64):
        self.cfg = cfg
        self.model = Model(cfg, w)
        self.S, self.prob_rows, self.max_rows = S, prob_rows, max_rows
        self.dev = torch.device("cpu")
        self.probs = torch.zeros(prob_rows, cfg.V, dtype=torch.float32)
        self.tok = {}
        self.memo = {}
        self.loop_rows = []
        self.last_cands = np.zeros(0, np.int32)

    @staticmethod
    def _fin(fin_ptr, n):
        if n == 0:
            return []
        return [int(x) for x in (ctypes.c_int32 * n).from_address(fin_ptr.value)]

    @staticmethod
    def _rows(slots, pos, depth, fin, anc, extra):
        for p, a in zip(pos, anc):
            assert p == len(fin) + len(a)
        return types.SimpleNamespace(n=len(slots), slots=list(slots), pos=list(pos), depth=list(depth), fin=list(fin),
                                     anc=[list(a) for a in anc], extra=list(extra))

    def rows(self, slots, pos, depth, n_fin, anc, fin_ptr, extra=()):
        return self._rows(slots, pos, depth, self._fin(fin_ptr, n_fin), anc, extra)

    def rows_set(self, specs, fin):
        fin = [int(x) for x in fin]
        return [self._rows(sl, p, dp, fin[:nf], anc, extra) for sl, p, dp, nf, anc, extra in specs]

    def prelude(self, rows, tokens):
        for s, t in zip(rows.slots, tokens):
            self.tok[s] = int(t)

    def loop_step(self, rows):
        assert len(set(rows.slots)) == len(rows.slots)
        self.loop_rows.append(rows.n)

    noise = 0.0          # relative noise planted on the logits (tests of the decode checker)

    def readout(self, rows, greedy, T, top_p, out_rows, logits=None):
        for i in range(rows.n):
            o = int(out_rows[i])
            if o < 0:
                continue
            seq = tuple(self.tok[s] for s in rows.fin + rows.anc[i]) + (self.tok[rows.slots[i]],)
            if seq not in self.memo:
                self.memo[seq] = self.model.new_seq().extend(list(seq))
            lg = self.memo[seq][self.cfg.readout_depths[rows.depth[i]]]
            if self.noise:
                rng = np.random.Generator(np.random.PCG64(hash(seq) & 0xFFFFFFFF))
                lg = (lg * (1 + self.noise * rng.standard_normal(len(lg)))).astype(np.float32)
            if logits is not None:
                logits[i] = torch.from_numpy(np.asarray(lg, np.float32))
            self.probs[o] = torch.from_numpy(oreadout.distribution(lg, greedy, T, top_p))

    def verify(self, jobs, uniforms, cands=None):
        cands = [int(c) for c in cands] if cands is not None else []
        P = {}
        fx = lambda r: P.setdefault(r, osampler.fixed(self.probs[r].numpy()))
        out = np.zeros((len(jobs), 4), np.int32)
        for k, j in enumerate(jobs):
            op, pr, q1, q2, x1, x2, g, co, nc, fl = (int(v) for v in j)
            u = [int(v) for v in uniforms[k]]
            res = not (fl & L.LS_JOB_NON_RESIDUAL)
            if op == L.LS_JOB_SAMPLE:
                out[k] = (osampler.sample(fx(pr), u[5]), L.LS_OUT_DRAWN, 0, -1)
            elif op == L.LS_JOB_DRAW1:
                out[k] = (osampler.sample(fx(q1), u[0]), L.LS_OUT_DRAWN, 0, -1)
            elif op == L.LS_JOB_DRAW2:
                gate, t = osampler.draw2(fx(q1), fx(q2), x1, u[1], gated=bool(g), residual=res)
                out[k] = (t, L.LS_OUT_DRAWN, int(gate), -1)
            elif op == L.LS_JOB_VERIFY:
                t, o = osampler.verify(fx(pr), fx(q1), x1, u[2], u[4], bool(g), fx(q2) if g else None, x2, u[3],
                                       residual=res)
                out[k] = (t, o, 0, -1)
            elif op == L.LS_JOB_VERIFY_COPY:
                t, o, jj = osampler.verify_copy(fx(pr), cands[co:co + nc], u[8:8 + nc], u[4])
                out[k] = (t, o, 0, jj)
            elif op == L.LS_JOB_SCREEN:
                thr = (x1 & 0xFFFFFFFF) | ((x2 & 0xFFFFFFFF) << 32)
                A = fx(pr)
                cc = cands[co:co + nc]
                keep = sorted((c for c in cc if A[c] >= thr), key=lambda c: (-A[c], c))
                cands[co:co + nc] = keep + [c for c in cc if A[c] < thr]
                if keep:
                    out[k] = (-1, L.LS_OUT_SCREENED, 0, len(keep))
                else:
                    out[k] = (osampler.sample(A, u[0]), L.LS_OUT_DRAWN, 0, 0)
            else:
                raise AssertionError(op)
        self.last_cands = np.asarray(cands, np.int32)
        return out

    def sync_status(self):
        return L.LS_OK


def _run(wl, dec, n_new):
    cfg = wl.model
    w = weights.make_weights(cfg, seed=dec.seed_w)
    prompt = inputs.prompt(cfg.V, dec.prompt_len, seed=dec.seed_p, kind=dec.prompt_kind)
    e = OracleEngine(cfg, w)
    d = D.Decoder(e, dec, "spec")
    d.prefill(prompt)
    toks = d.decode(n_new)
    ref_toks, ref_recs = odecode.spec_decode_serial(e.model, prompt, n_new, dec)
    return d, e, toks, ref_toks, ref_recs


def _compare(d, toks, ref_toks, ref_recs, n_new):
    assert toks == ref_toks
    for i in range(1, n_new):
        g, r = d.records[i], ref_recs[i]
        got = (g["pos"], g["token"], g["outcome"], g["x1"], bool(g["gate"]), g["x2"])
        want = (r["pos"], r["token"], r["outcome"], r["x1"], bool(r["gate"]), r["x2"])
        assert got == want, (i, got, want)
        if r["cands"]:
            assert g["cands"] == r["cands"], i


TINY_S = replace(configs.TINY, readout_depths=(2, 3, 4))
CASES = {
    "greedy-single": (configs.TINY, configs.DecodeCfg(greedy=True, d1=2, max_branches=4, prompt_len=12)),
    "sample-single": (configs.TINY, configs.DecodeCfg(greedy=False, T=1.0, top_p=0.9, d1=2, prompt_len=12)),
    "sample-gated": (TINY_S, configs.DecodeCfg(greedy=False, T=1.0, top_p=0.9, d1=2, d2=3, prompt_len=12)),
    "sample-ungated": (TINY_S, configs.DecodeCfg(greedy=False, T=0.8, top_p=0.95, d1=2, d2=3, gate=False,
                                                 prompt_len=12)),
    "nonresidual-ungated": (TINY_S, configs.DecodeCfg(greedy=False, T=1.0, top_p=0.9, d1=2, d2=3, gate=False,
                                                      residual=False, prompt_len=12)),
    "nonresidual-gated": (TINY_S, configs.DecodeCfg(greedy=False, T=1.0, top_p=0.9, d1=2, d2=3, residual=False,
                                                    prompt_len=12)),
    "greedy-dual": (TINY_S, configs.DecodeCfg(greedy=True, d1=2, d2=3, prompt_len=12)),
}


@pytest.mark.parametrize("case", list(CASES))
def test_pipelined_equals_serial(case):
    cfg, dec = CASES[case]
    wl = configs.Workload(case, cfg, dec)
    n_new = 20
    d, e, toks, ref_toks, ref_recs = _run(wl, dec, n_new)
    _compare(d, toks, ref_toks, ref_recs, n_new)
    st = d.stats()
    assert st["gamma"] <= cfg.R / dec.d1 + 1e-9
    assert max(d.rows_hist) <= max(dec.max_branches, 1) + 1
    if case.startswith("sample-gated") or case.startswith("nonresidual"):
        # the cascade's second stage is exercised
        assert any(r["gate"] for r in d.records[1:])


MINI_COPY = configs.get("mini-huginn-copy")


@pytest.mark.parametrize("tau", [0.0, 0.03, 0.9], ids=["all-survive", "some-survive", "none-survive"])
def test_copy_proposals_pipelined_equals_serial(tau):
    """Copy-suffix candidates screened at depth 2 and verified by the point-mass cascade;
    with tau = 0.9 no candidate survives and every position falls back to one drawn
    proposal from the screening readout (the same device job).  A 32-token vocabulary makes
    copied candidates likely enough to be accepted."""
    cfg = replace(MINI_COPY.model, V=32)
    dec = replace(MINI_COPY.decode, prompt_len=64, tau=tau)
    wl = configs.Workload("copy", cfg, dec)
    n_new = 14
    d, e, toks, ref_toks, ref_recs = _run(wl, dec, n_new)
    _compare(d, toks, ref_toks, ref_recs, n_new)
    outs = [r["outcome"] for r in d.records[1:]]
    if tau == 0.0:
        assert L.LS_OUT_ACC_COPY in outs
        assert any(len(r["cands"]) > 1 for r in d.records[1:])
    if tau == 0.9:
        assert all(not r["cands"] for r in d.records[1:])


def test_branch_cap_keeps_the_serial_decisions():
    cfg, dec = CASES["sample-gated"]
    wl = configs.Workload("cap", cfg, dec)
    for cap in (1, 2):
        d, e, toks, ref_toks, ref_recs = _run(wl, replace(dec, max_branches=cap), 16)
        _compare(d, toks, ref_toks, ref_recs, 16)
        assert max(d.rows_hist) <= cap + 1


@pytest.mark.parametrize("noise", [0.0, 3e-3])
def test_decode_checker(noise):
    """The per-position checker the GPU decode tests use (tests/decode_checks.py), run on the
    CPU stand-in: with exact readouts every decision agrees with the reference; with noise
    planted on the readout logits the checker still passes (every decision equals the
    sampler's on the engine's own distributions, and every disagreement with the reference's
    own decision is flagged as within the measured error of a boundary), and a planted wrong
    decision is caught."""
    from tests.decode_checks import check_stream
    cfg, dec = CASES["sample-gated"]
    cfg = replace(cfg, dtype="bf16")           # the bf16 logit tolerance admits the planted noise
    w = weights.make_weights(cfg, seed=dec.seed_w)
    prompt = [int(t) for t in inputs.prompt(cfg.V, dec.prompt_len, seed=dec.seed_p)]
    e = OracleEngine(cfg, w)
    e.noise = noise
    d = D.Decoder(e, dec, "spec", trace=True)
    d.prefill(prompt)
    n_new = 16
    toks = d.decode(n_new)
    recs = d.records[:n_new]
    rep = check_stream(cfg, dec, e.model, prompt, toks, recs)
    if noise == 0.0:
        assert rep["oracle_agree"] == n_new and rep["max_rel_l2"] < 1e-12, rep
    else:
        assert rep["max_rel_l2"] > 1e-4
    bad = [dict(r) for r in recs]
    bad[5]["x1"] = (bad[5]["x1"] + 1) % cfg.V
    with pytest.raises(AssertionError):
        check_stream(cfg, dec, e.model, prompt, toks, bad)
