"""Host-side branch scheduler of pipelined self-speculative decoding.

LoopSpec page, section 2.2-2.4.  A branch is a fixed prefix plus its current loop depth.
After prefill the first token is committed from p_R and a root branch starts.  Every
pipeline step advances every active branch by one loop iteration in one batched call of the
shared block; a branch reaching d1 draws x1 from q1 = p_d1 and immediately spawns the child
branch prefix+x1 while it keeps deepening; at d2 the gate p_d2(x1) < p_d1(x1) decides whether
a second, residual proposal x2 ~ p_d2 (-) p_d1 is drawn and spawned; the root reaching R runs
the cascade, commits a token, keeps the accepted child's subtree (re-rooting) and prunes the
rest, or restarts from the committed token.  Children reuse the parent's KV by slot index;
pruning only returns slots to the free list.

The second proposal is the residual p_d2 (-) p_d1 (eq. 5) or, as an ablation (Table 3),
p_d2 with x1 masked out; the gate can be switched off (ungated forking).

Copy-suffix proposals (CopyLoop page) replace the draws: at the screening depth a branch
takes the candidates copied from its context (host), the device keeps those with
p_s(c) >= tau in screening order, the branch spawns one child per survivor, and the root
verifies them with the point-mass cascade; with no survivor the same device job draws a
single proposal from p_s.

When the branch cap (or the slot pool) would be exceeded, a proposal is still drawn and
verified but gets no precomputed child; if it is accepted a fresh branch starts at depth 0,
so the committed tokens do not depend on the cap.

One upload of row descriptors and job arrays and one read-back of the verification results
per step are the only host<->device crossings.
"""

import ctypes
import time

import numpy as np
import torch

from . import _lib as L
from . import copyprop

PURPOSES = list(range(6)) + list(range(8, 24))   # uniform words per job (index = purpose)


class Node:
    __slots__ = ("slot", "pos", "token", "depth", "parent", "kids", "kind", "x1", "x2", "gate", "q1_row",
                 "q2_row", "child1", "child2", "cands", "copy_kids", "qs_row", "alive", "trace")

    def __init__(self, slot, pos, token, parent=None, kind="root"):
        self.slot, self.pos, self.token = slot, pos, token
        self.depth = 0
        self.parent = parent
        self.kids = []
        self.kind = kind
        self.x1, self.x2, self.gate = -1, -1, False
        self.q1_row = self.q2_row = self.qs_row = -1
        self.child1 = self.child2 = None
        self.cands = []          # screened copy candidates (ordered)
        self.copy_kids = {}      # token -> child
        self.alive = True
        self.trace = {}          # depth -> (logits, probs) host copies (decoders built with trace=True)


class CapacityError(RuntimeError):
    pass


class Decoder:
    def __init__(self, engine, dec, mode="spec", trace=False):
        """mode: "spec" (pipelined speculative decoding) or "ar" (plain full-depth decoding
        on the same kernels, proposals off: only the readout at R runs).  trace: keep a host
        copy of every readout's logits and distribution on its branch and hand the committed
        branch's copies out with its record (for tests; it synchronises after every readout)."""
        self.e = engine
        self.trace = trace
        self.cfg = engine.cfg
        self.dec = dec
        self.mode = mode
        self.D = list(self.cfg.readout_depths)
        self.didx = {r: j for j, r in enumerate(self.D)}
        self.free_slots = list(range(engine.S - 1, -1, -1))
        self.free_prob = list(range(engine.prob_rows - 1, -1, -1))
        self.fin = []
        self.fin_np = np.zeros(engine.S, np.int32)     # host mirror of fin, shipped with each step's rows
        self.fin_dev = torch.zeros(engine.S, dtype=torch.int32, device=engine.dev)
        self.fin_ptr = ctypes.c_void_p(self.fin_dev.data_ptr())
        self.tokens = []
        self.records = []
        self.rows_hist = []
        self.steps = 0

    # ---- bookkeeping ------------------------------------------------------------------
    def _slot(self):
        if not self.free_slots:
            raise CapacityError("KV slot pool exhausted")
        return self.free_slots.pop()

    def _prob(self):
        if not self.free_prob:
            raise CapacityError("probability row pool exhausted")
        return self.free_prob.pop()

    def _release_probs(self, n):
        for attr in ("q1_row", "q2_row", "qs_row"):
            r = getattr(n, attr)
            if r >= 0:
                self.free_prob.append(r)
                setattr(n, attr, -1)

    def _prune(self, n):
        """Free n and its whole subtree (slots and probability rows)."""
        stack = [n]
        while stack:
            x = stack.pop()
            x.alive = False
            self._release_probs(x)
            self.free_slots.append(x.slot)
            stack.extend(x.kids)
            x.kids = []

    def _fin_append(self, slots, device=True):
        """Commit slots to the finished prefix.  Decode steps ship the host mirror with their
        rows, so only prefill (device=True) writes the device table."""
        a = len(self.fin)
        self.fin.extend(slots)
        self.fin_np[a:a + len(slots)] = slots
        if not device:
            return
        if self.fin_dev.is_cuda:
            self.e.up.copy_to(self.fin_dev.data_ptr() + 4 * a, slots)
        else:                                   # host-only engines (scheduler tests)
            self.fin_dev[a:a + len(slots)] = torch.tensor(np.asarray(slots, np.int32))

    def _path(self, n):
        p = []
        x = n.parent
        while x is not None:
            p.append(x.slot)
            x = x.parent
        return p[::-1]

    def _nodes(self):
        out, stack = [], [self.root]
        while stack:
            x = stack.pop()
            out.append(x)
            stack.extend(reversed(x.kids))
        return out

    def _uniforms(self, pos):
        return L.philox_uniforms(self.dec.seed_s, pos, PURPOSES)

    @staticmethod
    def _urow(words):
        u = np.zeros(L.LS_UNIFORMS_PER_JOB, np.uint32)
        u[:6] = words[:6]
        u[8:24] = words[6:22]
        return u

    def _trace_args(self, n):
        """Extra readout arguments of a traced decoder: a logits buffer for n rows."""
        if not self.trace:
            return {}
        if getattr(self, "_tr_logits", None) is None or self._tr_logits.shape[0] < n:
            self._tr_logits = torch.zeros(max(n, self.e.max_rows), self.cfg.V, dtype=torch.float32, device=self.e.dev)
        return {"logits": self._tr_logits}

    def _trace_rows(self, rows, prob_rows):
        """Host copies (logits, probabilities) of readout rows after the readout completed."""
        if self.e.dev.type == "cuda":
            torch.cuda.synchronize(self.e.dev)
        lg = self._tr_logits.cpu().numpy()
        pr = self.e.probs.cpu().numpy()
        return [(lg[i].copy(), pr[j].copy()) for i, j in zip(rows, prob_rows)]

    # ---- prefill ----------------------------------------------------------------------
    def prefill(self, prompt, chunk=None, progress=None, fast=None):
        """Run the prompt through P, all R loops and the readouts, then commit the first new
        token from p_R of the last prompt position.  Not part of the timed decode.
        `progress(done, total)`, if given, is called after each chunk of prompt positions.
        fast (default: whenever the engine offers it): ls_prefill per chunk of prompt
        positions (every depth as large-M matrix products), then one readout of the last
        position; otherwise chunks of at most max_rows positions through the decode calls."""
        cfg, e = self.cfg, self.e
        prompt = [int(t) for t in prompt]
        T0 = len(prompt)
        if T0 == 0:
            raise ValueError("prefill needs at least one prompt token")
        if fast is None:
            fast = hasattr(e, "prefill")
        if fast:
            return self._prefill_fast(prompt, chunk or e.prefill_chunk, progress)
        chunk = chunk or e.max_rows
        last_row = -1
        for c0 in range(0, T0, chunk):
            toks = prompt[c0:c0 + chunk]
            n = len(toks)
            slots = [self._slot() for _ in range(n)]
            pos = list(range(c0, c0 + n))
            anc = [slots[:i] for i in range(n)]
            r0 = e.rows(slots, pos, [0] * n, c0, anc, self.fin_ptr, extra=[np.asarray(toks, np.int32)])
            e.prelude(r0, r0.extra[0])
            final = c0 + n == T0
            for k in range(1, cfg.R + 1):
                rk = e.rows(slots, pos, [k] * n, c0, anc, self.fin_ptr)
                e.loop_step(rk)
                # coda caches are filled at every readout depth a later decode step may read
                need = (cfg.L_coda and (self.mode == "spec" or k == cfg.R)) or (final and k == cfg.R)
                if k in self.didx and need:
                    out_rows = [-1] * n
                    if final and k == cfg.R:
                        last_row = self._prob()
                        out_rows[-1] = last_row
                    rr = e.rows(slots, pos, [self.didx[k]] * n, c0, anc, self.fin_ptr,
                                extra=[np.asarray(out_rows, np.int32)])
                    e.readout(rr, self.dec.greedy, self.dec.T, self.dec.top_p, rr.extra[0],
                              **self._trace_args(n))
                    if self.trace and final and k == cfg.R:
                        self.prefill_trace = {k: self._trace_rows([n - 1], [last_row])[0]}
            self._fin_append(slots)
            if progress is not None:
                progress(c0 + n, T0)
        return self._first_token(prompt, last_row)

    def _prefill_fast(self, prompt, chunk, progress):
        cfg, e = self.cfg, self.e
        T0 = len(prompt)
        # coda caches: every readout depth a later decode step may read (spec), R only (AR)
        mask = (1 << len(self.D)) - 1 if self.mode == "spec" else 1 << self.didx[cfg.R]
        slots = []
        for c0 in range(0, T0, chunk):
            toks = prompt[c0:c0 + chunk]
            slots = [self._slot() for _ in toks]
            e.prefill(toks, slots, c0, self.fin_ptr, mask)
            self._fin_append(slots)
            if progress is not None:
                progress(c0 + len(toks), T0)
        # p_R of the last position: its readout over the committed prefix before it
        last_row = self._prob()
        rr = e.rows([slots[-1]], [T0 - 1], [self.didx[cfg.R]], T0 - 1, [[]], self.fin_ptr,
                    extra=[np.asarray([last_row], np.int32)])
        e.readout(rr, self.dec.greedy, self.dec.T, self.dec.top_p, rr.extra[0], **self._trace_args(1))
        if self.trace:
            self.prefill_trace = {cfg.R: self._trace_rows([0], [last_row])[0]}
        return self._first_token(prompt, last_row)

    def _first_token(self, prompt, last_row):
        """Commit the first new token, drawn from the prefill's p_R row."""
        e = self.e
        T0 = len(prompt)
        self.prompt_len = T0
        self.tokens = list(prompt)
        job = np.zeros((1, 10), np.int32)
        job[0, 0], job[0, 1] = L.LS_JOB_SAMPLE, last_row
        out = e.verify(job, self._urow(self._uniforms(T0))[None, :])
        self.free_prob.append(last_row)
        x0 = int(out[0, 0])
        st = e.sync_status()
        if st != L.LS_OK:
            raise L.LoopSpecError(st, "prefill")
        self.tokens.append(x0)
        self.records.append({"pos": T0, "token": x0, "outcome": L.LS_OUT_DRAWN, "x1": -1, "gate": False, "x2": -1})
        if self.trace:
            self.records[-1]["trace"] = self.prefill_trace
        self.root = Node(self._slot(), T0, x0)
        self.pending = [self.root]
        return x0

    # ---- one pipeline step ------------------------------------------------------------
    def _spawn(self, parent, token, kind, n_active):
        if n_active >= self.dec.max_branches or not self.free_slots:
            return None
        c = Node(self._slot(), parent.pos + 1, token, parent, kind)
        parent.kids.append(c)
        self.pending.append(c)
        return c

    def step(self):
        cfg, e, dec = self.cfg, self.e, self.dec
        R = cfg.R
        spec = self.mode == "spec"
        n_fin = len(self.fin)
        self.steps += 1
        # the step's three row sets (prelude of branches spawned last step, one loop iteration
        # for every active branch, readouts at the depths in D) go to the device in one copy
        pn = [x for x in self.pending if x.alive]
        self.pending = []
        act = [x for x in self._nodes() if x.depth < R]
        paths = [self._path(x) for x in act]
        rd = [(x, p) for x, p in zip(act, paths) if x.depth + 1 in self.didx and (spec or x.depth + 1 == R)]
        out_rows = [self._prob() for _ in rd]
        specs = []
        if pn:
            specs.append(([x.slot for x in pn], [x.pos for x in pn], [0] * len(pn), n_fin, [self._path(x) for x in pn],
                          [np.asarray([x.token for x in pn], np.int32)]))
        specs.append(([x.slot for x in act], [x.pos for x in act], [x.depth + 1 for x in act], n_fin, paths, []))
        if rd:
            specs.append(([x.slot for x, _ in rd], [x.pos for x, _ in rd], [self.didx[x.depth + 1] for x, _ in rd], n_fin,
                          [p for _, p in rd], [np.asarray(out_rows, np.int32)]))
        rs = e.rows_set(specs, self.fin_np[:n_fin])
        # 1. prelude
        if pn:
            rp = rs.pop(0)
            e.prelude(rp, rp.extra[0])
        # 2. loop iteration
        e.loop_step(rs[0])
        self.rows_hist.append(len(act))
        for x in act:
            x.depth += 1
        # 3. readouts
        if not rd:
            return
        rr = rs[1]
        e.readout(rr, dec.greedy, dec.T, dec.top_p, rr.extra[0], **self._trace_args(len(rd)))
        if self.trace:
            for (x, _), tr in zip(rd, self._trace_rows(range(len(rd)), out_rows)):
                x.trace[x.depth] = tr
        # 4. verification / draw / screening jobs
        jobs, us, cands, tags = [], [], [], []
        tmp_rows = []
        flags = 0 if getattr(dec, "residual", True) else L.LS_JOB_NON_RESIDUAL
        screen_off = {}
        for (x, _), prow in zip(rd, out_rows):
            keep_row = False
            if x.depth == R:
                j = np.zeros(10, np.int32)
                if not spec:
                    j[0], j[1] = L.LS_JOB_SAMPLE, prow
                elif dec.copy and x.cands:
                    j[0], j[1], j[7], j[8] = L.LS_JOB_VERIFY_COPY, prow, len(cands), len(x.cands)
                    cands.extend(x.cands)
                else:
                    j[0], j[1], j[2] = L.LS_JOB_VERIFY, prow, x.q1_row
                    j[3] = x.q2_row if x.gate else -1
                    j[4], j[5], j[6] = x.x1, x.x2 if x.gate else -1, int(x.gate)
                    j[9] = flags
                jobs.append(j); tags.append(("verify", x)); us.append(self._urow(self._uniforms(x.pos + 1)))
            elif spec and dec.copy and x.depth == dec.screen_depth:
                # copy candidates from the committed prefix and the branch path (host); the
                # device keeps those reaching tau in screening order, or draws one proposal
                x.qs_row = prow
                keep_row = True
                prefix = self.tokens + [y.token for y in self._ancestors_and_self(x)]
                cc = copyprop.candidates(prefix, dec.copy_max_cands)
                thr = copyprop.threshold(dec.tau)
                j = np.zeros(10, np.int32)
                j[0], j[1], j[7], j[8] = L.LS_JOB_SCREEN, prow, len(cands), len(cc)
                j[4:6] = np.array([thr & 0xFFFFFFFF, thr >> 32], np.uint32).view(np.int32)
                screen_off[x] = len(cands)
                cands.extend(cc)
                jobs.append(j); tags.append(("screen", x)); us.append(self._urow(self._uniforms(x.pos + 1)))
            elif spec and not dec.copy and x.depth == dec.d1:
                x.q1_row = prow
                keep_row = True
                j = np.zeros(10, np.int32)
                j[0], j[2] = L.LS_JOB_DRAW1, prow
                jobs.append(j); tags.append(("draw1", x)); us.append(self._urow(self._uniforms(x.pos + 1)))
            elif spec and not dec.copy and dec.d2 is not None and x.depth == dec.d2:
                x.q2_row = prow
                keep_row = True
                j = np.zeros(10, np.int32)
                j[0], j[2], j[3], j[4], j[6] = L.LS_JOB_DRAW2, x.q1_row, prow, x.x1, int(dec.gate)
                j[9] = flags
                jobs.append(j); tags.append(("draw2", x)); us.append(self._urow(self._uniforms(x.pos + 1)))
            if not keep_row:
                tmp_rows.append(prow)
        res = e.verify(np.asarray(jobs, np.int32).reshape(-1, 10), np.asarray(us, np.uint32).reshape(-1, 24),
                       np.asarray(cands, np.int32) if cands else None) if jobs else np.zeros((0, 4), np.int32)
        for r in tmp_rows:
            self.free_prob.append(r)
        # 5. host updates: verification first (it decides which subtree survives)
        results = list(zip(tags, res))
        for (tag, x), o in results:
            if tag == "verify":
                self._commit(x, int(o[0]), int(o[1]), int(o[3]))
        n_active = sum(1 for y in self._nodes() if y.depth < R) + len(self.pending)
        spawn = []
        for (tag, x), o in results:
            if not x.alive:
                continue
            if tag == "draw1":
                x.x1 = int(o[0])
                spawn.append((-x.depth, 0, x, x.x1, "p1"))
            elif tag == "draw2":
                x.gate = bool(o[2])
                if x.gate:
                    x.x2 = int(o[0])
                    spawn.append((-x.depth, 1, x, x.x2, "p2"))
            elif tag == "screen":
                n_s = int(o[3])
                if n_s > 0:
                    # survivors, in screening order, at the front of the job's candidate range
                    c0 = screen_off[x]
                    x.cands = [int(c) for c in e.last_cands[c0:c0 + n_s]]
                    for c in x.cands:
                        spawn.append((-x.depth, 0, x, c, "copy"))
                else:
                    # no survivor: the job drew one proposal from p_s
                    x.q1_row, x.qs_row = x.qs_row, -1
                    x.x1 = int(o[0])
                    spawn.append((-x.depth, 0, x, x.x1, "p1"))
        spawn.sort(key=lambda t: (t[0], t[1]))
        for _, _, x, tok, kind in spawn:
            c = self._spawn(x, tok, kind, n_active)
            if c is not None:
                n_active += 1
            if kind == "p1":
                x.child1 = c
            elif kind == "p2":
                x.child2 = c
            elif c is not None:
                x.copy_kids[tok] = c

    def _ancestors_and_self(self, x):
        out = []
        while x is not None and x is not self.root:
            out.append(x)
            x = x.parent
        out = out[::-1]
        # the root's token is already committed (it is the last entry of self.tokens)
        return out

    def _commit(self, root, token, outcome, aux):
        """The root verified at depth R: commit, re-root onto the accepted child or restart."""
        assert root is self.root
        pos = root.pos + 1
        self.tokens.append(token)
        self.records.append({"pos": pos, "token": token, "outcome": outcome, "x1": root.x1, "gate": root.gate,
                             "x2": root.x2 if root.gate else -1, "aux": aux, "cands": list(root.cands)})
        if self.trace:
            self.records[-1]["trace"] = root.trace
        nxt = None
        if outcome == L.LS_OUT_ACC1:
            nxt = root.child1
        elif outcome == L.LS_OUT_ACC2:
            nxt = root.child2
        elif outcome == L.LS_OUT_ACC_COPY:
            nxt = root.copy_kids.get(token)
        for k in root.kids:
            if k is not nxt:
                self._prune(k)
        root.kids = []
        root.alive = False
        self._release_probs(root)
        self._fin_append([root.slot], device=False)
        if nxt is None or not nxt.alive:
            nxt = Node(self._slot(), pos, token)
            self.pending.append(nxt)
        nxt.parent = None
        self.root = nxt

    # ---- restart from the prefilled state ----------------------------------------------
    def snapshot(self):
        """Host state right after prefill.  Decoding never writes the prompt's slots, so
        restoring this state replays the same decode on the same device caches."""
        return {"prompt_len": self.prompt_len, "free_slots": list(self.free_slots), "free_prob": list(self.free_prob),
                "fin": list(self.fin),
                "tokens": list(self.tokens), "records": list(self.records), "root": (self.root.slot, self.root.pos,
                                                                                      self.root.token)}

    def restore(self, snap):
        """Return to a snapshot, also from another decoder of the same engine (e.g. plain
        decoding from a speculative decoder's prefill)."""
        self.prompt_len = snap["prompt_len"]
        self.free_slots = list(snap["free_slots"])
        self.free_prob = list(snap["free_prob"])
        self.fin = list(snap["fin"])
        self.fin_np[:len(self.fin)] = self.fin
        self.tokens = list(snap["tokens"])
        self.records = list(snap["records"])
        self.root = Node(*snap["root"])
        self.pending = [self.root]
        self.steps = 0
        self.rows_hist = []

    # ---- full decode ------------------------------------------------------------------
    def decode(self, n_new, progress=None):
        """Steps until n_new tokens (including the one from prefill) are committed.
        `progress(committed, n_new)`, if given, is called after each pipeline step."""
        while len(self.tokens) - self.prompt_len < n_new:
            self.step()
            if progress is not None:
                progress(len(self.tokens) - self.prompt_len, n_new)
        st = self.e.sync_status()
        if st != L.LS_OK:
            raise L.LoopSpecError(st, "decode")
        n = len(self.tokens) - self.prompt_len
        return self.tokens[self.prompt_len:self.prompt_len + n_new]

    def stats(self):
        recs = self.records[1:]
        cnt = lambda o: sum(1 for r in recs if r["outcome"] == o)
        R, d1 = self.cfg.R, self.dec.d1
        d2 = self.dec.d2 if self.dec.d2 is not None else R
        N = len(recs)
        n1, n2 = cnt(L.LS_OUT_ACC1) + cnt(L.LS_OUT_ACC_COPY), cnt(L.LS_OUT_ACC2)
        gamma = N * R / max(1, n1 * d1 + n2 * d2 + (N - n1 - n2) * R) if N else 0.0
        return {"steps": self.steps, "committed": N + 1, "accept1": n1, "accept2": n2,
                "fallback": cnt(L.LS_OUT_RESAMPLED), "gate_open": sum(1 for r in recs if r["gate"]),
                "gamma": gamma, "rows_mean": float(np.mean(self.rows_hist)) if self.rows_hist else 0.0,
                "rows_max": int(max(self.rows_hist)) if self.rows_hist else 0,
                "rows_hist": {int(k): int(v) for k, v in zip(*np.unique(self.rows_hist, return_counts=True))}
                if self.rows_hist else {}}


def generate(engine, prompt, n_new, dec, mode="spec"):
    """Prefill + decode; returns (tokens, records, stats) with decode-only wall time."""
    d = Decoder(engine, dec, mode)
    d.prefill(prompt)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    toks = d.decode(n_new)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    st = d.stats()
    st["decode_seconds"] = dt
    st["tokens_per_s"] = (n_new - 1) / dt if dt > 0 else 0.0
    return toks, d.records[:n_new], st
