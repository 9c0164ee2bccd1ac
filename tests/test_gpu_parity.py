"""GPU parity of the libloopspec calls against the CPU reference, through the C ABI.

Every input is seeded and synthetic; the reference sees the same inputs, never a value the
GPU produced.  Tolerances (per-row relative L2): 1e-5 for the fp32 model, 2e-2 for bf16
models; verification outputs must be bit-identical.
"""

import ctypes as C
from dataclasses import replace

import numpy as np
import pytest
import torch

from oracle import philox as ophilox
from oracle import readout as oreadout
from oracle import sampler as osampler
from oracle.model import Model
from synth import configs, inputs, weights
from oracle import copyprop as ocopyprop
from tests.decode_checks import check_distribution
from tests.gpu_helpers import as_f64, branch_rows, kv_values, oracle_row_block, rel_l2, to_dev, tol

pytestmark = pytest.mark.gpu


def _L():
    from looped_transformer_self_amd import _lib
    return _lib

SMALL_CFGS = [configs.TINY, configs.MINI_OURO, configs.MINI_HUGINN]


def _engine(cfg, w, S, max_rows=32, max_jobs=256, prob_rows=64):
    from looped_transformer_self_amd.engine import Engine
    return Engine(cfg, w, slot_capacity=S, max_rows=max_rows, max_keys=S, max_jobs=max_jobs, prob_rows=prob_rows)


def _fill_cache(e, cfg, which, n_blocks, S, seed):
    vals = kv_values(cfg, n_blocks, S, seed)
    t = {"core": e.kv_core, "pre": e.kv_pre, "coda": e.kv_coda}[which]
    t.copy_(to_dev(vals).reshape(-1))
    return vals


def _fin_table(fin, S):
    t = torch.zeros(S, dtype=torch.int32, device="cuda")
    if fin:
        t[:len(fin)] = torch.tensor(fin, dtype=torch.int32, device="cuda")
    return t


@pytest.mark.parametrize("cfg", SMALL_CFGS, ids=lambda c: c.name)
@pytest.mark.parametrize("M,n_fin", [(5, 300), (20, 37), (1, 0), (40, 50), (128, 20)])
def test_loop_step_parity(cfg, M, n_fin):
    """Row counts across the kernel's row-tile variants (1, 2, 4 and 8 tiles of 16 rows), up
    to the workspace maximum of 128 rows per call."""
    print(f"[loop_step] {cfg.name} M={M} n_fin={n_fin}", flush=True)
    S = max(384, n_fin + 4 * M + 8)
    w = weights.make_weights(cfg, seed=0)
    e = _engine(cfg, w, S, max_rows=max(32, M))
    m = Model(cfg, w)
    kv = _fill_cache(e, cfg, "core", cfg.R * cfg.L, S, seed=11)
    H0 = inputs.hidden_rows(S, cfg.d, seed=12)
    e.H.copy_(torch.from_numpy(H0))
    rng = np.random.Generator(np.random.PCG64(13 + M))
    fin, slots, anc, pos, depth = branch_rows(M, n_fin, lambda i: 1 + (i * 3) % cfg.R, rng, S)
    fin_t = _fin_table(fin, S)
    rows = e.rows(slots, pos, depth, n_fin, anc, C.c_void_p(fin_t.data_ptr()))
    e.loop_step(rows)
    assert e.sync_status() == 0
    Hg = e.H.cpu().numpy()
    kvg = e.kv_core.view(cfg.R * cfg.L, S, 2, cfg.d).cpu().numpy()
    if cfg.dtype == "bf16":
        kvg = kvg.view(np.uint16)
    for i in range(M):
        k = depth[i]
        blocks = [as_f64(kv[(k - 1) * cfg.L + l], cfg) for l in range(cfg.L)]
        h_ref, kvs = oracle_row_block(m, m.core, H0[slots[i]][None].astype(np.float64), pos[i], fin + anc[i],
                                      blocks, cfg)
        assert rel_l2(Hg[slots[i]], h_ref[0]) <= tol(cfg), (i, rel_l2(Hg[slots[i]], h_ref[0]))
        for l in range(cfg.L):
            got = as_f64(kvg[(k - 1) * cfg.L + l, slots[i]], cfg)
            assert rel_l2(got[0], kvs[l][0]) <= tol(cfg) and rel_l2(got[1], kvs[l][1]) <= tol(cfg), (i, l)
    # rows not in the step keep their hidden state
    others = sorted(set(range(S)) - set(slots))
    assert np.array_equal(Hg[others], H0[others])


def _readout_ref(m, cfg, w, h, pos, keys, coda_blocks, j):
    """Oracle logits of C at readout index j for one hidden row."""
    hh = h[None].astype(np.float64)
    if cfg.L_coda:
        hh, _ = oracle_row_block(m, m.coda, hh, pos, keys, coda_blocks, cfg)
    a = m.rmsnorm(hh, m.g_final)
    from oracle.numerics import round_f32, store
    return round_f32(store(a, cfg.dtype) @ m.emb.T)[0]


@pytest.mark.parametrize("cfg", SMALL_CFGS, ids=lambda c: c.name)
@pytest.mark.parametrize("mode", ["greedy", "sample", "sample_t1"])
@pytest.mark.parametrize("M", [7, 37])
def test_readout_parity(cfg, mode, M):
    """7 rows in one launch; 37 rows in launches of 16, 16 and 5 rows (the row check runs with
    the first)."""
    print(f"[readout] {cfg.name} {mode} M={M}", flush=True)
    S = max(300, 260 + 4 * M + 8)
    greedy, T, top_p = {"greedy": (True, 1.0, 1.0), "sample": (False, 0.8, 0.9), "sample_t1": (False, 1.0, 0.9)}[mode]
    w = weights.make_weights(cfg, seed=0)
    e = _engine(cfg, w, S, max_rows=max(32, M))
    m = Model(cfg, w)
    nD = len(cfg.readout_depths)
    coda = _fill_cache(e, cfg, "coda", nD * cfg.L_coda, S, seed=21) if cfg.L_coda else None
    H0 = inputs.hidden_rows(S, cfg.d, seed=22)
    e.H.copy_(torch.from_numpy(H0))
    rng = np.random.Generator(np.random.PCG64(23))
    fin, slots, anc, pos, depth = branch_rows(M, 260, lambda i: i % nD, rng, S)
    fin_t = _fin_table(fin, S)
    out_rows = np.arange(M, dtype=np.int32)[::-1].copy()
    rows = e.rows(slots, pos, depth, 260, anc, C.c_void_p(fin_t.data_ptr()), extra=[out_rows])
    lg = torch.zeros(M, cfg.V, device="cuda")
    am = torch.zeros(M, dtype=torch.int32, device="cuda")
    e.readout(rows, greedy, T, top_p, rows.extra[0], argmax=am, logits=lg)
    assert e.sync_status() == 0
    lg, am, pg = lg.cpu().numpy(), am.cpu().numpy(), e.probs.cpu().numpy()
    for i in range(M):
        blocks = [as_f64(coda[depth[i] * cfg.L_coda + l], cfg) for l in range(cfg.L_coda)] if cfg.L_coda else []
        ref = _readout_ref(m, cfg, w, H0[slots[i]], pos[i], fin + anc[i], blocks, depth[i])
        assert rel_l2(lg[i], ref) <= tol(cfg), (i, rel_l2(lg[i], ref))
        assert am[i] == int(np.argmax(lg[i]))
        # the distribution: the reference processing of the GPU's own logits
        check_distribution(pg[out_rows[i]], lg[i], greedy, T, top_p)


def _py(P):
    return [int(x) for x in P]


def ocopyprop_threshold(tau):
    """The reference's screening threshold floor(tau * 2^40) (CopyLoop reading)."""
    return int(tau * (1 << ocopyprop.SHIFT))


@pytest.mark.parametrize("V", [37, 1000, 49152])
def test_verify_bit_exact(V):
    print(f"[verify] V={V}", flush=True)
    L = _L()
    cfg = replace(configs.TINY, V=V)
    w = weights.make_weights(replace(cfg, V=16), seed=0)
    w["emb"] = np.zeros((V, cfg.d), np.float32)
    e = _engine(cfg, w, S=16, max_jobs=256, prob_rows=48)
    n_rows = 48
    P = np.concatenate([inputs.distributions(16, V, 31, sparsity=0.0, peaked=1.0),
                        inputs.distributions(16, V, 32, sparsity=0.7, peaked=2.0),
                        inputs.distributions(16, V, 33, sparsity=0.95, peaked=0.5)])
    # a few one-hot rows (greedy readouts) and an exact copy (q == p)
    P[3] = 0; P[3, 5 % V] = 1
    P[4] = 0; P[4, 7 % V] = 1
    P[5] = P[6]
    e.probs.copy_(torch.from_numpy(P))
    fx = [osampler.fixed(p) for p in P]
    rng = np.random.Generator(np.random.PCG64(34))
    n_jobs = 240 if V < 10000 else 48
    jobs = np.zeros((n_jobs, 10), np.int32)
    us = inputs.uniforms_u32((n_jobs, 24), 35)
    cands_all = []
    thr_of = {}
    for k in range(n_jobs):
        op = k % 6
        p, q1, q2 = (int(x) for x in rng.integers(0, n_rows, 3))
        if k % 17 == 0:
            q1 = p
        x1 = osampler.sample(fx[q1], int(us[k, 0]))
        j = jobs[k]
        j[0], j[1], j[2], j[3], j[4] = op, p, q1, q2, x1
        res = (k // 6) % 3 != 2                      # every third DRAW2 / VERIFY job: non-residual
        if op in (2, 3) and not res:
            j[9] = L.LS_JOB_NON_RESIDUAL
        if op == 2:
            j[6] = k % 2
        if op == 3:
            g, x2 = osampler.draw2(fx[q1], fx[q2], x1, int(us[k, 1]), gated=bool(k % 2), residual=res)
            j[6], j[5] = int(g), x2
        if op in (4, 5):
            nc = int(rng.integers(0, 17))
            c = rng.choice(V, size=min(nc, V), replace=False).tolist()
            j[7], j[8] = len(cands_all), len(c)
            cands_all.extend(c)
        if op == 5:
            # thresholds around the candidates' masses: none, some and all survive
            tau = [0.0, 1.0 / V, 2.0 / V, 0.5][(k // 6) % 4]
            thr = ocopyprop_threshold(tau)
            thr_of[k] = thr
            j[4:6] = np.array([thr & 0xFFFFFFFF, thr >> 32], np.uint32).view(np.int32)
    out = e.verify(jobs, us, np.asarray(cands_all, np.int32) if cands_all else None)
    assert e.sync_status() == 0
    got_cands = e.last_cands
    for k in range(n_jobs):
        op, p, q1, q2, x1, x2, g, co, nc, fl = (int(v) for v in jobs[k][:10])
        u = [int(v) for v in us[k]]
        res = not (fl & L.LS_JOB_NON_RESIDUAL)
        if op == 0:
            want = (osampler.sample(fx[p], u[5]), osampler.DRAWN, 0)
        elif op == 1:
            want = (osampler.sample(fx[q1], u[0]), osampler.DRAWN, 0)
        elif op == 2:
            gate, t = osampler.draw2(fx[q1], fx[q2], x1, u[1], gated=bool(g), residual=res)
            want = (t, osampler.DRAWN, int(gate))
        elif op == 3:
            t, o = osampler.verify(fx[p], fx[q1], x1, u[2], u[4], bool(g), fx[q2], x2, u[3], residual=res)
            want = (t, o, 0)
        elif op == 4:
            t, o, jj = osampler.verify_copy(fx[p], cands_all[co:co + nc], u[8:8 + nc], u[4])
            want = (t, o, 0)
            assert out[k, 3] == jj
        else:
            cc = cands_all[co:co + nc]
            keep = [c for c in cc if fx[p][c] >= thr_of[k]]
            keep.sort(key=lambda c: (-fx[p][c], c))
            assert out[k, 3] == len(keep)
            assert got_cands[co:co + len(keep)].tolist() == keep
            assert sorted(got_cands[co:co + nc].tolist()) == sorted(cc)
            if keep:
                want = (-1, L.LS_OUT_SCREENED, 0)
            else:
                want = (osampler.sample(fx[p], u[0]), osampler.DRAWN, 0)
        assert tuple(int(v) for v in out[k, :3]) == want, (k, op, out[k], want)


@pytest.mark.parametrize("cfg", [configs.TINY, configs.MINI_OURO, configs.MINI_HUGINN], ids=lambda c: c.name)
def test_prelude_parity(cfg):
    print(f"[prelude] {cfg.name}", flush=True)
    S = 200
    w = weights.make_weights(cfg, seed=0)
    e = _engine(cfg, w, S)
    m = Model(cfg, w)
    pre = _fill_cache(e, cfg, "pre", cfg.L_pre, S, seed=41) if cfg.L_pre else None
    rng = np.random.Generator(np.random.PCG64(42))
    M = 6
    fin, slots, anc, pos, depth = branch_rows(M, 150, lambda i: 0, rng, S)
    toks = rng.integers(0, cfg.V, size=M).astype(np.int32)
    fin_t = _fin_table(fin, S)
    rows = e.rows(slots, pos, depth, 150, anc, C.c_void_p(fin_t.data_ptr()), extra=[toks])
    e.prelude(rows, rows.extra[0])
    assert e.sync_status() == 0
    Hg = e.H.cpu().numpy()
    for i in range(M):
        h = m.r32(m.emb[toks[i]][None])
        if cfg.L_pre:
            h, _ = oracle_row_block(m, m.pre, h, pos[i], fin + anc[i], [as_f64(pre[l], cfg) for l in range(cfg.L_pre)],
                                    cfg)
        assert rel_l2(Hg[slots[i]], h[0]) <= tol(cfg)


def test_descriptor_errors_are_reported_not_faulted():
    cfg = configs.TINY
    S = 64
    w = weights.make_weights(cfg, seed=0)
    e = _engine(cfg, w, S)
    fin_t = _fin_table([], S)
    from looped_transformer_self_amd import _lib as L
    # empty call
    rows = e.rows([], [], [], 0, [], C.c_void_p(fin_t.data_ptr()))
    e.loop_step(rows)
    assert e.sync_status() == L.LS_OK
    # slot out of range and depth out of range are rejected on the device
    rows = e.rows([S + 5, 3], [0, 0], [1, 9], 0, [[], []], C.c_void_p(fin_t.data_ptr()))
    e.loop_step(rows)
    assert e.sync_status() == L.LS_ERR_INVALID
    # host-side capacity checks
    with pytest.raises(L.LoopSpecError):
        e.loop_step(e.rows(list(range(40)), [0] * 40, [1] * 40, 0, [[]] * 40, C.c_void_p(fin_t.data_ptr())))


@pytest.mark.parametrize("cfg", [configs.TINY, configs.MINI_OURO, configs.MINI_HUGINN], ids=lambda c: c.name)
@pytest.mark.parametrize("bad", ["token", "slot"])
def test_prelude_bad_rows_are_reported_not_faulted(cfg, bad):
    """A token outside the vocabulary or a slot outside the cache in a prelude call is reported
    through the error word, with and without prelude layers; a good row of the same call still
    gets its embedding row (checked where P is the embedding alone)."""
    print(f"[prelude-bad] {cfg.name} {bad}", flush=True)
    S = 64
    w = weights.make_weights(cfg, seed=0)
    e = _engine(cfg, w, S)
    from looped_transformer_self_amd import _lib as L
    m = Model(cfg, w)
    fin = [0, 1, 2]
    slots, toks = [5, 6], np.array([3, 4], np.int32)
    if bad == "token":
        toks[1] = cfg.V + 10
    else:
        slots[1] = S + 3
    fin_t = _fin_table(fin, S)
    rows = e.rows(slots, [3, 3], [0, 0], len(fin), [[], []], C.c_void_p(fin_t.data_ptr()), extra=[toks])
    e.prelude(rows, rows.extra[0])
    assert e.sync_status() == L.LS_ERR_INVALID
    if not cfg.L_pre:
        Hg = e.H.cpu().numpy()
        assert rel_l2(Hg[5], m.r32(m.emb[3][None])[0]) <= tol(cfg)


@pytest.mark.parametrize("cfg", [configs.MINI_OURO, configs.MINI_HUGINN], ids=lambda c: c.name)
def test_readout_bad_rows_are_reported_not_faulted(cfg):
    """A readout row with a slot outside the cache or a readout depth outside the model's list is
    reported through the error word (the row check runs inside the LM-head kernel for models
    without coda layers); the good row of the call still gets its logits."""
    print(f"[readout-bad] {cfg.name}", flush=True)
    S = 64
    w = weights.make_weights(cfg, seed=0)
    e = _engine(cfg, w, S)
    from looped_transformer_self_amd import _lib as L
    e.H.copy_(torch.from_numpy(inputs.hidden_rows(S, cfg.d, seed=5)))
    fin_t = _fin_table([0, 1, 2], S)
    nD = len(cfg.readout_depths)
    for slots, depth in (([5, S + 2], [0, 0]), ([5, 6], [0, nD])):
        rows = e.rows(slots, [3, 3], depth, 3, [[], []], C.c_void_p(fin_t.data_ptr()),
                      extra=[np.arange(2, dtype=np.int32)])
        lg = torch.zeros(2, cfg.V, device="cuda")
        e.readout(rows, True, 1.0, 1.0, rows.extra[0], logits=lg)
        assert e.sync_status() == L.LS_ERR_INVALID
        assert np.all(np.isfinite(lg.cpu().numpy()[0])) and np.abs(lg.cpu().numpy()[0]).max() > 0


@pytest.mark.parametrize("bad", ["fin_slot", "ancestor_slot", "position"])
def test_bad_key_slots_are_reported_not_faulted(bad):
    """A prefix slot or an ancestor slot outside the cache, or a position that does not match
    the key count, is skipped by the kernels and reported through the error word; the call
    never reads outside the cache."""
    cfg = configs.TINY
    S = 64
    w = weights.make_weights(cfg, seed=0)
    e = _engine(cfg, w, S)
    from looped_transformer_self_amd import _lib as L
    fin = [0, 1, 2, 3]
    anc = [[], [10]]
    pos = [4, 5]
    if bad == "fin_slot":
        fin[2] = S + 7
    elif bad == "ancestor_slot":
        anc[1] = [-5]
    else:
        pos[1] = 9
    fin_t = _fin_table(fin, S)
    rows = e.rows([20, 21], pos, [1, 2], len(fin), anc, C.c_void_p(fin_t.data_ptr()))
    e.loop_step(rows)
    assert e.sync_status() == L.LS_ERR_INVALID


READ_MODES = {"greedy": (True, 1.0, 1.0), "t1-p0.9": (False, 1.0, 0.9), "t0.7-p0.95": (False, 0.7, 0.95),
              "t1-p1": (False, 1.0, 1.0)}


@pytest.mark.parametrize("V", [1000, 20000, 49152, 65536])
@pytest.mark.parametrize("mode", list(READ_MODES))
def test_readout_distribution_at_benchmark_vocabularies(V, mode):
    """LoopSpec page, section 2.1 (temperature, top-p, normalisation) at the vocabularies of
    the benchmark shapes: 49152 (Ouro) and 65536 (Huginn) plus 1000 and 20000, so every
    register-resident row layout of the distribution kernel runs (16, 32, 48 and 64 ids per
    thread).  A narrow model (d 256, bf16, the streaming LM-head kernel) keeps the reference
    cheap; the distribution is compared with the reference processing of the GPU's own
    logits, element by element."""
    print(f"[readout-V] V={V} {mode}", flush=True)
    greedy, T, top_p = READ_MODES[mode]
    cfg = replace(configs.MINI_OURO, V=V)
    w = weights.make_weights(cfg, seed=0)
    S = 64
    e = _engine(cfg, w, S, max_rows=16, prob_rows=16)
    m = Model(cfg, {**w, "core": [], "pre": [], "coda": []})
    M = 5
    H0 = inputs.hidden_rows(S, cfg.d, seed=70, scale=3.0)
    e.H.copy_(torch.from_numpy(H0))
    slots = [3, 9, 17, 30, 41]
    fin_t = _fin_table([0, 1], S)
    rows = e.rows(slots, [2] * M, [0, 1, 2, 2, 1], 2, [[]] * M, C.c_void_p(fin_t.data_ptr()),
                  extra=[np.arange(M, dtype=np.int32)])
    lg = torch.zeros(M, V, device="cuda")
    am = torch.zeros(M, dtype=torch.int32, device="cuda")
    e.readout(rows, greedy, T, top_p, rows.extra[0], argmax=am, logits=lg)
    assert e.sync_status() == 0
    lg, am, pg = lg.cpu().numpy(), am.cpu().numpy(), e.probs.cpu().numpy()
    e.close()
    from oracle.numerics import round_f32, store
    nb = 0
    for i in range(M):
        ref = round_f32(store(m.rmsnorm(H0[slots[i]][None].astype(np.float64), m.g_final), cfg.dtype) @ m.emb.T)[0]
        assert rel_l2(lg[i], ref) <= tol(cfg), (i, rel_l2(lg[i], ref))
        assert am[i] == int(np.argmax(lg[i]))
        nb += check_distribution(pg[i], lg[i], greedy, T, top_p)
    print(f"  top-p boundary tokens differing: {nb}", flush=True)


def test_wait_limit_gives_up_and_reports():
    """Every dependency wait inside a launch is bounded.  With the bound forced to zero from
    the host, every wait that would block gives up at its first poll: the launch still runs
    to its end (no wait is left spinning), it is reported as a timeout, and after the bound
    is restored and the workspace re-bound the same call is correct again."""
    import time
    L = _L()
    cfg = configs.MINI_OURO
    S = 128
    w = weights.make_weights(cfg, seed=0)
    e = _engine(cfg, w, S)
    m = Model(cfg, w)
    kv = _fill_cache(e, cfg, "core", cfg.R * cfg.L, S, seed=81)
    H0 = inputs.hidden_rows(S, cfg.d, seed=82)
    rng = np.random.Generator(np.random.PCG64(83))
    fin, slots, anc, pos, depth = branch_rows(3, 40, lambda i: 1 + i, rng, S)
    fin_t = _fin_table(fin, S)
    L.check(L.lib.ls_set_wait_limit(e.h, 0.0), "ls_set_wait_limit")
    e.H.copy_(torch.from_numpy(H0))
    t0 = time.perf_counter()
    e.loop_step(e.rows(slots, pos, depth, len(fin), anc, C.c_void_p(fin_t.data_ptr())))
    st = e.sync_status()
    dt = time.perf_counter() - t0
    assert st == L.LS_ERR_HIP and b"timed out" in L.lib.ls_last_error(), (st, L.lib.ls_last_error())
    assert dt < 1.0, dt
    L.check(L.lib.ls_set_wait_limit(e.h, 2.0), "ls_set_wait_limit")
    L.check(L.lib.ls_bind_workspace(e.h, e.ws_ptr, e.max_rows, e.max_keys, e.max_jobs, e.stream_ptr()),
            "ls_bind_workspace")
    e.H.copy_(torch.from_numpy(H0))
    e.loop_step(e.rows(slots, pos, depth, len(fin), anc, C.c_void_p(fin_t.data_ptr())))
    assert e.sync_status() == L.LS_OK
    Hg = e.H.cpu().numpy()
    for i in range(3):
        k = depth[i]
        blocks = [as_f64(kv[(k - 1) * cfg.L + l], cfg) for l in range(cfg.L)]
        h_ref, _ = oracle_row_block(m, m.core, H0[slots[i]][None].astype(np.float64), pos[i], fin + anc[i], blocks, cfg)
        assert rel_l2(Hg[slots[i]], h_ref[0]) <= tol(cfg)
    e.close()
