"""Parity at the benchmark's full model sizes, on sampled rows the CPU reference can compute
one by one (Ouro-1.4B, Ouro-2.6B and Huginn-3.5B shapes, bf16, through the C ABI, in the same
kernel configurations the benchmark uses).

Inputs are seeded and synthetic: weights from `synth.weights`, hidden rows and KV cache
entries from `synth.inputs`; only the cache entries the checked rows attend to are drawn,
the rest stay zero.  Tolerance: per-row relative L2 <= 2e-2 (bf16).
"""

import ctypes as C
import gc

import numpy as np
import pytest
import torch

from oracle.model import Model
from synth import configs, inputs, weights
from tests.decode_checks import check_distribution
from tests.gpu_helpers import as_f64, oracle_row_block, rel_l2, to_dev, tol

pytestmark = pytest.mark.gpu

FULL = {"C2": (configs.OURO_14, 768), "C3": (configs.OURO_26, 1536), "C4": (configs.HUGINN, 2048)}


@pytest.fixture(scope="module", params=["C2", "C3", "C4"])
def full_model(request):
    cfg, n_fin = FULL[request.param]
    print(f"[fullsize] {request.param}: drawing weights", flush=True)
    w = weights.make_weights(cfg, seed=0)
    from looped_transformer_self_amd.engine import Engine
    S = n_fin + 64
    e = Engine(cfg, w, slot_capacity=S, max_rows=16, max_keys=S, max_jobs=16, prob_rows=16)
    yield request.param, cfg, w, e, n_fin, S
    e.close()
    del e
    gc.collect()
    torch.cuda.empty_cache()


def _rows(cfg, n_fin, S, depths, seed):
    """Rows at the given depths: shared finished prefix of n_fin slots, 0-3 ancestors each."""
    rng = np.random.Generator(np.random.PCG64(seed))
    perm = rng.permutation(S)
    fin = perm[:n_fin].tolist()
    rest = perm[n_fin:].tolist()
    slots, anc = [], []
    for _ in depths:
        na = int(rng.integers(0, 4))
        anc.append([rest.pop() for _ in range(na)])
        slots.append(rest.pop())
    pos = [n_fin + len(a) for a in anc]
    return fin, slots, anc, pos


def _fill_blocks(e, cfg, tensor, blocks, slots, S, seed):
    """Draw cache entries for `slots` of each block index in `blocks`; returns {block: f64 [S][2][d]}."""
    view = tensor.view(-1, S, 2, cfg.d)
    ref = {}
    for bi, b in enumerate(blocks):
        vals = np.zeros((S, 2, cfg.d), np.uint16)
        vals[slots] = inputs.bf16_bits_normal((len(slots), 2, cfg.d), seed + bi)
        view[b].copy_(to_dev(vals).view(view.dtype))
        ref[b] = as_f64(vals, cfg)
    return ref


@pytest.mark.timeout(900)
def test_loop_step_full_size(full_model):
    key, cfg, w, e, n_fin, S = full_model
    depths = [cfg.R, 2, 1]
    fin, slots, anc, pos = _rows(cfg, n_fin, S, depths, seed=31)
    keyset = sorted(set(fin) | {x for a in anc for x in a})
    blocks = sorted({(k - 1) * cfg.L + l for k in depths for l in range(cfg.L)})
    print(f"[fullsize] {key}: loop_step, {len(depths)} rows, {n_fin} prefix keys", flush=True)
    ref_blocks = _fill_blocks(e, cfg, e.kv_core, blocks, keyset, S, seed=100)
    H0 = np.zeros((S, cfg.d), np.float32)
    H0[slots] = inputs.hidden_rows(len(slots), cfg.d, seed=32)
    e.H.copy_(torch.from_numpy(H0))
    fin_t = torch.tensor(fin, dtype=torch.int32, device="cuda")
    rows = e.rows(slots, pos, depths, n_fin, anc, C.c_void_p(fin_t.data_ptr()))
    e.loop_step(rows)
    assert e.sync_status() == 0
    Hg = e.H.cpu().numpy()
    kvg = e.kv_core.view(-1, S, 2, cfg.d)
    m = Model(cfg, {**w, "emb": w["emb"][:1], "pre": [], "coda": []})
    for i, k in enumerate(depths):
        blks = [ref_blocks[(k - 1) * cfg.L + l] for l in range(cfg.L)]
        h_ref, kvs = oracle_row_block(m, m.core, H0[slots[i]][None].astype(np.float64), pos[i], fin + anc[i], blks, cfg)
        err = rel_l2(Hg[slots[i]], h_ref[0])
        print(f"[fullsize] {key}: row {i} depth {k} rel-L2 {err:.2e}", flush=True)
        assert err <= tol(cfg), (i, err)
        for l in (0, cfg.L - 1):
            got = as_f64(kvg[(k - 1) * cfg.L + l, slots[i]].cpu().numpy().view(np.uint16), cfg)
            assert rel_l2(got[0], kvs[l][0]) <= tol(cfg) and rel_l2(got[1], kvs[l][1]) <= tol(cfg), (i, l)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("smp", [(False, 1.0, 0.9), (False, 0.7, 0.95), (True, 1.0, 1.0)],
                         ids=["t1-p0.9", "t0.7-p0.95", "greedy"])
def test_readout_full_size(full_model, smp):
    key, cfg, w, e, n_fin, S = full_model
    if key == "C3":
        pytest.skip("the Ouro-2.6B shape has the Ouro-1.4B readout")
    greedy, T, top_p = smp
    nD = len(cfg.readout_depths)
    js = [0, nD - 1]
    fin, slots, anc, pos = _rows(cfg, n_fin if cfg.L_coda else 8, S, js, seed=41)
    print(f"[fullsize] {key}: readout, {len(js)} rows, V={cfg.V}", flush=True)
    ref_blocks = {}
    if cfg.L_coda:
        keyset = sorted(set(fin) | {x for a in anc for x in a})
        blocks = sorted({j * cfg.L_coda + l for j in js for l in range(cfg.L_coda)})
        ref_blocks = _fill_blocks(e, cfg, e.kv_coda, blocks, keyset, S, seed=200)
    H0 = np.zeros((S, cfg.d), np.float32)
    H0[slots] = inputs.hidden_rows(len(slots), cfg.d, seed=42)
    e.H.copy_(torch.from_numpy(H0))
    fin_t = torch.tensor(fin if fin else [0], dtype=torch.int32, device="cuda")
    out_rows = np.arange(len(js), dtype=np.int32)
    rows = e.rows(slots, pos, js, len(fin), anc, C.c_void_p(fin_t.data_ptr()), extra=[out_rows])
    lg = torch.zeros(len(js), cfg.V, device="cuda")
    am = torch.zeros(len(js), dtype=torch.int32, device="cuda")
    e.readout(rows, greedy, T, top_p, rows.extra[0], argmax=am, logits=lg)
    assert e.sync_status() == 0
    lg, am, pg = lg.cpu().numpy(), am.cpu().numpy(), e.probs.cpu().numpy()
    m = Model(cfg, {**w, "core": [], "pre": []})
    from oracle.numerics import round_f32, store
    for r, j in enumerate(js):
        h = H0[slots[r]][None].astype(np.float64)
        if cfg.L_coda:
            blks = [ref_blocks[j * cfg.L_coda + l] for l in range(cfg.L_coda)]
            h, _ = oracle_row_block(m, m.coda, h, pos[r], fin + anc[r], blks, cfg)
        ref = round_f32(store(m.rmsnorm(h, m.g_final), cfg.dtype) @ m.emb.T)[0]
        err = rel_l2(lg[r], ref)
        print(f"[fullsize] {key}: readout row {r} rel-L2 {err:.2e}", flush=True)
        assert err <= tol(cfg), (r, err)
        assert am[r] == int(np.argmax(lg[r]))
        # the distribution: the reference processing of the GPU's own logits, element by element
        nb = check_distribution(pg[r], lg[r], greedy, T, top_p)
        print(f"[fullsize] {key}: readout row {r}: top-p boundary tokens differing {nb}", flush=True)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("M", [40, 128])
def test_loop_step_full_size_many_rows(full_model, M):
    """Ouro-1.4B shape with many rows per call: the row-tile variants for 4 and 8 tiles, the
    activation row staged in several chunks (RMSNorm factors from the per-tile sums of
    squares) and, at 128 rows, the shallower weight ring.  Three rows are checked."""
    key, cfg, w, _, _, _ = full_model
    if key != "C2":
        pytest.skip("one full-size shape is enough for the row-count variants")
    from looped_transformer_self_amd.engine import Engine
    n_fin = 256
    S = n_fin + 4 * M + 16
    e = Engine(cfg, w, slot_capacity=S, max_rows=M, max_keys=S, max_jobs=16, prob_rows=16)
    depths = [1 + (i * 3) % cfg.R for i in range(M)]
    fin, slots, anc, pos = _rows(cfg, n_fin, S, depths, seed=51 + M)
    check = [0, M // 2, M - 1]
    keyset = sorted(set(fin) | {x for i in check for x in anc[i]})
    blocks = sorted({(depths[i] - 1) * cfg.L + l for i in check for l in range(cfg.L)})
    print(f"[fullsize] {key}: loop_step, {M} rows, {n_fin} prefix keys, rows {check} checked", flush=True)
    ref_blocks = _fill_blocks(e, cfg, e.kv_core, blocks, keyset, S, seed=300)
    H0 = np.zeros((S, cfg.d), np.float32)
    H0[slots] = inputs.hidden_rows(len(slots), cfg.d, seed=52)
    e.H.copy_(torch.from_numpy(H0))
    fin_t = torch.tensor(fin, dtype=torch.int32, device="cuda")
    rows = e.rows(slots, pos, depths, n_fin, anc, C.c_void_p(fin_t.data_ptr()))
    e.loop_step(rows)
    assert e.sync_status() == 0
    Hg = e.H.cpu().numpy()
    kvg = e.kv_core.view(-1, S, 2, cfg.d)
    m = Model(cfg, {**w, "emb": w["emb"][:1], "pre": [], "coda": []})
    for i in check:
        k = depths[i]
        blks = [ref_blocks[(k - 1) * cfg.L + l] for l in range(cfg.L)]
        h_ref, kvs = oracle_row_block(m, m.core, H0[slots[i]][None].astype(np.float64), pos[i], fin + anc[i], blks, cfg)
        err = rel_l2(Hg[slots[i]], h_ref[0])
        print(f"[fullsize] {key}: {M} rows, row {i} depth {k} rel-L2 {err:.2e}", flush=True)
        assert err <= tol(cfg), (i, err)
        for l in (0, cfg.L - 1):
            got = as_f64(kvg[(k - 1) * cfg.L + l, slots[i]].cpu().numpy().view(np.uint16), cfg)
            assert rel_l2(got[0], kvs[l][0]) <= tol(cfg) and rel_l2(got[1], kvs[l][1]) <= tol(cfg), (i, l)
    e.close()
    del e
    gc.collect()
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("n_fin", [4800, 8192])
def test_loop_step_full_size_long_prefix(full_model, n_fin):
    """Huginn-3.5B shape with a 4800-key finished prefix, and with the stress workload's
    8192-key context: 55 heads x 75 (128) key chunks give every consumer wave several chunks,
    so each attention unit walks several 64-key sub-units (the last unit a ragged number of
    them) before its partial is merged; rows sharing a depth walk the same units one after
    another (groups of 2, 3 and 1 rows)."""
    key, cfg, w, _, _, _ = full_model
    if key != "C4":
        pytest.skip("the long-prefix unit layout needs many heads and keys (Huginn shape)")
    from looped_transformer_self_amd.engine import Engine
    S = n_fin + 64
    e = Engine(cfg, w, slot_capacity=S, max_rows=16, max_keys=S, max_jobs=16, prob_rows=16)
    depths = [cfg.R, cfg.R, 2, 2, 2, 1]                  # depth groups of 2, 3 and 1 rows
    fin, slots, anc, pos = _rows(cfg, n_fin, S, depths, seed=61)
    keyset = sorted(set(fin) | {x for a in anc for x in a})
    blocks = sorted({(k - 1) * cfg.L + l for k in depths for l in range(cfg.L)})
    print(f"[fullsize] {key}: loop_step, {len(depths)} rows, {n_fin} prefix keys", flush=True)
    ref_blocks = _fill_blocks(e, cfg, e.kv_core, blocks, keyset, S, seed=400)
    H0 = np.zeros((S, cfg.d), np.float32)
    H0[slots] = inputs.hidden_rows(len(slots), cfg.d, seed=62)
    e.H.copy_(torch.from_numpy(H0))
    fin_t = torch.tensor(fin, dtype=torch.int32, device="cuda")
    rows = e.rows(slots, pos, depths, n_fin, anc, C.c_void_p(fin_t.data_ptr()))
    e.loop_step(rows)
    assert e.sync_status() == 0
    Hg = e.H.cpu().numpy()
    kvg = e.kv_core.view(-1, S, 2, cfg.d)
    m = Model(cfg, {**w, "emb": w["emb"][:1], "pre": [], "coda": []})
    for i, k in enumerate(depths):
        blks = [ref_blocks[(k - 1) * cfg.L + l] for l in range(cfg.L)]
        h_ref, kvs = oracle_row_block(m, m.core, H0[slots[i]][None].astype(np.float64), pos[i], fin + anc[i], blks, cfg)
        err = rel_l2(Hg[slots[i]], h_ref[0])
        print(f"[fullsize] {key}: long prefix, row {i} depth {k} rel-L2 {err:.2e}", flush=True)
        assert err <= tol(cfg), (i, err)
        for l in (0, cfg.L - 1):
            got = as_f64(kvg[(k - 1) * cfg.L + l, slots[i]].cpu().numpy().view(np.uint16), cfg)
            assert rel_l2(got[0], kvs[l][0]) <= tol(cfg) and rel_l2(got[1], kvs[l][1]) <= tol(cfg), (i, l)
    e.close()
    del e
    gc.collect()
    torch.cuda.empty_cache()
