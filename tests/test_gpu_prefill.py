"""ls_prefill against the CPU reference.

The call runs P, every loop iteration 1..R of B and the coda layers at the readout depths
over whole chunks of prompt positions (LoopSpec page, section 2.1, eq. 1 applied to the
prompt; section 2.4: prelude, loop and coda caches indexed by depth).  The reference is the
float64 model processing the same prompt in one pass (`Seq.extend`); compared are H^(R) of
every position and every cache entry the call wrote, row by row (relative L2), at 1e-5 for
the fp32 model and 2e-2 for bf16 models, raised to twice the distance of a second reference
(the same model with float32-accumulated products) where R iterations carry rounding-level
differences further.  Chunks are ragged (not multiples of the 128-row product tiles or the
64-row attention blocks), split in two (the second chunk attends to the first through the
committed-prefix table), and slots are scattered.
"""

import ctypes
import gc

import numpy as np
import pytest
import torch

from looped_transformer_self_amd import _lib as L
from looped_transformer_self_amd.engine import Engine
from oracle import numerics
from oracle.model import Model
from synth import configs, inputs, weights
from tests.gpu_helpers import rel_l2, tol

pytestmark = pytest.mark.gpu


def _f64(a, cfg):
    return numerics.bf16_bits_to_f64(a.view(np.uint16)) if cfg.dtype == "bf16" else a.astype(np.float64)


def _gpu_prefill(cfg, w, prompt, chunks, mask, S, seed=3):
    """Run ls_prefill over the chunks; returns (slots, H rows [T0][d], cache arrays)."""
    T0 = len(prompt)
    slots = [int(s) for s in np.random.Generator(np.random.PCG64(seed)).permutation(S)[:T0]]
    e = Engine(cfg, w, slot_capacity=S, max_rows=16)
    try:
        fin = torch.zeros(S, dtype=torch.int32, device="cuda")
        fin[:T0] = torch.tensor(slots, dtype=torch.int32)
        c0 = 0
        for n in chunks:
            e.prefill(prompt[c0:c0 + n], slots[c0:c0 + n], c0, ctypes.c_void_p(fin.data_ptr()), mask)
            c0 += n
        assert c0 == T0
        st = e.sync_status()
        assert st == L.LS_OK, L.lib.ls_last_error()
        H = e.H.cpu().numpy()[slots].astype(np.float64)
        ent = (S, 2, cfg.d)
        kv = {"core": e.kv_core.cpu().numpy().reshape(cfg.R, cfg.L, *ent)}
        if cfg.L_pre:
            kv["pre"] = e.kv_pre.cpu().numpy().reshape(cfg.L_pre, *ent)
        if cfg.L_coda:
            kv["coda"] = e.kv_coda.cpu().numpy().reshape(len(cfg.readout_depths), cfg.L_coda, *ent)
    finally:
        e.close()
    return slots, H, kv


def _rows_close(got, ref, alt, base, what):
    """Per-row relative L2 of got against ref, bounded by max(base, 2 * the alternative
    reference's own distance from ref)."""
    worst = 0.0
    for i in range(ref.shape[0]):
        r = rel_l2(got[i], ref[i])
        bound = max(base, 2.0 * rel_l2(alt[i], ref[i])) if alt is not None else base
        assert r <= bound, f"{what} row {i}: rel {r:.3e} > {bound:.3e}"
        worst = max(worst, r)
    return worst


def _check_caches(cfg, kv, slots, seq, alt_seq, mask, depths_core):
    base = tol(cfg)
    T0 = len(slots)
    checked = 0

    def cmp(arr, key, what):
        nonlocal checked
        c = seq.caches[key]
        a = alt_seq.caches[key] if alt_seq is not None else None
        for half, (ref, al) in enumerate(((c.K[:T0], a.K[:T0] if a else None), (c.Vv[:T0], a.Vv[:T0] if a else None))):
            _rows_close(_f64(arr[slots, half, :], cfg), ref, al, base, f"{what} {'KV'[half]}")
        checked += 1

    for l in range(cfg.L_pre):
        cmp(kv["pre"][l], ("pre", 0, l), f"prelude layer {l}")
    for k in depths_core:
        for l in range(cfg.L):
            cmp(kv["core"][k - 1, l], ("core", k, l), f"depth {k} layer {l}")
    for j, r in enumerate(cfg.readout_depths):
        if not cfg.L_coda:
            break
        if mask >> j & 1:
            for l in range(cfg.L_coda):
                cmp(kv["coda"][j, l], ("coda", r, l), f"coda depth {r} layer {l}")
        else:
            assert not np.any(kv["coda"][j][:, slots]), f"coda caches of depth {r} written without its mask bit"
    return checked


SMALL = [configs.TINY, configs.MINI_OURO, configs.MINI_HUGINN]


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
@pytest.mark.parametrize("chunks", [(150,), (100, 50), (1,), (130, 1)], ids=lambda c: "+".join(map(str, c)))
def test_prefill_matches_reference(cfg, chunks):
    T0 = sum(chunks)
    print(f"[prefill] {cfg.name} chunks {chunks}", flush=True)
    w = weights.make_weights(cfg, seed=0)
    prompt = [int(t) for t in inputs.prompt(cfg.V, T0, seed=1)]
    full = (1 << len(cfg.readout_depths)) - 1
    mask = full if chunks != (130, 1) else 1 << (len(cfg.readout_depths) - 1)   # AR: R only
    slots, H, kv = _gpu_prefill(cfg, w, prompt, chunks, mask, S=T0 + 40)
    depths = tuple(r for j, r in enumerate(cfg.readout_depths) if mask >> j & 1)
    seqs = []
    for products in ("f64", "f32"):
        s = Model(cfg, w, products=products).new_seq()
        _, hid = s.extend(prompt, depths=depths, last_only=False, keep_hidden=True)
        seqs.append((s, hid))
    (seq, hid), (alt, hid_alt) = seqs
    worst = _rows_close(H, hid[cfg.R], hid_alt[cfg.R], tol(cfg), "H^(R)")
    n = _check_caches(cfg, kv, slots, seq, alt, mask, range(1, cfg.R + 1))
    print(f"[prefill] {cfg.name} {chunks}: H^(R) worst rel {worst:.2e}; {n} caches checked", flush=True)


def test_prefill_full_size_ouro():
    """Ouro-1.4B shape (d 2048, 16 x 128 heads, 24-layer block, F 5632, R 4), 48 positions:
    H^(R) and every loop cache against the reference."""
    wl = configs.get("C2")
    cfg = wl.model
    w = weights.make_weights(cfg, seed=wl.decode.seed_w)
    prompt = [int(t) for t in inputs.prompt(cfg.V, 48, seed=1)]
    slots, H, kv = _gpu_prefill(cfg, w, prompt, (48,), 1, S=64)
    print("[prefill] C2 shape: GPU done; reference passes", flush=True)
    seqs = []
    for products in ("f64", "f32"):
        s = Model(cfg, w, products=products).new_seq()
        _, hid = s.extend(prompt, depths=(cfg.R,), last_only=False, keep_hidden=True)
        seqs.append((s, hid))
        gc.collect()
    (seq, hid), (alt, hid_alt) = seqs
    worst = _rows_close(H, hid[cfg.R], hid_alt[cfg.R], tol(cfg), "H^(R)")
    _check_caches(cfg, kv, slots, seq, alt, 1, range(1, cfg.R + 1))
    print(f"[prefill] C2 shape: H^(R) worst rel {worst:.2e}", flush=True)


def test_prefill_full_size_huginn_depth_R():
    """Huginn-3.5B shape, 48 positions: H^(R) after all 32 loop iterations and the loop
    caches of every depth against the reference, bounded by the float32-products reference's
    own distance (32 iterations of a random-init block carry rounding-level differences to a
    few per cent)."""
    wl = configs.get("C4")
    cfg = wl.model
    w = weights.make_weights(cfg, seed=wl.decode.seed_w)
    prompt = [int(t) for t in inputs.prompt(cfg.V, 48, seed=1)]
    slots, H, kv = _gpu_prefill(cfg, w, prompt, (48,), 1 << (len(cfg.readout_depths) - 1), S=64)
    print("[prefill] C4 shape, depth R: GPU done; reference passes", flush=True)
    seqs = []
    for products in ("f64", "f32"):
        s = Model(cfg, w, products=products).new_seq()
        _, hid = s.extend(prompt, depths=(cfg.R,), last_only=False, keep_hidden=True)
        seqs.append((s, hid))
        gc.collect()
    (seq, hid), (alt, hid_alt) = seqs
    worst = _rows_close(H, hid[cfg.R], hid_alt[cfg.R], tol(cfg), "H^(R)")
    n = _check_caches(cfg, kv, slots, seq, alt, 1 << (len(cfg.readout_depths) - 1), range(1, cfg.R + 1))
    alt_d = max(rel_l2(hid_alt[cfg.R][i], hid[cfg.R][i]) for i in range(len(prompt)))
    print(f"[prefill] C4 shape: H^(R) worst rel {worst:.2e} (float32-products reference {alt_d:.2e}); "
          f"{n} caches checked", flush=True)


def test_prefill_full_size_huginn():
    """Huginn-3.5B shape (d 5280 = 41 x 128 + 32, 55 x 96 heads, F 17920, prelude 2, core 4),
    140 positions in chunks of 130 and 10: the prelude caches and the loop caches of depths
    1 and 2 (all their layers) against the reference, which stops at depth 2."""
    wl = configs.get("C4")
    cfg = wl.model
    w = weights.make_weights(cfg, seed=wl.decode.seed_w)
    prompt = [int(t) for t in inputs.prompt(cfg.V, 140, seed=1)]
    slots, H, kv = _gpu_prefill(cfg, w, prompt, (130, 10), 1 << (len(cfg.readout_depths) - 1), S=160)
    del H
    print("[prefill] C4 shape: GPU done; reference pass to depth 2", flush=True)
    m = Model(cfg, w)
    seq = m.new_seq()
    h = seq.prelude(prompt, 0)
    for k in (1, 2):
        h = seq.loop(h, k, 0)
    del m
    gc.collect()
    base = tol(cfg)
    for l in range(cfg.L_pre):
        for half, ref in enumerate((seq.caches[("pre", 0, l)].K, seq.caches[("pre", 0, l)].Vv)):
            _rows_close(_f64(kv["pre"][l][slots, half, :], cfg), ref[:140], None, base, f"prelude {l}")
    for k in (1, 2):
        for l in range(cfg.L):
            c = seq.caches[("core", k, l)]
            for half, ref in enumerate((c.K, c.Vv)):
                _rows_close(_f64(kv["core"][k - 1, l][slots, half, :], cfg), ref[:140], None, base,
                            f"depth {k} layer {l}")
    print("[prefill] C4 shape: prelude and depth 1-2 caches within tolerance", flush=True)


def test_prefill_rejects_bad_tokens_and_slots():
    """A token outside [0, V) or a slot outside [0, S) is reported in the error word, not
    turned into an out-of-bounds access; an undersized scratch is refused before launch."""
    cfg = configs.MINI_OURO
    w = weights.make_weights(cfg, seed=0)
    S = 64
    e = Engine(cfg, w, slot_capacity=S, max_rows=16)
    try:
        fin = torch.zeros(S, dtype=torch.int32, device="cuda")
        fp = ctypes.c_void_p(fin.data_ptr())
        e.prefill([1, 2, cfg.V + 5], [0, 1, 2], 0, fp, 1)
        assert e.sync_status() == L.LS_ERR_INVALID
        e2 = Engine(cfg, w, slot_capacity=S, max_rows=16)
        try:
            e2.prefill([1, 2, 3], [0, S + 3, 2], 0, fp, 1)
            assert e2.sync_status() == L.LS_ERR_INVALID
            st = L.lib.ls_prefill(e2.h, ctypes.c_void_p(fin.data_ptr()), ctypes.c_void_p(fin.data_ptr()), 4, fp, 0, 1,
                                  ctypes.c_void_p(e2.H.data_ptr()), ctypes.byref(e2.kv),
                                  ctypes.c_void_p(e2.pws.data_ptr()), 16, e2.stream_ptr())
            assert st == L.LS_ERR_CAPACITY
        finally:
            e2.close()
    finally:
        e.close()
