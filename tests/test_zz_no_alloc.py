"""ls_loop_step_static, the loop step for callers that cannot allocate device memory: the same
kernels as ls_loop_step on the library's static per-GPU scratch instead of a bound workspace.
Its results must equal ls_loop_step's bit for bit (every reduction in the kernels has a fixed
order), on two calls in a row, the second with fewer rows and keys; sizes beyond the static
scratch are rejected before anything is enqueued."""

import ctypes as C

import numpy as np
import pytest
import torch

from synth import configs, inputs, weights
from tests.gpu_helpers import branch_rows, kv_values, to_dev

pytestmark = pytest.mark.gpu


def _static(e, rows, err):
    from looped_transformer_self_amd import _lib as L
    return L.lib.ls_loop_step_static(e.h, C.byref(rows.s), C.c_void_p(e.H.data_ptr()), C.byref(e.kv),
                                     C.c_void_p(err.data_ptr()) if err is not None else C.c_void_p(0), e.stream_ptr())


@pytest.mark.parametrize("cfg", [configs.MINI_OURO, configs.MINI_HUGINN], ids=lambda c: c.name)
def test_static_loop_step_equals_loop_step(cfg):
    from looped_transformer_self_amd import _lib as L
    from looped_transformer_self_amd.engine import Engine
    print(f"[static] {cfg.name}", flush=True)
    S = 512
    w = weights.make_weights(cfg, seed=0)
    e = Engine(cfg, w, slot_capacity=S, max_rows=32, max_keys=S, max_jobs=16, prob_rows=16)
    e.kv_core.copy_(to_dev(kv_values(cfg, cfg.R * cfg.L, S, seed=91)).reshape(-1))
    H0 = torch.from_numpy(inputs.hidden_rows(S, cfg.d, seed=92)).cuda()
    KV0 = e.kv_core.clone()
    rng = np.random.Generator(np.random.PCG64(93))
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    for M, n_fin in ((20, 300), (5, 40)):             # the second call is smaller
        fin, slots, anc, pos, depth = branch_rows(M, n_fin, lambda i: 1 + (i * 3) % cfg.R, rng, S)
        fin_t = torch.zeros(S, dtype=torch.int32, device="cuda")
        fin_t[:n_fin] = torch.tensor(fin, dtype=torch.int32, device="cuda")
        rows = e.rows(slots, pos, depth, n_fin, anc, C.c_void_p(fin_t.data_ptr()))
        e.H.copy_(H0)
        e.kv_core.copy_(KV0)
        e.loop_step(rows)
        assert e.sync_status() == L.LS_OK
        want_h, want_kv = e.H.clone(), e.kv_core.clone()
        e.H.copy_(H0)
        e.kv_core.copy_(KV0)
        err.zero_()
        L.check(_static(e, rows, err), "ls_loop_step_static")
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        assert torch.equal(e.H.view(torch.int32), want_h.view(torch.int32)), M
        assert torch.equal(e.kv_core, want_kv), M
        # without an error word the call works the same
        e.H.copy_(H0)
        e.kv_core.copy_(KV0)
        L.check(_static(e, rows, None), "ls_loop_step_static")
        torch.cuda.synchronize()
        assert torch.equal(e.H.view(torch.int32), want_h.view(torch.int32)), M
    e.close()


def test_static_loop_step_rejects_oversized_calls():
    """Calls whose buffers exceed the static scratch (here the attention partials of
    LS_MAX_ROWS rows over 10000 prefix keys), more rows than LS_MAX_ROWS, or more keys than
    the kernels index come back as LS_ERR_CAPACITY before any device work."""
    from looped_transformer_self_amd import _lib as L
    from looped_transformer_self_amd.engine import Engine
    cfg = configs.MINI_OURO
    w = weights.make_weights(cfg, seed=0)
    e = Engine(cfg, w, slot_capacity=64, max_rows=8, max_keys=64, max_jobs=4, prob_rows=4)
    fin_t = torch.zeros(64, dtype=torch.int32, device="cuda")
    rows = e.rows([1], [0], [1], 0, [[]], C.c_void_p(fin_t.data_ptr()))
    rows.s.n = L.LS_MAX_ROWS
    rows.s.n_fin = 10_000
    st = _static(e, rows, None)
    assert st == L.LS_ERR_CAPACITY and b"static scratch" in L.lib.ls_last_error()
    rows.s.n = L.LS_MAX_ROWS + 1
    rows.s.n_fin = 0
    assert _static(e, rows, None) == L.LS_ERR_CAPACITY
    rows.s.n = 1
    rows.s.n_fin = (1 << 30) + 1
    assert _static(e, rows, None) == L.LS_ERR_CAPACITY
    e.close()
