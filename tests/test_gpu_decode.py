"""End-to-end pipelined decoding on the GPU against the serial CPU reference, on the small
shapes (real head dimensions, small widths and vocabularies), through the C ABI.

Every committed position is checked by `decode_checks.check_stream`: logits at each traced
readout depth against the reference along the same stream, the readout distribution
against the reference processing of the GPU's own logits, the decision against the
reference sampler on the GPU's own distributions (exactly), and the reference's own
decision wherever it is not within the measured error of a boundary.  The modes cover the
LoopSpec page's single proposal, residual second proposal with and without the gate, the
non-residual ablation of Table 3, greedy and sampled readouts, plain full-depth decoding on
the same kernels, and the CopyLoop page's copy-suffix proposals screened at a shallow depth.
"""

from dataclasses import replace

import pytest

from oracle.model import Model
from synth import configs, inputs, weights
from tests.decode_checks import check_stream, run_gpu_decode

pytestmark = pytest.mark.gpu

CASES = {
    "tiny": ("tiny", {}),
    "tiny-sample": ("tiny-sample", {}),
    "mini-ouro": ("mini-ouro", {}),
    "mini-ouro-greedy": ("mini-ouro-greedy", {}),
    "mini-ouro-ungated": ("mini-ouro", {"gate": False}),
    "mini-ouro-nonresidual": ("mini-ouro", {"residual": False, "gate": False}),
    "mini-ouro-nonresidual-gated": ("mini-ouro", {"residual": False}),
    "mini-huginn": ("mini-huginn", {}),
    "mini-huginn-sample": ("mini-huginn-sample", {}),
    "mini-huginn-copy": ("mini-huginn-copy", {}),
    "mini-huginn-copy-tau": ("mini-huginn-copy", {"tau": 0.002}),
}


def _setup(key, over):
    wl = configs.get(key)
    cfg, dec = wl.model, replace(wl.decode, **over)
    w = weights.make_weights(cfg, seed=dec.seed_w)
    prompt = [int(t) for t in inputs.prompt(cfg.V, dec.prompt_len, seed=dec.seed_p, kind=dec.prompt_kind)]
    return cfg, dec, w, prompt


@pytest.mark.parametrize("case", list(CASES))
def test_decode_matches_reference(case):
    key, over = CASES[case]
    print(f"[decode] {case}", flush=True)
    cfg, dec, w, prompt = _setup(key, over)
    n_new = dec.new_tokens
    toks, recs, st = run_gpu_decode(cfg, dec, w, prompt, n_new)
    rep = check_stream(cfg, dec, Model(cfg, w), prompt, toks, recs)
    print(f"  {rep}; stats {st}", flush=True)
    assert st["gamma"] <= cfg.R / (dec.screen_depth if dec.copy else dec.d1) + 1e-9
    if dec.greedy:
        assert rep["greedy_checked"] >= n_new - 2
        assert rep["near_boundary"] <= 2, rep


@pytest.mark.parametrize("key", ["tiny", "mini-ouro", "mini-huginn"])
def test_plain_decoding_matches_reference(key):
    """Full-depth autoregressive decoding on the same kernels (proposals off)."""
    print(f"[decode-ar] {key}", flush=True)
    cfg, dec, w, prompt = _setup(key, {})
    n_new = dec.new_tokens
    toks, recs, st = run_gpu_decode(cfg, dec, w, prompt, n_new, mode="ar")
    rep = check_stream(cfg, dec, Model(cfg, w), prompt, toks, recs, mode="ar")
    print(f"  {rep}", flush=True)
    assert st["steps"] == (n_new - 1) * cfg.R


def test_branch_cap_does_not_change_tokens():
    cfg, dec, w, prompt = _setup("mini-ouro", {})
    n_new = 12
    t_full, _, st_full = run_gpu_decode(cfg, dec, w, prompt, n_new)
    t_cap, _, st_cap = run_gpu_decode(cfg, replace(dec, max_branches=1), w, prompt, n_new)
    assert t_full == t_cap
    assert st_cap["rows_max"] <= 1
