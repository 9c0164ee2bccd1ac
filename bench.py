"""Benchmark: committed tokens/s at batch 1 of pipelined self-speculative decoding on the
Ouro-1.4B-shaped looped decoder (bf16, vocab 49152, d 2048, 16 heads, shared 24-layer block
applied R = 4 times, SwiGLU 5632; prompt 512 random tokens, 256 new tokens, T = 1.0, top-p
0.9, first proposal at depth 2, residual second proposal at depth 3, <= 8 active branches),
random-init weights and synthetic prompt.

One step = one complete decode of the 256 new tokens from the prefilled state (prefill is
excluded from timing, as on the LoopSpec page, section 3.1): every pipeline step of it runs
the prelude of new branches, ls_loop_step over all active rows, ls_readout at the readout
depths and ls_verify, plus the host scheduler.  `value` counts the tokens committed inside
the timed decode (the first new token comes from the prefill readout).

Also reported: the roofline of ls_loop_step (algorithmic HBM bytes per call / its
event-timed duration, against 8 TB/s), and the CPU reference (plain NumPy full-depth
autoregressive decoding) timed on a bounded sample on the host cores.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def cpu_baseline(cfg, dec, w, prompt_len=16, n_tok=3):
    """Plain full-depth AR decoding by the CPU reference on a bounded sample: a 16-token
    prompt (the workload's first 16 prompt tokens) and 3 decoded tokens; decode-only rate."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import philox, readout, sampler
    from oracle.model import Model
    from synth import inputs

    prompt = list(inputs.prompt(cfg.V, dec.prompt_len, seed=dec.seed_p))[:prompt_len]
    m = Model(cfg, w)
    seq = m.new_seq()
    lg = seq.extend(prompt, depths=(cfg.R,))[cfg.R]
    t0 = time.perf_counter()
    pos = len(prompt)
    for i in range(n_tok):
        P = sampler.fixed(readout.distribution(lg, dec.greedy, dec.T, dec.top_p))
        x = sampler.sample(P, philox.uniform(dec.seed_s, pos, philox.P_AR))
        pos += 1
        lg = seq.extend([x], depths=(cfg.R,))[cfg.R]
    dt = time.perf_counter() - t0
    threads = max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
    return {"value": n_tok / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"float64 NumPy full-depth AR decode of {n_tok} tokens after a {prompt_len}-token prefix "
                      f"of the workload prompt (prefill untimed), same weights",
            "cpu": _cpu_model()}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class _Progress:
    """Prints '[bench] <what> done/total' to stderr at most every `every` seconds."""

    def __init__(self, what, every=20.0):
        self.what, self.every, self.last = what, every, time.perf_counter()

    def __call__(self, done, total):
        now = time.perf_counter()
        if now - self.last >= self.every or done >= total:
            self.last = now
            print(f"[bench] {self.what} {done}/{total}", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="C2")
    ap.add_argument("--mode", default="spec", choices=["spec", "ar"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; multi-GPU runs are not supported "
                                   f"(asked for --gpus {args.gpus})"}))
        sys.exit(2)

    import numpy as np
    import torch

    from looped_transformer_self_amd.decoder import Decoder
    from looped_transformer_self_amd.engine import Engine
    from synth import configs, inputs, weights

    wl = configs.get(args.workload)
    cfg, dec = wl.model, wl.decode
    n_new = dec.new_tokens
    print(f"[bench] workload {wl.key}: generating weights", file=sys.stderr, flush=True)
    w = weights.make_weights(cfg, seed=dec.seed_w)
    prompt = inputs.prompt(cfg.V, dec.prompt_len, seed=dec.seed_p, kind=dec.prompt_kind)
    S = dec.prompt_len + n_new + 4 * dec.max_branches + 64
    e = Engine(cfg, w, slot_capacity=S, max_rows=max(16, dec.max_branches), max_keys=S, max_jobs=64,
               prob_rows=4 * dec.max_branches + 16)
    d = Decoder(e, dec, args.mode)
    print("[bench] prefill", file=sys.stderr, flush=True)
    d.prefill(prompt, progress=_Progress("prefill"))
    snap = d.snapshot()
    torch.cuda.synchronize()
    for i in range(args.warmup):
        d.restore(snap)
        d.decode(n_new, progress=_Progress(f"warmup {i}"))
        print(f"[bench] warmup {i} done", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    e.prof = []
    stats = []
    t0 = time.perf_counter()
    for i in range(args.steps):
        d.restore(snap)
        toks = d.decode(n_new, progress=_Progress(f"step {i}", every=60.0))
        stats.append(d.stats())
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    committed = args.steps * (n_new - 1)
    value = committed / dt
    # ls_loop_step roofline over the timed region
    t_ms = sum(b.elapsed_time(en) for b, en, _ in e.prof)
    by = sum(e.loop_step_bytes(h) for _, _, h in e.prof)
    n_calls = len(e.prof)
    e.prof = None
    achieved = by / (t_ms * 1e-3) / 1e9 if t_ms > 0 else 0.0
    print(f"[bench] {n_calls} ls_loop_step calls, {by / n_calls / 1e9:.3f} GB/call, "
          f"{t_ms / n_calls * 1e3:.1f} us/call", file=sys.stderr, flush=True)
    st = stats[-1]
    out = {
        "metric": "committed tokens/s at batch 1",
        "value": round(value, 3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dt / args.steps * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded random-init weights, uniform random prompt)",
        "config": {"workload": f"{wl.key}: {wl.description}", "prompt_len": dec.prompt_len, "new_tokens": n_new,
                   "mode": args.mode, "batch": 1},
        "roofline": {"kernel": "ls_loop_step (one call: all layers of the shared block, all active rows)",
                     "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "bytes_per_call": round(by / n_calls), "us_per_call": round(t_ms / n_calls * 1e3, 2)},
        "decode_stats": {k: (round(v, 4) if isinstance(v, float) else v) for k, v in st.items()},
    }
    if not args.no_cpu_baseline:
        print("[bench] CPU reference baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(cfg, dec, w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
