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


COPY_BYTES = 1 << 30            # size of the plain device copy that calibrates the HBM byte counters
LOOP_KERNEL = "void ls::k_mega<"  # profile name prefix of the loop-block launches (ls_loop_step)
TRAFFIC_SOURCES = ["mega.hip", "common.h", "kernels.h", "loopspec_abi.hip"]


def _kernel_source_sha():
    """sha256 over the sources that define the loop-block kernel and its launch."""
    import hashlib
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, "looped_transformer_self_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _measured_traffic(workload):
    """HBM bytes per ls_loop_step launch from the committed counter summary of this workload,
    if it was taken on the current kernel sources; else None."""
    import glob
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*_traffic.md"))):
        with open(path) as f:
            for line in f:
                line = line.strip()
                if line.startswith('{"kernel": "k_mega"'):
                    rec = json.loads(line)
                    if rec.get("workload") == workload and rec.get("source_sha256") == _kernel_source_sha():
                        return rec
    return None


def copy_calibration():
    """One plain device-to-device copy of COPY_BYTES, the reference for the byte counters."""
    import torch
    a = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES}), flush=True)


def _db(d):
    """The rocpd SQLite database rocprofv3 wrote under directory d."""
    import glob
    import sqlite3
    hits = sorted(glob.glob(os.path.join(d, "**", "*_results.db"), recursive=True))
    if not hits:
        raise SystemExit(f"no rocprofv3 database under {d}")
    return sqlite3.connect(hits[0])


def _counter_per_dispatch(d, counter, prefix):
    rows = _db(d).execute("select dispatch_id, value from counters_collection where counter_name = ? and "
                          "substr(kernel_name, 1, ?) = ? order by dispatch_id", (counter, len(prefix), prefix))
    return [float(v) for _, v in rows]


def _profile_commands(a):
    """The command sequence that produces the databases this summary reads (directory names
    taken from the arguments)."""
    b = "python3 -u bench.py --steps 1 --warmup 0 --no-cpu-baseline"
    cmds = [f"rocprofv3 --kernel-trace --stats -d {a.trace_dir} -o c2 -- {b} > {a.bench_log} 2>&1",
            f"rocprofv3 --pmc FETCH_SIZE -d {a.fetch_dir} -o c2 -- {b}",
            f"rocprofv3 --pmc WRITE_SIZE -d {a.write_dir} -o c2 -- {b}"]
    if a.mfma_dir:
        cmds.append(f"rocprofv3 --pmc MfmaUtil MfmaFlopsBF16 -d {a.mfma_dir} -o c2 -- {b}")
    cmds += [f"rocprofv3 --pmc FETCH_SIZE -d {a.copy_fetch_dir} -o copy -- python3 -u bench.py --copy-calibration",
             f"rocprofv3 --pmc WRITE_SIZE -d {a.copy_write_dir} -o copy -- python3 -u bench.py --copy-calibration"]
    summ = (f"python3 bench.py --pmc-summary --workload {a.workload} --bench-log {a.bench_log} "
            f"--trace-dir {a.trace_dir} --fetch-dir {a.fetch_dir} --write-dir {a.write_dir} "
            f"--copy-fetch-dir {a.copy_fetch_dir} --copy-write-dir {a.copy_write_dir}")
    if a.mfma_dir:
        summ += f" --mfma-dir {a.mfma_dir}"
    return cmds + [summ + (f" --out {a.out}" if a.out else "")]


def pmc_summary(a):
    """Digest of the rocprofv3 runs of one benchmark command: the loop-block kernel's
    per-launch duration (kernel trace) and HBM bytes (FETCH_SIZE / WRITE_SIZE runs, scaled
    by the same counters on a plain copy of known size), over the launches of the timed
    region.  Prints a markdown summary with one machine-readable JSON line."""
    import re
    log = open(a.bench_log).read()
    m = re.search(r"ls_loop_step launches: (\d+) before the timed region, (\d+) in it", log)
    nb, nt = int(m.group(1)), int(m.group(2))
    alg = float(re.search(r"algorithmic bytes per ls_loop_step launch: ([0-9.]+)", log).group(1))
    ev_us = float(re.search(r"event-timed us per ls_loop_step launch: ([0-9.]+)", log).group(1))
    bench_line = json.loads([l for l in log.splitlines() if l.startswith('{"metric"')][-1])
    db = _db(a.trace_dir)
    dur = [(e - b) / 1e3 for b, e in db.execute(
        "select start, end from kernels where substr(name, 1, ?) = ? order by dispatch_id",
        (len(LOOP_KERNEL), LOOP_KERNEL))]
    st = [avg for name, avg in db.execute("select name, average from top_kernels") if name.startswith(LOOP_KERNEL)]
    fe = _counter_per_dispatch(a.fetch_dir, "FETCH_SIZE", LOOP_KERNEL)
    wr = _counter_per_dispatch(a.write_dir, "WRITE_SIZE", LOOP_KERNEL)
    for name, v in (("kernel trace", dur), ("FETCH_SIZE run", fe), ("WRITE_SIZE run", wr)):
        if len(v) != nb + nt:
            raise SystemExit(f"{name}: {len(v)} loop-block launches, the bench log says {nb} + {nt}")
    cf = max(_counter_per_dispatch(a.copy_fetch_dir, "FETCH_SIZE", "__amd_rocclr_copyBuffer"))
    cw = max(_counter_per_dispatch(a.copy_write_dir, "WRITE_SIZE", "__amd_rocclr_copyBuffer"))
    kf, kw = COPY_BYTES / (cf * 1024), COPY_BYTES / (cw * 1024)
    sl = slice(nb, nb + nt)
    mean = lambda v: sum(v) / len(v)
    f_b, w_b = mean(fe[sl]) * 1024 * kf, mean(wr[sl]) * 1024 * kw
    rec = {"kernel": "k_mega", "workload": a.workload, "source_sha256": _kernel_source_sha(),
           "launches": nt, "fetch_bytes_per_launch": round(f_b), "write_bytes_per_launch": round(w_b),
           "traffic_bytes_per_launch": round(f_b + w_b), "algorithmic_bytes_per_launch": round(alg),
           "copy_scale_fetch": round(kf, 4), "copy_scale_write": round(kw, 4),
           "trace_us_per_launch": round(mean(dur[sl]), 2), "event_us_per_launch": ev_us}
    out = [f"# k_mega (ls_loop_step) on workload {a.workload}: duration and HBM traffic per launch", "",
           "Commands (repo root, MI355X, one GPU), in this order:", ""]
    cmds = a.commands or _profile_commands(a)
    out += [f"    {c}" for c in cmds]
    out += ["", f"Timed region: launches {nb}..{nb + nt - 1} of the loop-block kernel (the {nb} before it are "
            "the untimed prefill/warmup); the decode is deterministic, so every run makes the same launches.", "",
            "| quantity | value |", "|---|---|",
            f"| launches in the timed region | {nt} |",
            f"| kernel-trace mean duration, timed launches (us) | {mean(dur[sl]):.1f} |",
            f"| kernel-trace mean duration, all {nb + nt} launches (us) | {mean(dur):.1f} |",
            f"| rocprofv3 top_kernels average, all launches (us) | {st[0] if st else float('nan'):.1f} |",
            f"| HIP-event mean duration in bench.py, timed launches (us) | {ev_us:.1f} |",
            f"| copy calibration: FETCH_SIZE / WRITE_SIZE of a {COPY_BYTES >> 20} MiB copy (KiB) | {cf:.0f} / {cw:.0f} |",
            f"| scale to bytes (fetch, write) | {kf:.4f}, {kw:.4f} |",
            f"| HBM bytes fetched per launch | {f_b / 1e9:.4f} GB |",
            f"| HBM bytes written per launch | {w_b / 1e9:.4f} GB |",
            f"| algorithmic bytes per launch | {alg / 1e9:.4f} GB |",
            f"| traffic / algorithmic | {(f_b + w_b) / alg:.3f} |",
            f"| bench line | {bench_line['value']} {bench_line['unit']}, frac {bench_line['roofline']['frac']} |",
            "", "All kernels of the kernel-trace run (rocprofv3 top_kernels; prefill and decode):", "",
            "| kernel | calls | total us | avg us | % |", "|---|---|---|---|---|"]
    if a.mfma_dir:
        # matrix-core use of the same launches: MfmaUtil (busy cycles of the MFMA units, % of
        # all SIMDs' cycles) and MfmaFlopsBF16 (512 flops per bf16 MFMA op counted), both
        # rocprofv3 derived counters; issued flops include the zero rows of tiles with M < 16
        mu = _counter_per_dispatch(a.mfma_dir, "MfmaUtil", LOOP_KERNEL)
        mf = _counter_per_dispatch(a.mfma_dir, "MfmaFlopsBF16", LOOP_KERNEL)
        for name, v in (("MfmaUtil run", mu), ("MfmaFlopsBF16 run", mf)):
            if len(v) != nb + nt:
                raise SystemExit(f"{name}: {len(v)} loop-block launches, the bench log says {nb} + {nt}")
        util, flops = mean(mu[sl]), mean(mf[sl])
        tflops = flops / (mean(dur[sl]) * 1e-6) / 1e12
        rec.update({"mfma_util_percent": round(util, 3), "mfma_flops_per_launch": round(flops),
                    "mfma_tflops": round(tflops, 2)})
        at = next(i for i, x in enumerate(out) if x.startswith("| bench line |"))
        out[at:at] = [f"| MFMA busy (MfmaUtil), timed launches | {util:.2f} % |",
                      f"| MFMA flops issued per launch (MfmaFlopsBF16) | {flops / 1e12:.3f} T |",
                      f"| MFMA rate issued / bf16 dense peak | {tflops:.1f} of 2500 TFLOP/s ({tflops / 2500:.4f}) |"]
    for name, calls, tot, avg, pct in db.execute(
            "select name, total_calls, total_duration, average, percentage from top_kernels"):
        out.append(f"| `{name[:90]}` | {calls} | {tot:.0f} | {avg:.1f} | {pct:.2f} |")
    out += ["", "Machine-readable (read by bench.py while the kernel sources are unchanged):", "",
            json.dumps(rec), ""]
    text = "\n".join(out)
    if a.out:
        with open(a.out, "w") as f:
            f.write(text)
    print(text)


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
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run one plain device copy of 1 GiB (byte-counter calibration)")
    ap.add_argument("--pmc-summary", action="store_true",
                    help="summarise rocprofv3 outputs of a benchmark run (no GPU)")
    ap.add_argument("--bench-log")
    ap.add_argument("--trace-dir")
    ap.add_argument("--fetch-dir")
    ap.add_argument("--write-dir")
    ap.add_argument("--copy-fetch-dir")
    ap.add_argument("--copy-write-dir")
    ap.add_argument("--mfma-dir", help="rocprofv3 --pmc MfmaUtil MfmaFlopsBF16 run of the same command")
    ap.add_argument("--out")
    ap.add_argument("--commands", nargs="*", default=[])
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(args)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; multi-GPU runs are not supported "
                                   f"(asked for --gpus {args.gpus})"}))
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

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
    n_before = e.n_loop_calls
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
    print(f"[bench] ls_loop_step launches: {n_before} before the timed region, {n_calls} in it", file=sys.stderr)
    print(f"[bench] algorithmic bytes per ls_loop_step launch: {by / n_calls:.1f}", file=sys.stderr)
    print(f"[bench] event-timed us per ls_loop_step launch: {t_ms / n_calls * 1e3:.2f}", file=sys.stderr, flush=True)
    traffic = _measured_traffic(wl.key)
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
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic["traffic_bytes_per_launch"] if traffic else None,
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                     "bytes_per_call": round(by / n_calls), "us_per_call": round(t_ms / n_calls * 1e3, 2),
                     "launches": n_calls},
        "decode_stats": {k: (round(v, 4) if isinstance(v, float) else v) for k, v in st.items()},
    }
    if traffic and "mfma_util_percent" in traffic:
        # matrix-core use of the same kernel from the committed counter summary
        out["roofline"]["mfma_util_percent"] = traffic["mfma_util_percent"]
        out["roofline"]["mfma_tflops_issued"] = traffic["mfma_tflops"]
    if not args.no_cpu_baseline:
        print("[bench] CPU reference baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(cfg, dec, w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
