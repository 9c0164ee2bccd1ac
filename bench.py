"""Benchmark: committed tokens/s at batch 1 of pipelined self-speculative decoding.

Default workload: the Huginn/Raven-3.5B-shaped looped decoder (bf16, vocabulary 65536,
d 5280, 55 heads of 96, prelude 2 layers, shared core block of 4 layers applied R = 32 times,
coda 2 layers recomputed per readout, SwiGLU 17920), random-init weights, a 2048-token
synthetic prompt, 512 new tokens, greedy, proposals at depths 8 and 16, <= 16 active
branches: the largest configuration of the workload list that fits one GPU.  --workload
selects the others (C1-C5).

One step = one slice of 32 committed tokens of the workload's decode (prefill is excluded
from timing, as on the LoopSpec page, section 3.1).  Steps continue the same decode; when it
has committed all new tokens the next step restarts it from the prefilled state.  The timed
region starts a fresh decode, so K steps cover the first 32*K tokens (wrapping every
n_new - 1 decode-committed tokens).  Every pipeline step runs the prelude of new branches,
ls_loop_step over all active rows, ls_readout at the readout depths and ls_verify, plus the
host scheduler.  `value` counts the tokens committed inside the timed region.

Also reported: the same kernels in plain full-depth mode (proposals off) over the first
slices, and the speed-up over it; the roofline of ls_loop_step (algorithmic HBM bytes per
call / its event-timed duration, against 8 TB/s); and the CPU reference (plain NumPy
full-depth autoregressive decoding) timed on a bounded sample on the host cores.
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
    prompt (the workload's first 16 prompt tokens) and 3 decoded tokens; decode-only rate.
    The workload's own context is cut because the float64 prefill of a 2048-token prompt
    through the Huginn shape alone is ~220 TFLOP; at batch 1 a decoded token's cost is its
    weight products (attention over 2048 keys adds ~5 % to them)."""
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
                      f"of the workload prompt (prefill untimed; the workload's {dec.prompt_len}-token context "
                      f"is cut to bound the float64 prefill), same weights",
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


def prefill_report(cfg, dec, mode, seconds):
    """Prefill (untimed in the decode metric, LoopSpec page section 3.1): wall time of
    Decoder.prefill for the workload prompt (ls_prefill chunks plus the last position's
    readout), and the rate of its matrix products against the dense bf16 matrix-core peak.
    Matrix flops: 2 * positions * (layer weights of P, of R loop iterations of B and of the
    coda at every readout depth whose caches are filled) plus the causal attention products
    (4 * d per (query, key) pair per layer)."""
    T0, d, F = dec.prompt_len, cfg.d, cfg.F
    per_layer = 4 * d * d + 3 * F * d
    n_coda = len(cfg.readout_depths) if mode == "spec" else 1
    layers = cfg.L_pre + cfg.R * cfg.L + (n_coda * cfg.L_coda if cfg.L_coda else 0)
    flops = 2.0 * T0 * per_layer * layers + 4.0 * d * (T0 * (T0 + 1) / 2) * layers
    peak = 2500.0 if cfg.dtype == "bf16" else 157.3
    tf = flops / seconds / 1e12
    return {"tokens": T0, "seconds": round(seconds, 3), "tokens_per_s": round(T0 / seconds, 1),
            "matrix_tflops": round(tf, 1), "peak_tflops": peak, "frac": round(tf / peak, 4),
            "note": "ls_prefill: every layer of every depth as matrix products over 2048-position chunks"}


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
    w = a.workload.lower()
    b = f"python3 -u bench.py --workload {a.workload} --steps 2 --warmup 0 --no-cpu-baseline --no-ar"
    cmds = [f"rocprofv3 --kernel-trace --stats -d {a.trace_dir} -o {w} -- {b} > {a.bench_log} 2>&1",
            f"rocprofv3 --pmc FETCH_SIZE -d {a.fetch_dir} -o {w} -- {b}",
            f"rocprofv3 --pmc WRITE_SIZE -d {a.write_dir} -o {w} -- {b}"]
    if a.mfma_dir:
        cmds.append(f"rocprofv3 --pmc MfmaUtil MfmaFlopsBF16 -d {a.mfma_dir} -o {w} -- {b}")
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


def microbench(workload, Ms=(1, 2, 3, 4, 8, 16, 128), reps=10):
    """ls_loop_step at fixed row counts M on the workload's model shape: rows at loop depths
    spread over 1..R, each attending to a finished prefix of the workload's full context
    (prompt + new tokens), inputs resident in HBM (seeded synthetic hidden rows and KV
    entries).  Per M: event-timed microseconds per call, algorithmic bytes per call, GB/s and
    the fraction of 8 TB/s.  Also two streaming-read references over a 4 GiB buffer:
    ls_measure_stream_read (the loads ls_loop_step's producer waves issue, with no consumers:
    the achievable rate of that load pattern on this device) and PyTorch's sum (reads only, a
    plain library kernel)."""
    import ctypes

    import torch

    from looped_transformer_self_amd.engine import Engine
    from synth import configs, weights

    wl = configs.get(workload)
    cfg, dec = wl.model, wl.decode
    n_fin = dec.prompt_len + dec.new_tokens
    Mmax = max(Ms)
    S = n_fin + Mmax + 8
    w = weights.make_weights(cfg, seed=dec.seed_w)
    e = Engine(cfg, w, slot_capacity=S, max_rows=Mmax, max_keys=S, max_jobs=4, prob_rows=4)
    g = torch.Generator(device="cuda").manual_seed(7)
    kv = e.kv_core.view(torch.bfloat16) if cfg.dtype == "bf16" else e.kv_core
    for i in range(0, kv.numel(), 1 << 28):
        n = min(1 << 28, kv.numel() - i)
        kv[i:i + n] = torch.randn(n, generator=g, device="cuda", dtype=torch.float32).to(kv.dtype)
    e.H.copy_(torch.randn(e.H.shape, generator=g, device="cuda"))
    fin = torch.arange(S, dtype=torch.int32, device="cuda")
    fin_ptr = ctypes.c_void_p(fin.data_ptr())
    res = []
    for M in Ms:
        if M > Mmax:
            continue
        slots = list(range(n_fin, n_fin + M))
        depth = [1 + (cfg.R - 1 - (i * cfg.R) // M) % cfg.R for i in range(M)]
        rows = e.rows(slots, [n_fin] * M, depth, n_fin, [[]] * M, fin_ptr)
        for _ in range(2):
            e.loop_step(rows)
        torch.cuda.synchronize()
        b, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b.record()
        for _ in range(reps):
            e.loop_step(rows)
        en.record()
        torch.cuda.synchronize()
        assert e.sync_status() == 0
        us = b.elapsed_time(en) / reps * 1e3
        by = e.loop_step_bytes(rows.host)
        res.append({"M": M, "distinct_depths": len(set(depth)), "us": round(us, 1), "bytes": by,
                    "GB_s": round(by / us / 1e3, 1), "frac": round(by / us / 1e3 / HBM_PEAK_GBS, 4)})
        print(f"[microbench] {wl.key} M={M}: {us:.1f} us, {by / 1e9:.3f} GB, {by / us / 1e3:.0f} GB/s", file=sys.stderr,
              flush=True)
    e.close()
    from looped_transformer_self_amd import _lib as L
    x = torch.empty(1 << 31, dtype=torch.bfloat16, device="cuda").normal_(generator=g)
    n_wg = torch.cuda.get_device_properties(0).multi_processor_count
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def stream_read():
        L.check(L.lib.ls_measure_stream_read(ctypes.c_void_p(x.data_ptr()), x.numel() * 2, n_wg, stream),
                "ls_measure_stream_read")
    for _ in range(2):
        stream_read()
    torch.cuda.synchronize()
    b, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    b.record()
    for _ in range(reps):
        stream_read()
    en.record()
    torch.cuda.synchronize()
    slab_gbs = x.numel() * 2 / (b.elapsed_time(en) / reps * 1e-3) / 1e9
    for _ in range(2):
        x.sum(dtype=torch.float32)
    torch.cuda.synchronize()
    b, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    b.record()
    for _ in range(reps):
        x.sum(dtype=torch.float32)
    en.record()
    torch.cuda.synchronize()
    read_gbs = x.numel() * 2 / (b.elapsed_time(en) / reps * 1e-3) / 1e9
    out = {"workload": f"{wl.key}: {wl.description}", "prefix_keys": n_fin, "loop_step": res,
           "streaming_read_GB_s": round(slab_gbs, 1),
           "streaming_read_note": "ls_measure_stream_read over 4 GiB: the producer waves' load pattern, no consumers",
           "torch_sum_GB_s": round(read_gbs, 1)}
    print(json.dumps(out), flush=True)


def phase_stamps(workload, Ms=(1, 4, 7)):
    """Per-phase timeline of one ls_loop_step launch at fixed row counts M (rows at distinct
    depths, the workload's full context, synthetic hidden rows and KV as in the
    microbenchmark): ls_debug_trace's wall-clock stamps (100 MHz) of phase begin and end per
    workgroup, for the first four layers, as medians (and the maximum end) over workgroups in
    microseconds from the launch's first stamp.  Prints a markdown table."""
    import ctypes

    import numpy as np
    import torch

    from looped_transformer_self_amd import _lib as L
    from looped_transformer_self_amd.engine import Engine
    from synth import configs, weights

    wl = configs.get(workload)
    cfg, dec = wl.model, wl.decode
    n_fin = dec.prompt_len + dec.new_tokens
    S = n_fin + max(Ms) + 8
    w = weights.make_weights(cfg, seed=dec.seed_w)
    e = Engine(cfg, w, slot_capacity=S, max_rows=max(Ms), max_keys=S, max_jobs=4, prob_rows=4)
    g = torch.Generator(device="cuda").manual_seed(7)
    kv = e.kv_core.view(torch.bfloat16) if cfg.dtype == "bf16" else e.kv_core
    for i in range(0, kv.numel(), 1 << 28):
        n = min(1 << 28, kv.numel() - i)
        kv[i:i + n] = torch.randn(n, generator=g, device="cuda", dtype=torch.float32).to(kv.dtype)
    e.H.copy_(torch.randn(e.H.shape, generator=g, device="cuda"))
    fin = torch.arange(S, dtype=torch.int32, device="cuda")
    fin_ptr = ctypes.c_void_p(fin.data_ptr())
    buf = torch.zeros(1024 * (4 * 8 * 8 + 32), dtype=torch.int64, device="cuda")
    names = ["QKV", "attention", "O", "GU", "DOWN"]
    out = [f"# ls_loop_step phase timeline on workload {wl.key} ({wl.description}), {n_fin} prefix keys", "",
           f"Command (repo root, MI355X, one GPU): python3 bench.py --phase-stamps --workload {wl.key}", "",
           "Microseconds from the launch's first stamp; each cell is begin / median end / latest end of the "
           "phase over workgroups (ls_debug_trace wall-clock stamps).", ""]
    for M in Ms:
        slots = list(range(n_fin, n_fin + M))
        depth = [1 + (cfg.R - 1 - (i * cfg.R) // M) % cfg.R for i in range(M)]
        rows = e.rows(slots, [n_fin] * M, depth, n_fin, [[]] * M, fin_ptr)
        for _ in range(3):
            e.loop_step(rows)
        torch.cuda.synchronize()
        grid = ctypes.c_int()
        buf.zero_()
        L.check(L.lib.ls_debug_trace(e.h, ctypes.c_void_p(buf.data_ptr()), ctypes.byref(grid)), "ls_debug_trace")
        b, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b.record()
        e.loop_step(rows)
        en.record()
        torch.cuda.synchronize()
        L.check(L.lib.ls_debug_trace(e.h, None, ctypes.byref(grid)), "ls_debug_trace")
        assert e.sync_status() == 0
        G = grid.value
        st = buf[:G * 256].cpu().numpy().reshape(G, 4, 8, 8).astype(np.float64)
        us = (st - st[st > 0].min()) / 100.0
        out += [f"## M = {M} (distinct depths {len(set(depth))}), grid {G}, event-timed "
                f"{b.elapsed_time(en) * 1e3:.0f} us", "", "| layer | " + " | ".join(names) + " |",
                "|---|" + "---|" * len(names)]
        for l in range(min(4, cfg.L)):
            cells = []
            for ph in range(1, 6):
                ok = st[:, l, ph, 1] > 0
                cells.append(f"{np.median(us[ok, l, ph, 0]):.0f} / {np.median(us[ok, l, ph, 1]):.0f} / "
                             f"{us[ok, l, ph, 1].max():.0f}" if ok.any() else "-")
            out.append(f"| {l} | " + " | ".join(cells) + " |")
        out.append("")
    e.close()
    print("\n".join(out), flush=True)


SLICE = 32                      # committed tokens per benchmark step
AR_SLICES = 2                   # slices decoded again in plain full-depth mode


class SliceRunner:
    """Steps of the benchmark: consecutive slices of SLICE committed tokens of one decode,
    restarted from the prefilled snapshot after its last token."""

    def __init__(self, d, snap, n_new):
        self.d, self.snap, self.n_new = d, snap, n_new
        self.done = n_new               # forces a restart at the first step
        self.finished = []              # stats of completed decodes

    def restart(self):
        if self.done > 1:
            self.finished.append(self.d.stats())
        self.d.restore(self.snap)
        self.done = 1                   # the first new token comes from the prefill

    def step(self, progress=None):
        if self.done >= self.n_new:
            self.restart()
        before = self.done
        self.d.decode(min(self.n_new, self.done + SLICE))
        self.done = len(self.d.tokens) - self.d.prompt_len
        return self.done - before


def _merge_stats(stats, gamma_depths=None):
    out = {}
    for st in stats:
        for k, v in st.items():
            if k == "rows_hist":
                h = out.setdefault(k, {})
                for r, c in v.items():
                    h[r] = h.get(r, 0) + c
            elif isinstance(v, (int, float)) and k not in ("gamma", "rows_mean", "rows_max"):
                out[k] = out.get(k, 0) + v
    n_rows = sum(r * c for r, c in out.get("rows_hist", {}).items())
    if gamma_depths:
        # eq. 9 over all decodes: N R / (N1 d1 + N2 d2 + (N - N1 - N2) R)
        d1, d2, R = gamma_depths
        n1, n2 = out.get("accept1", 0), out.get("accept2", 0)
        N = n1 + n2 + out.get("fallback", 0)
        out["gamma"] = N * R / max(1, n1 * d1 + n2 * d2 + (N - n1 - n2) * R)
    n_steps = sum(out.get("rows_hist", {}).values())
    out["rows_mean"] = n_rows / n_steps if n_steps else 0.0
    out["rows_max"] = max(out.get("rows_hist", {0: 0}))
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="C4")
    ap.add_argument("--mode", default="spec", choices=["spec", "ar"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ar", action="store_true", help="skip the plain full-depth comparison")
    ap.add_argument("--microbench", action="store_true",
                    help="ls_loop_step at fixed row counts on the workload's shape, and a streaming-read reference")
    ap.add_argument("--phase-stamps", action="store_true",
                    help="per-phase timeline of ls_loop_step at 1, 4 and 7 rows (markdown)")
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
    if args.microbench:
        microbench(args.workload)
        return
    if args.phase_stamps:
        phase_stamps(args.workload)
        return

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
    torch.cuda.synchronize()
    tp = time.perf_counter()
    d.prefill(prompt, progress=_Progress("prefill"))
    torch.cuda.synchronize()
    t_pre = time.perf_counter() - tp
    snap = d.snapshot()
    run = SliceRunner(d, snap, n_new)
    for i in range(args.warmup):
        run.step()
        print(f"[bench] warmup step {i} done", file=sys.stderr, flush=True)
    run.restart()                             # the timed region starts a fresh decode
    run.finished = []
    torch.cuda.synchronize()
    e.prof = []
    n_before = e.n_loop_calls
    committed, step_s = 0, []
    prog = _Progress("step", every=30.0)
    t0 = time.perf_counter()
    for i in range(args.steps):
        ts = time.perf_counter()
        committed += run.step()
        step_s.append(time.perf_counter() - ts)
        prog(i + 1, args.steps)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    value = committed / dt
    run.finished.append(d.stats())
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
        "data": "synthetic (seeded random-init weights, synthetic prompt)",
        "config": {"workload": f"{wl.key}: {wl.description}", "prompt_len": dec.prompt_len, "new_tokens": n_new,
                   "mode": args.mode, "batch": 1, "step": f"{SLICE} committed tokens of the decode",
                   "timed_tokens": committed},
        "roofline": {"kernel": "ls_loop_step (one call: all layers of the shared block, all active rows)",
                     "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic["traffic_bytes_per_launch"] if traffic else None,
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                     "bytes_per_call": round(by / n_calls), "us_per_call": round(t_ms / n_calls * 1e3, 2),
                     "launches": n_calls},
        "decode_stats": {k: (round(v, 4) if isinstance(v, float) else v) for k, v in _merge_stats(
            run.finished, (dec.screen_depth if dec.copy else dec.d1, dec.d2 or cfg.R, cfg.R)).items()},
    }
    out["prefill"] = prefill_report(cfg, dec, args.mode, t_pre)
    if traffic and "mfma_util_percent" in traffic:
        # matrix-core use of the same kernel from the committed counter summary
        out["roofline"]["mfma_util_percent"] = traffic["mfma_util_percent"]
        out["roofline"]["mfma_tflops_issued"] = traffic["mfma_tflops"]
    if args.mode == "spec" and not args.no_ar:
        # the same kernels with proposals off, over the first AR_SLICES slices of a fresh decode,
        # against the spec steps that decoded the same slices
        n_ar = min(AR_SLICES, args.steps, (n_new - 2) // SLICE + 1)
        da = Decoder(e, dec, "ar")
        ra = SliceRunner(da, snap, n_new)
        torch.cuda.synchronize()
        ta = time.perf_counter()
        c_ar = sum(ra.step() for _ in range(n_ar))
        torch.cuda.synchronize()
        t_ar = time.perf_counter() - ta
        spec_s = sum(step_s[:n_ar])
        out["ar_mode"] = {"value": round(c_ar / t_ar, 3), "unit": "tokens/s", "tokens": c_ar,
                          "spec_value_same_tokens": round(c_ar / spec_s, 3),
                          "speedup": round(t_ar / spec_s, 4),
                          "note": "same kernels, proposals off (full-depth decoding), same first tokens"}
        print(f"[bench] plain full-depth mode: {c_ar / t_ar:.2f} tokens/s", file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        print("[bench] CPU reference baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(cfg, dec, w)
    print(json.dumps(out), flush=True)
    e.close()


if __name__ == "__main__":
    main()
