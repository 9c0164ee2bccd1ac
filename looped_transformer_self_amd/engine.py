"""Device-resident model state and thin wrappers over the libloopspec calls.

PyTorch provides device memory and the stream; every computation runs in the HIP kernels
behind the C ABI.  Holds: weights (uploaded once), the depth-indexed KV caches, the
slot-indexed hidden states H[S][d], a pool of probability rows, and the workspace.
"""

import ctypes as C
import os

import numpy as np
import torch

from . import _lib as L


def _ptr(t):
    return C.c_void_p(t.data_ptr()) if t is not None else C.c_void_p(0)


_hip = None


def _hip_runtime():
    """The HIP runtime library that torch and libloopspec already share (found by soname, never
    loaded a second time), for raw asynchronous copies."""
    global _hip
    if _hip is None:
        _hip = C.CDLL("libamdhip64.so.7", mode=os.RTLD_NOLOAD | os.RTLD_GLOBAL)
        _hip.hipMemcpyAsync.argtypes = [C.c_void_p, C.c_void_p, C.c_size_t, C.c_int, C.c_void_p]
        _hip.hipMemcpyAsync.restype = C.c_int
        _hip.hipEventCreateWithFlags.argtypes = [C.POINTER(C.c_void_p), C.c_uint]
        _hip.hipEventCreateWithFlags.restype = C.c_int
        _hip.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]
        _hip.hipEventRecord.restype = C.c_int
        _hip.hipEventSynchronize.argtypes = [C.c_void_p]
        _hip.hipEventSynchronize.restype = C.c_int
        _hip.hipEventDestroy.argtypes = [C.c_void_p]
        _hip.hipEventDestroy.restype = C.c_int
    return _hip


class Uploader:
    """Packs host int32/uint32 arrays into one pinned buffer and ships them with a single
    host-to-device copy per call (hipMemcpyAsync on the engine's stream).  A ring of buffers
    guarded by reusable events keeps a pending copy from being overwritten."""

    H2D = 1   # hipMemcpyHostToDevice

    def __init__(self, dev, stream_ptr, words=1 << 20, ring=4):
        self.dev = dev
        self.stream = stream_ptr
        self.host = [torch.empty(words, dtype=torch.int32, pin_memory=True) for _ in range(ring)]
        self.hnp = [h.numpy() for h in self.host]
        self.hptr = [h.data_ptr() for h in self.host]
        self.devb = [torch.empty(words, dtype=torch.int32, device=dev) for _ in range(ring)]
        self.dptr = [d.data_ptr() for d in self.devb]
        self.hip = _hip_runtime()
        self.events = []
        for _ in range(ring):
            ev = C.c_void_p()
            if self.hip.hipEventCreateWithFlags(C.byref(ev), 2):          # hipEventDisableTiming
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.events.append(ev)
        self.recorded = [False] * ring
        self.i = 0

    def close(self):
        """Destroy the events; call before the process exits (interpreter teardown may run
        after the HIP runtime has shut down, when a destructor's HIP call is unsafe)."""
        for ev in self.events:
            self.hip.hipEventDestroy(ev)
        self.events = []
        self.recorded = []

    def _slot(self):
        k = self.i
        self.i = (self.i + 1) % len(self.host)
        if self.recorded[k] and self.hip.hipEventSynchronize(self.events[k]):
            raise RuntimeError("hipEventSynchronize failed")
        return k

    def _ship(self, k, dst, words, src_off=0):
        err = self.hip.hipMemcpyAsync(dst, self.hptr[k] + 4 * src_off, 4 * words, self.H2D, self.stream)
        if err:
            raise RuntimeError(f"hipMemcpyAsync failed ({err})")
        if self.hip.hipEventRecord(self.events[k], self.stream):
            raise RuntimeError("hipEventRecord failed")
        self.recorded[k] = True

    def copy_to(self, dst_ptr, array):
        """Asynchronous copy of a small int32 array to device address dst_ptr (stream order)."""
        a = np.asarray(array, np.int32)
        k = self._slot()
        self.hnp[k][:len(a)] = a
        self._ship(k, dst_ptr, len(a))

    def ship_words(self, head, words):
        """One copy of an int32 array followed by a list of ints; returns the device base
        address and the buffer that holds it."""
        k = self._slot()
        nh, total = len(head), len(head) + len(words)
        if total > len(self.hnp[k]):
            raise ValueError("upload larger than the staging buffer")
        hb = self.hnp[k]
        hb[:nh] = head
        hb[nh:total] = words
        self._ship(k, self.dptr[k], total)
        return self.dptr[k], self.devb[k]

    def pack(self, arrays):
        k = self._slot()
        offs, total = [], 0
        for a in arrays:
            offs.append(total)
            total += (len(a) + 63) // 64 * 64          # 256-byte alignment per array
        if total > len(self.hnp[k]):
            raise ValueError("upload larger than the staging buffer")
        hb = self.hnp[k]
        for a, o in zip(arrays, offs):
            if len(a):
                a = np.asarray(a)
                hb[o:o + len(a)] = a.view(np.int32) if a.dtype != np.int32 else a
        self._ship(k, self.dptr[k], total)
        base = self.dptr[k]
        return [C.c_void_p(base + 4 * o) for o in offs], self.devb[k]


class Rows:
    """An ls_rows descriptor whose arrays live in an uploaded device buffer."""

    def __init__(self, struct, keep):
        self.s = struct
        self.keep = keep
        self.n = struct.n


class Engine:
    def __init__(self, cfg, weights, slot_capacity, max_rows=16, max_keys=None, max_jobs=64, prob_rows=64,
                 device="cuda"):
        self.cfg = cfg
        self.dev = torch.device(device)
        self._stream = C.c_void_p(torch.cuda.current_stream(self.dev).cuda_stream)
        self.S = int(slot_capacity)
        self.max_rows = max_rows
        self.max_keys = int(max_keys or slot_capacity)
        self.max_jobs = max_jobs
        self.prob_rows = prob_rows
        bf16 = cfg.dtype == "bf16"
        self.wdtype = torch.int16 if bf16 else torch.float32

        def up(a):
            a = np.ascontiguousarray(a)
            if a.dtype == np.uint16:
                a = a.view(np.int16)
            return torch.from_numpy(a).to(self.dev)

        self.w = {"emb": up(weights["emb"]), "g_final": up(weights["g_final"])}
        self.layers = {}
        for part in ("pre", "core", "coda"):
            self.layers[part] = [{k: up(v) for k, v in lw.items()} for lw in weights[part]]

        def lp(lw):
            return L.ls_layer_ptrs(*[_ptr(lw[k]) for k in ("Wq", "Wk", "Wv", "Wo", "Wg", "Wu", "Wd", "g1", "g2")])

        self._lp = {p: (L.ls_layer_ptrs * max(1, len(v)))(*[lp(x) for x in v]) for p, v in self.layers.items()}
        wp = L.ls_weight_ptrs(_ptr(self.w["emb"]), _ptr(self.w["g_final"]), self._lp["pre"], self._lp["core"],
                              self._lp["coda"])
        desc = L.ls_model_desc()
        desc.V, desc.d, desc.n_heads, desc.head_dim, desc.F = cfg.V, cfg.d, cfg.n_heads, cfg.head_dim, cfg.F
        desc.L, desc.L_pre, desc.L_coda, desc.R = cfg.L, cfg.L_pre, cfg.L_coda, cfg.R
        desc.n_readout = len(cfg.readout_depths)
        for i, r in enumerate(cfg.readout_depths):
            desc.readout_depths[i] = r
        desc.dtype = L.LS_BF16 if bf16 else L.LS_F32
        desc.rope_theta = cfg.rope_theta
        desc.norm_eps = cfg.norm_eps
        desc.slot_capacity = self.S
        self.desc = desc
        h = C.c_void_p()
        L.check(L.lib.ls_model_create(C.byref(desc), C.byref(wp), C.byref(h)), "ls_model_create")
        self.h = h

        d = cfg.d
        ent = 2 * d
        self.kv_core = torch.zeros(cfg.R * cfg.L * self.S * ent, dtype=self.wdtype, device=self.dev)
        self.kv_pre = (torch.zeros(cfg.L_pre * self.S * ent, dtype=self.wdtype, device=self.dev)
                       if cfg.L_pre else None)
        self.kv_coda = (torch.zeros(len(cfg.readout_depths) * cfg.L_coda * self.S * ent, dtype=self.wdtype,
                                    device=self.dev) if cfg.L_coda else None)
        self.kv = L.ls_kv(_ptr(self.kv_core), _ptr(self.kv_pre), _ptr(self.kv_coda))
        self.H = torch.zeros(self.S, d, dtype=torch.float32, device=self.dev)
        self.probs = torch.zeros(prob_rows, cfg.V, dtype=torch.float32, device=self.dev)
        nb = L.lib.ls_workspace_bytes(h, max_rows, self.max_keys, max_jobs)
        self.ws = torch.empty(nb + 256, dtype=torch.uint8, device=self.dev)
        off = (-self.ws.data_ptr()) % 256
        self.ws_ptr = C.c_void_p(self.ws.data_ptr() + off)
        L.check(L.lib.ls_bind_workspace(h, self.ws_ptr, max_rows, self.max_keys, max_jobs, self.stream_ptr()),
                "ls_bind_workspace")
        self.up = Uploader(self.dev, self._stream)
        # verification results: pinned host memory that the verify kernel writes directly, so
        # reading them needs no device-to-host copy after the stream synchronisation
        self.vout_host = torch.zeros(max_jobs * 4, dtype=torch.int32, pin_memory=True)
        # verification inputs (jobs, uniforms, copy candidates) in pinned host memory that the
        # kernel reads once per job: no host-to-device copy ahead of it.  verify() returns only
        # after the stream has synchronised, so the next call may overwrite them.
        self._vin_jobs = max_jobs
        self.vin_host = torch.zeros(max_jobs * (10 + 24 + 16), dtype=torch.int32, pin_memory=True)
        self.vin_np = self.vin_host.numpy()
        self.pws = None           # prefill scratch (allocated at the first prefill, sized for its chunk)
        self.pws_bytes = 0
        self.prefill_chunk = 2048 # prompt positions per ls_prefill call
        self.prof = None          # list of (start event, end event, row metadata) when profiling
        self.n_loop_calls = 0     # ls_loop_step launches with at least one row, since creation

    def close(self):
        """Release the model handle, the events and the device buffers, in that order, after
        the engine's stream has drained.  Programs call this before they exit: left to
        interpreter teardown, these releases can run after the HIP runtime (or a profiler
        attached to it) has already shut down."""
        if getattr(self, "h", None) is None:
            return
        torch.cuda.current_stream(self.dev).synchronize()
        L.lib.ls_model_destroy(self.h)
        self.h = None
        self.up.close()
        for name in ("kv_core", "kv_pre", "kv_coda", "H", "probs", "ws", "pws", "w", "layers", "vout_host",
                     "vin_host"):
            setattr(self, name, None)
        self.vin_np = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def stream_ptr(self):
        """The stream every call of this engine is issued on: the current stream when the
        engine was created."""
        return self._stream

    # ---- descriptors -----------------------------------------------------------------
    def rows(self, slots, pos, depth, n_fin, anc_lists, fin_ptr, extra=()):
        """Build an ls_rows over uploaded arrays.  anc_lists: per row list of ancestor slots.
        fin_ptr: device pointer (c_void_p) of the finished-prefix slot table.  `extra` arrays
        ride along in the same upload; their device pointers are returned too."""
        n = len(slots)
        anc_off = np.zeros(n + 1, np.int32)
        for i, a in enumerate(anc_lists):
            anc_off[i + 1] = anc_off[i] + len(a)
        anc = np.concatenate([np.asarray(a, np.int32) for a in anc_lists]) if anc_off[-1] else np.zeros(1, np.int32)
        ptrs, keep = self.up.pack([np.asarray(slots, np.int32), np.asarray(pos, np.int32),
                                   np.asarray(depth, np.int32), anc_off, anc, *extra])
        s = L.ls_rows()
        s.n, s.n_fin = n, int(n_fin)
        s.max_anc = int(max((len(a) for a in anc_lists), default=0))
        s.slot, s.pos, s.depth = ptrs[0], ptrs[1], ptrs[2]
        s.fin_slots = fin_ptr
        s.anc_off, s.anc_slots = ptrs[3], ptrs[4]
        r = Rows(s, keep)
        r.extra = ptrs[5:]
        r.host = (int(n_fin), list(slots), list(depth), anc_lists)
        return r

    def rows_set(self, specs, fin):
        """Several ls_rows over ONE upload: specs are (slots, pos, depth, n_fin, anc_lists,
        extra) tuples as for rows(); `fin` (int32 array) is the finished-prefix slot table,
        shipped in the same copy and shared by every descriptor.  The descriptors' arrays are
        laid end to end after it (int32 elements need no wider alignment).  This runs between
        a step's verification result and its next launch, so it is kept to plain list work."""
        words, layout = [], []
        nf = len(fin)
        for slots, pos, depth, n_fin, anc_lists, extra in specs:
            o_slot = nf + len(words)
            words += slots
            words += pos
            words += depth
            o_off = nf + len(words)
            acc = mx = 0
            words.append(0)
            for a in anc_lists:
                na = len(a)
                acc += na
                if na > mx:
                    mx = na
                words.append(acc)
            o_anc = nf + len(words)
            for a in anc_lists:
                words += a
            if acc == 0:
                words.append(0)
            o_extra = []
            for x in extra:
                o_extra.append(nf + len(words))
                words += x.tolist() if isinstance(x, np.ndarray) else list(x)
            layout.append((o_slot, o_off, o_anc, mx, o_extra))
        base, keep = self.up.ship_words(fin, words)
        out = []
        for (slots, pos, depth, n_fin, anc_lists, extra), (o_slot, o_off, o_anc, mx, o_extra) in zip(specs, layout):
            n = len(slots)
            s = L.ls_rows(n, n_fin, mx, base + 4 * o_slot, base + 4 * (o_slot + n), base + 4 * (o_slot + 2 * n), base,
                          base + 4 * o_off, base + 4 * o_anc)
            r = Rows(s, keep)
            r.extra = [C.c_void_p(base + 4 * o) for o in o_extra]
            r.host = (n_fin, slots, depth, anc_lists)
            out.append(r)
        return out

    # ---- calls ---------------------------------------------------------------------------
    def prelude(self, rows, tokens_ptr):
        L.check(L.lib.ls_prelude(self.h, C.byref(rows.s), tokens_ptr, _ptr(self.H), C.byref(self.kv),
                                 self.stream_ptr()), "ls_prelude")

    def prefill(self, tokens, slots, n_fin, fin_ptr, coda_mask):
        """ls_prefill of one chunk of prompt positions n_fin .. n_fin + len(tokens) - 1 into
        `slots` (the committed prefix's slot table at fin_ptr), H[slots] = H^(R) afterwards."""
        n = len(tokens)
        need = int(L.lib.ls_prefill_workspace_bytes(self.h, n))
        if self.pws is None or self.pws_bytes < need:
            self.pws = None
            self.pws = torch.empty(need + 256, dtype=torch.uint8, device=self.dev)
            self.pws_bytes = need
        ptr = self.pws.data_ptr() + (-self.pws.data_ptr()) % 256
        arrs, _keep = self.up.pack([np.asarray(tokens, np.int32), np.asarray(slots, np.int32)])
        L.check(L.lib.ls_prefill(self.h, arrs[0], arrs[1], n, fin_ptr, int(n_fin), int(coda_mask), _ptr(self.H),
                                 C.byref(self.kv), C.c_void_p(ptr), self.pws_bytes, self.stream_ptr()), "ls_prefill")

    def loop_step(self, rows):
        if self.prof is not None and rows.n:
            b, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            b.record()
        L.check(L.lib.ls_loop_step(self.h, C.byref(rows.s), _ptr(self.H), C.byref(self.kv), self.stream_ptr()),
                "ls_loop_step")
        self.n_loop_calls += rows.n > 0
        if self.prof is not None and rows.n:
            e.record()
            self.prof.append((b, e, rows.host))

    def loop_step_bytes(self, host):
        """Algorithmic HBM bytes of one ls_loop_step: block weights once, the unique KV
        entries read (distinct (depth, slot) pairs over all rows' keys, for every layer), the
        KV entries written, and the hidden rows read and written."""
        cfg = self.cfg
        n_fin, slots, depth, anc = host
        es = 2 if cfg.dtype == "bf16" else 4
        w = cfg.L * (4 * cfg.d * cfg.d + 3 * cfg.F * cfg.d) * es
        keys = 0
        for dep in set(depth):
            extra = set()
            for s_, d_, a in zip(slots, depth, anc):
                if d_ == dep:
                    extra.update(a)
                    extra.add(s_)
            keys += n_fin + len(extra)
        ent = 2 * cfg.d * es
        return w + keys * cfg.L * ent + len(slots) * cfg.L * ent + 2 * len(slots) * cfg.d * 4

    def readout(self, rows, greedy, T, top_p, out_rows_ptr, argmax=None, logits=None):
        smp = L.ls_sampling(int(bool(greedy)), float(T), float(top_p))
        L.check(L.lib.ls_readout(self.h, C.byref(rows.s), _ptr(self.H), C.byref(smp), _ptr(self.probs),
                                 out_rows_ptr, self.prob_rows, _ptr(argmax), _ptr(logits), C.byref(self.kv),
                                 self.stream_ptr()), "ls_readout")

    def verify(self, jobs, uniforms, cands=None):
        """jobs: int32 array [n][10]; uniforms: uint32 [n][24]; cands: int32 array or None.
        Returns an int32 numpy array [n][4] (token, outcome, gate, aux) after a stream sync;
        `last_cands` then holds the candidate array as the kernel left it (screening jobs
        reorder their range)."""
        n = len(jobs)
        ncand = len(cands) if cands is not None else 0
        if n > self._vin_jobs or ncand > 16 * self._vin_jobs:
            raise ValueError("more verification jobs or candidates than the engine was built for")
        mj = self._vin_jobs
        vin, base = self.vin_np, self.vin_host.data_ptr()
        vin[:10 * n] = np.asarray(jobs, np.int32).ravel()
        vin[10 * mj:10 * mj + 24 * n] = np.asarray(uniforms, np.uint32).ravel().view(np.int32)
        if ncand:
            vin[34 * mj:34 * mj + ncand] = np.asarray(cands, np.int32)
        L.check(L.lib.ls_verify(self.h, C.c_void_p(base), n, _ptr(self.probs), self.prob_rows,
                                C.c_void_p(base + 4 * 34 * mj) if ncand else C.c_void_p(0), ncand,
                                C.c_void_p(base + 4 * 10 * mj), _ptr(self.vout_host), self.stream_ptr()),
                "ls_verify")
        torch.cuda.current_stream().synchronize()
        # candidate ranges as the screening jobs left them (survivors first)
        self.last_cands = vin[34 * mj:34 * mj + ncand].copy()
        return self.vout_host[:4 * n].numpy().reshape(n, 4).copy()

    def sync_status(self):
        return L.lib.ls_sync_status(self.h, self.stream_ptr())
