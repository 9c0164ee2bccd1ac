"""Looped decoder P -> B^r -> C, plain NumPy float64 (test infrastructure only).

LoopSpec page, section 2.1, eq. 1: H^(0) = P(X), H^(r) = B(H^(r-1)), p_r = C(H^(r)),
1 <= r <= R.  The pages give only this abstraction; the layer internals below are the
plainest reading consistent with the model families they name (pre-RMSNorm blocks,
multi-head attention with rotary positions, SwiGLU MLP, no biases, tied LM head).

KV caches are indexed by loop depth (section 2.1 on Fig. 2 and section 2.4: KV from
different depths is never mixed): the shared block at loop iteration k reads and writes
the cache of depth k; the Raven/Huginn-style prelude has its own cache; the coda, which
is re-run at every readout depth r, keeps one cache per readout depth (section 2.4:
the pre/post modules also need caches).

All positions of a sequence are processed through `Seq.extend`, which appends new
positions and runs P, every loop iteration 1..R and the requested readouts; calling it
once on a whole sequence is the full recomputation of eq. 1, calling it token by token is
the cached autoregressive form.
"""

import numpy as np

from .numerics import round_f32, store, weight_f64


class KV:
    """One layer's cache at one depth: keys/values of positions 0..n-1 (float64 holding
    storage-rounded values)."""

    def __init__(self, d, cap=64):
        self.K = np.zeros((cap, d))
        self.Vv = np.zeros((cap, d))
        self.n = 0

    def append(self, k, v):
        need = self.n + k.shape[0]
        if need > self.K.shape[0]:
            cap = max(need, 2 * self.K.shape[0])
            K2 = np.zeros((cap, self.K.shape[1])); K2[: self.n] = self.K[: self.n]
            V2 = np.zeros((cap, self.K.shape[1])); V2[: self.n] = self.Vv[: self.n]
            self.K, self.Vv = K2, V2
        self.K[self.n:need] = k
        self.Vv[self.n:need] = v
        self.n = need


class Model:
    def __init__(self, cfg, weights, products="f64"):
        """products: "f64" (the reference) computes every matrix product in float64.  "f32"
        computes them with float32 operands and accumulation instead (the stored values are
        float32-exact, so only the summation precision changes): a second implementation of
        the same model, used to measure how far rounding-level differences carry through
        many loop iterations."""
        self.cfg = cfg
        self.dt = cfg.dtype
        # float32 tensors of the model (residual stream, queries, products); left
        # unrounded in the "f64" pinning mode
        self.r32 = (lambda x: x) if cfg.dtype == "f64" else round_f32
        wdt = np.float64 if products == "f64" else np.float32
        if products == "f64":
            self.mm = lambda a, W: a @ W.T
        elif products == "f32":
            self.mm = lambda a, W: (np.asarray(a, np.float32) @ W.T).astype(np.float64)
        else:
            raise ValueError(products)
        self.emb = weight_f64(weights["emb"]).astype(wdt, copy=False)     # [V, d], also the tied head

        def conv(layers):
            return [{k: (weight_f64(v).astype(wdt, copy=False) if k.startswith("W") else np.asarray(v, np.float64))
                     for k, v in lw.items()} for lw in layers]

        self.pre = conv(weights["pre"])
        self.core = conv(weights["core"])
        self.coda = conv(weights["coda"])
        self.g_final = np.asarray(weights["g_final"], np.float64)
        hd = cfg.head_dim
        self.inv_freq = cfg.rope_theta ** (-np.arange(0, hd // 2, dtype=np.float64) * 2.0 / hd)

    # ---- building blocks -------------------------------------------------------------
    def rmsnorm(self, h, g):
        """h / sqrt(mean(h^2) + eps) * g, row-wise."""
        ms = np.mean(h * h, axis=-1, keepdims=True)
        return h / np.sqrt(ms + self.cfg.norm_eps) * g

    def rope(self, x, pos):
        """Rotary embedding, rotate-half convention, per head: the pair (i, i + hd/2) is
        rotated by angle pos * theta^(-2i/hd)."""
        n = x.shape[0]
        hd = self.cfg.head_dim
        half = hd // 2
        xh = x.reshape(n, self.cfg.n_heads, hd)
        ang = np.asarray(pos, np.float64)[:, None] * self.inv_freq[None, :]      # [n, half]
        c = np.cos(ang)[:, None, :]
        s = np.sin(ang)[:, None, :]
        a, b = xh[..., :half], xh[..., half:]
        out = np.concatenate([a * c - b * s, b * c + a * s], axis=-1)
        return out.reshape(n, -1)

    def attention(self, q, kv, first_pos):
        """Causal multi-head attention of n new rows at positions first_pos.. over the
        cache (which already holds them).  Row i sees keys 0..first_pos+i inclusive."""
        n = q.shape[0]
        H, hd = self.cfg.n_heads, self.cfg.head_dim
        T = first_pos + n
        K = kv.K[:T].reshape(T, H, hd)
        Vv = kv.Vv[:T].reshape(T, H, hd)
        qh = q.reshape(n, H, hd)
        out = np.empty((n, H, hd))
        scale = 1.0 / np.sqrt(hd)
        for i0 in range(0, n, 256):
            i1 = min(n, i0 + 256)
            s = np.einsum("ihe,the->hit", qh[i0:i1], K) * scale               # [H, rows, T]
            rows = np.arange(i0, i1) + first_pos
            mask = np.arange(T)[None, :] > rows[:, None]                        # future keys
            s[:, mask] = -np.inf
            s -= s.max(axis=-1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=-1, keepdims=True)
            out[i0:i1] = np.einsum("hit,the->ihe", p, Vv)
        return out.reshape(n, -1)

    def layer(self, lw, h, first_pos, kv):
        """One pre-norm block on n consecutive new positions; appends their K/V to kv."""
        dt = self.dt
        R32 = self.r32
        n = h.shape[0]
        pos = np.arange(first_pos, first_pos + n)
        a = store(self.rmsnorm(h, lw["g1"]), dt)
        q = R32(self.mm(a, lw["Wq"]))
        k = R32(self.mm(a, lw["Wk"]))
        v = R32(self.mm(a, lw["Wv"]))
        q = R32(self.rope(q, pos))
        k = store(self.rope(k, pos), dt)
        v = store(v, dt)
        assert kv.n == first_pos, "positions must be appended in order"
        kv.append(k, v)
        o = store(self.attention(q, kv, first_pos), dt)
        h = R32(h + R32(self.mm(o, lw["Wo"])))
        b = store(self.rmsnorm(h, lw["g2"]), dt)
        g = R32(self.mm(b, lw["Wg"]))
        u = R32(self.mm(b, lw["Wu"]))
        act = store(g / (1.0 + np.exp(-g)) * u, dt)                            # silu(g) * u
        h = R32(h + R32(self.mm(act, lw["Wd"])))
        return h

    # ---- sequences ---------------------------------------------------------------------
    def new_seq(self):
        return Seq(self)


class Seq:
    """State of one token sequence: all per-depth caches and the processed length."""

    def __init__(self, model: Model):
        self.m = model
        self.n = 0
        self.caches = {}

    def cache(self, kind, depth, layer):
        key = (kind, depth, layer)
        if key not in self.caches:
            self.caches[key] = KV(self.m.cfg.d)
        return self.caches[key]

    def prelude(self, tokens, first):
        """P: embedding (plus the prelude layers of the Raven/Huginn family)."""
        m = self.m
        R32 = m.r32
        h = R32(m.emb[np.asarray(tokens)])
        for l, lw in enumerate(m.pre):
            h = m.layer(lw, h, first, self.cache("pre", 0, l))
        return h

    def loop(self, h, k, first):
        """Loop iteration k (1..R) of the shared block B, using cache depth k."""
        m = self.m
        for l, lw in enumerate(m.core):
            h = m.layer(lw, h, first, self.cache("core", k, l))
        return h

    def readout_logits(self, h, r, first):
        """C at depth r up to the logits: coda layers (cache of readout depth r), final
        RMSNorm, tied LM head.  Returns float32-valued logits [n, V]."""
        m = self.m
        for l, lw in enumerate(m.coda):
            h = m.layer(lw, h, first, self.cache("coda", r, l))
        a = store(m.rmsnorm(h, m.g_final), m.dt)
        return m.r32(m.mm(a, m.emb))

    def extend(self, tokens, depths=None, last_only=True, keep_hidden=False):
        """Append tokens; run P, loops 1..R, and readouts at `depths` (default: all of D).

        Returns {r: logits} (rows of the last position only if last_only).  With
        keep_hidden, also returns {r: H^(r)} for r = 0..R.
        """
        m = self.m
        cfg = m.cfg
        depths = cfg.readout_depths if depths is None else tuple(depths)
        first = self.n
        h = self.prelude(tokens, first)
        hidden = {0: h} if keep_hidden else None
        logits = {}
        for k in range(1, cfg.R + 1):
            h = self.loop(h, k, first)
            if keep_hidden:
                hidden[k] = h
            if k in depths:
                lg = self.readout_logits(h, k, first)
                logits[k] = lg[-1] if last_only else lg
        self.n += len(tokens)
        return (logits, hidden) if keep_hidden else logits
