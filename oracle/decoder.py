"""CPU oracle for the batch-1 decode step of a Laneformer-2B-shaped decoder.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import or call this
module; only the tests, the smoke check and the benchmark's CPU-baseline leg
do. It shares no code with the HIP library: both sides receive the same seeded
fp16 inputs and compute independently.

What it computes (Kog Laneformer 2B blog, "Designing the architecture"): a
largely ordinary decoder-only transformer, pre-norm, with causal
grouped-query attention (32 query / 16 key-value heads), sliding-window
attention on some layers, and a KV cache that every new token reads in full
(the cache, like the weights, is what the blog says each token must stream).
Inference runs in FP16 at batch 1 and decodes greedily (asector.ru summary,
"Performance and infrastructure"; blog TL;DR).

Precision: all arithmetic in float64 from the exact fp16 weights. Following
the FP16 inference the pages state, the cached keys and values are rounded to
fp16 when stored, exactly as the cache format holds them; nothing else is
rounded.

Readings of points the pages leave open (each is a parameter or a fixed
choice, stated once here):
  * pre-norm RMSNorm before attention and FFN, and a final RMSNorm before the
    untied LM head; eps from the config (1e-5);
  * rotary embedding on q and k, half-split pairs (c, c + hd/2), angle
    p * theta^(-2c/hd), absolute positions from 0;
  * query head i reads key/value head floor(i * Hkv / Hq): consecutive query
    heads share a kv head, which keeps each lane's heads self-contained;
  * a sliding window of width W shows keys j with p - W < j <= p (the current
    key counts toward W); W = 0 means full causal attention;
  * SwiGLU: silu(gate) * up, silu(u) = u / (1 + exp(-u)); no biases; scores
    scaled by 1/sqrt(hd);
  * greedy choice = the lowest index among the maximal logits, compared in
    float32 (the precision the GPU path decides in).
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


# ----------------------------------------------------------------- primitives

def rmsnorm(x, gain, eps):
    """gain * x / sqrt(mean(x^2) + eps) over the last axis."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return gain * (x / np.sqrt(ms + eps))


def rope_angles(positions, head_dim, theta):
    """Angles p * theta^(-2c/hd) for c in [0, hd/2): shape [..., hd/2]."""
    c = np.arange(head_dim // 2, dtype=F64)
    inv_freq = np.power(F64(theta), -2.0 * c / head_dim)
    return np.multiply.outer(np.asarray(positions, dtype=F64), inv_freq)


def apply_rope(u, positions, theta):
    """Rotate each (u_c, u_{c+hd/2}) pair by its angle.

    u: [T, H, hd] with positions [T], or [H, hd] with a scalar position."""
    hd = u.shape[-1]
    half = hd // 2
    ang = rope_angles(positions, hd, theta)
    if u.ndim == 3:
        ang = ang[:, None, :]
    cos, sin = np.cos(ang), np.sin(ang)
    a, b = u[..., :half], u[..., half:]
    return np.concatenate([a * cos - b * sin, a * sin + b * cos], axis=-1)


def silu(u):
    return u / (1.0 + np.exp(-u))


def kv_head_of(i, n_q, n_kv):
    """The key/value head that query head i reads."""
    return (i * n_kv) // n_q


def visible_range(p, window):
    """[lo, hi) of the keys position p attends to."""
    lo = 0 if window == 0 else max(0, p - window + 1)
    return lo, p + 1


def softmax(s):
    e = np.exp(s - np.max(s, axis=-1, keepdims=True))
    return e / np.sum(e, axis=-1, keepdims=True)


def attend(q, K, V, n_kv):
    """Decode attention of one position.

    q: [Hq, hd]; K, V: [n, Hkv, hd] (the visible keys). Returns [Hq, hd]."""
    n_q, hd = q.shape
    out = np.empty_like(q)
    for i in range(n_q):
        g = kv_head_of(i, n_q, n_kv)
        s = (K[:, g, :] @ q[i]) / np.sqrt(F64(hd))
        out[i] = softmax(s) @ V[:, g, :]
    return out


def greedy(logits):
    """Index of the maximal logit; the lowest such index on exact ties.

    The choice is taken on the logits rounded to float32, the precision in
    which the GPU path holds and compares its logits, so both sides decide in
    the same precision."""
    return int(np.argmax(np.asarray(logits, dtype=F64).astype(np.float32)))


def to_cache(a, kv_fp16):
    return a.astype(np.float16).astype(F64) if kv_fp16 else a


# ---------------------------------------------------------------- the decoder

class OracleDecoder:
    """The decoder on the CPU, holding float64 copies of the fp16 weights.

    weights: dict name -> fp16 array as made by synth.make_weights.
    cache_weights=False converts each matrix when used and drops it after,
    which bounds memory for one-off full-size steps."""

    def __init__(self, cfg, weights, kv_fp16=True, cache_weights=True):
        self.cfg = cfg
        self.src = weights
        self.kv_fp16 = kv_fp16
        self.cache_weights = cache_weights
        self._w = {}

    def w(self, name):
        if name in self._w:
            return self._w[name]
        a = np.asarray(self.src[name], dtype=F64)
        if self.cache_weights:
            self._w[name] = a
        return a

    def lw(self, l, name):
        return self.w(f"layers.{l}.{name}")

    # ------------------------------------------------------------- the cache
    def new_cache(self, length=None):
        c = self.cfg
        n = c.max_ctx if length is None else length
        shape = (c.n_layers, n, c.n_kv_heads, c.head_dim)
        return {"K": np.zeros(shape, F64), "V": np.zeros(shape, F64), "len": 0}

    def load_cache(self, cache, K, V):
        """Adopt given cache content (fp16 values, post-rotation keys) for
        positions [0, len(K))."""
        n = K.shape[1]
        cache["K"][:, :n] = np.asarray(K, F64)
        cache["V"][:, :n] = np.asarray(V, F64)
        cache["len"] = n

    # ------------------------------------------------------------ components
    def qkv(self, l, h):
        """Project normed input h [..., d] to q [..., Hq, hd], k, v [..., Hkv, hd]."""
        c = self.cfg
        y = h @ self.lw(l, "wqkv").T
        nq, nk = c.n_q_heads * c.head_dim, c.n_kv_heads * c.head_dim
        lead = y.shape[:-1]
        q = y[..., :nq].reshape(*lead, c.n_q_heads, c.head_dim)
        k = y[..., nq:nq + nk].reshape(*lead, c.n_kv_heads, c.head_dim)
        v = y[..., nq + nk:].reshape(*lead, c.n_kv_heads, c.head_dim)
        return q, k, v

    def ffn(self, l, x):
        """SwiGLU block on the residual x (pre-norm); returns its output."""
        c = self.cfg
        h = rmsnorm(x, self.lw(l, "ffn_norm"), c.rms_eps)
        gu = h @ self.lw(l, "wgate_up").T
        gate, up = gu[..., :c.ffn], gu[..., c.ffn:]
        return (silu(gate) * up) @ self.lw(l, "wdown").T

    def head(self, x):
        c = self.cfg
        return rmsnorm(x, self.w("final_norm"), c.rms_eps) @ self.w("lm_head").T

    def embed(self, tokens):
        return self.w("embed")[np.asarray(tokens)]

    # -------------------------------------------------- one position (decode)
    def step(self, cache, token=None, x=None):
        """Append one position at p = cache['len'] and return its logits
        (or, with vocab == 0, the output hidden vector)."""
        c = self.cfg
        p = cache["len"]
        if p >= cache["K"].shape[1]:
            raise ValueError("cache full")
        x = self.embed(token) if token is not None else np.asarray(x, F64).copy()
        for l in range(c.n_layers):
            h = rmsnorm(x, self.lw(l, "attn_norm"), c.rms_eps)
            q, k, v = self.qkv(l, h)
            q = apply_rope(q, p, c.rope_theta)
            k = apply_rope(k, p, c.rope_theta)
            cache["K"][l, p] = to_cache(k, self.kv_fp16)
            cache["V"][l, p] = to_cache(v, self.kv_fp16)
            lo, hi = visible_range(p, c.windows[l])
            o = attend(q, cache["K"][l, lo:hi], cache["V"][l, lo:hi], c.n_kv_heads)
            x = x + self.lw(l, "wo") @ o.reshape(-1)
            x = x + self.ffn(l, x)
        cache["len"] = p + 1
        return self.head(x) if c.vocab else x

    # --------------------------------------- whole sequence, explicit masks
    def mask(self, T, window, start=0):
        """Boolean [T, start+T]: row t (position start+t) may see key j."""
        pos = start + np.arange(T)[:, None]
        j = np.arange(start + T)[None, :]
        m = j <= pos
        if window:
            m &= (pos - j) < window
        return m

    def forward_sequence(self, tokens=None, xs=None, cache=None):
        """Process positions [0, T) at once with explicit mask matrices and a
        brute-force softmax. Returns logits [T, V] (hidden [T, d] if vocab == 0).
        If cache is given, its positions [0, T) are filled as decode would."""
        c = self.cfg
        X = self.embed(tokens) if tokens is not None else np.asarray(xs, F64).copy()
        T = X.shape[0]
        pos = np.arange(T)
        group = c.n_q_heads // c.n_kv_heads
        for l in range(c.n_layers):
            H = rmsnorm(X, self.lw(l, "attn_norm"), c.rms_eps)
            q, k, v = self.qkv(l, H)
            q = apply_rope(q, pos, c.rope_theta)
            k = to_cache(apply_rope(k, pos, c.rope_theta), self.kv_fp16)
            v = to_cache(v, self.kv_fp16)
            if cache is not None:
                cache["K"][l, :T] = k
                cache["V"][l, :T] = v
            M = self.mask(T, c.windows[l])
            O = np.empty((T, c.n_q_heads, c.head_dim))
            for i in range(c.n_q_heads):
                g = i // group
                S = (q[:, i, :] @ k[:, g, :].T) / np.sqrt(F64(c.head_dim))
                S = np.where(M, S, -np.inf)
                O[:, i, :] = softmax(S) @ v[:, g, :]
            X = X + O.reshape(T, -1) @ self.lw(l, "wo").T
            X = X + self.ffn(l, X)
        if cache is not None:
            cache["len"] = T
        return self.head(X) if c.vocab else X

    # ------------------------------------------------------------ generation
    def generate(self, prompt, n_steps, force=None):
        """Prefill the prompt, then n_steps greedy steps.

        Returns (logits [n_steps+1, V], tokens [n_steps+1]): row 0 is the last
        prompt position, row s the s-th generated position. `force`, if given,
        maps a step index to the token fed there instead of the greedy one."""
        cache = self.new_cache()
        z = self.forward_sequence(tokens=prompt, cache=cache)[-1]
        logits = [z]
        toks = [greedy(z)]
        for s in range(n_steps):
            t = toks[-1] if force is None or s not in force else force[s]
            z = self.step(cache, token=t)
            logits.append(z)
            toks.append(greedy(z))
        return np.stack(logits), np.array(toks, dtype=np.int64)
