"""fp64 decoder-only model: per-token decoder and cacheless recompute.

Test infrastructure only (see the package docstring).

The model is the plain pre-norm transformer the synthetic workloads describe:

  x = E[t]
  per layer:  h = rmsnorm(x) * g_attn
              q, k, v = Wq h, Wk h, Wv h            (one q/k/v vector per head)
              q, k    = rope(q, pos), rope(k, pos)  (rotate-half, theta ** (-2i/dh))
              o_j     = softmax_t(q_j . k_t / sqrt(dh)) . v_t   over t = 0..pos,
                        with KV head j // (n_q / n_kv) for query head j
              x      += Wo concat(o)
              h       = rmsnorm(x) * g_mlp
              x      += Wd (act(Wg h) * (Wu h))     act = SiLU or tanh-GELU
  logits = E (rmsnorm(x) * g_final)                 (tied LM head)

Weights are canonical [out, in]; every matrix is widened exactly to fp64.
"""
from __future__ import annotations

import math

import numpy as np

from seeded_inputs.weights import f32_from_bf16_bits


# ---------------------------------------------------------------- primitives
def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * g over the last axis."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def rope_angles(pos, head_dim: int, theta: float) -> np.ndarray:
    """Angle pos * theta^(-2i/dh) for i < dh/2; pos may be a vector."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv = theta ** (-2.0 * i / head_dim)
    return np.multiply.outer(np.asarray(pos, dtype=np.float64), inv)


def rope(u: np.ndarray, ang: np.ndarray) -> np.ndarray:
    """Rotate pairs (u_i, u_{i+dh/2}) by ang_i.  u: [..., heads, dh]; ang: [..., dh/2]."""
    half = u.shape[-1] // 2
    c = np.cos(ang)[..., None, :]
    s = np.sin(ang)[..., None, :]
    u1, u2 = u[..., :half], u[..., half:]
    return np.concatenate([u1 * c - u2 * s, u2 * c + u1 * s], axis=-1)


def softmax(s: np.ndarray) -> np.ndarray:
    e = np.exp(s - np.max(s, axis=-1, keepdims=True))
    return e / np.sum(e, axis=-1, keepdims=True)


def attend_one(q: np.ndarray, K: np.ndarray, V: np.ndarray, group: int) -> np.ndarray:
    """One query position against cached positions.  q [nq, dh]; K, V [T, nkv, dh]."""
    nq, dh = q.shape
    out = np.empty_like(q)
    for j in range(nq):
        kv = j // group
        s = K[:, kv, :] @ q[j] / math.sqrt(dh)
        out[j] = softmax(s) @ V[:, kv, :]
    return out


def silu(x):
    return x / (1.0 + np.exp(-x))


def gelu_tanh(x):
    return 0.5 * x * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (x + 0.044715 * x ** 3)))


ACTS = {"swiglu": silu, "geglu": gelu_tanh}


def mlp(h, wg, wu, wd, act: str):
    return (ACTS[act](h @ wg.T) * (h @ wu.T)) @ wd.T


# ---------------------------------------------------------------- weights
def _f64(bits: np.ndarray) -> np.ndarray:
    return f32_from_bf16_bits(bits).astype(np.float64)


class Fp64Model:
    """Exact fp64 view of a ``seeded_inputs.ModelWeights``.

    ``cache=True`` keeps widened matrices (small models); otherwise every
    access widens the stored bf16 / int4 data again.
    """

    def __init__(self, weights, cache: bool = True):
        self.w = weights
        self.cfg = weights.cfg
        self.cache = cache
        self._memo = {}

    def _get(self, key, make):
        if not self.cache:
            return make()
        if key not in self._memo:
            self._memo[key] = make()
        return self._memo[key]

    def linear(self, layer: int, name: str) -> np.ndarray:
        def make():
            L = self.w.layers[layer]
            if self.cfg.weight_fmt == "int4":
                q = L[name].astype(np.float64)
                s = _f64(L[name + "_s"])
                o, i = q.shape
                return (q.reshape(o, i // 64, 64) * s[:, :, None]).reshape(o, i)
            return _f64(L[name])
        return self._get((layer, name), make)

    def gain(self, layer: int, name: str) -> np.ndarray:
        if name == "g_final":
            return self._get(("g_final",), lambda: _f64(self.w.g_final))
        return self._get((layer, name), lambda: _f64(self.w.layers[layer][name]))

    def embed_rows(self, ids) -> np.ndarray:
        return _f64(self.w.embed[np.asarray(ids)])

    def lm_head(self, h: np.ndarray, chunk: int = 16384) -> np.ndarray:
        """Logits E h for h [..., d] (tied head), widened chunk by chunk."""
        if self.cache:
            E = self._get(("embed",), lambda: _f64(self.w.embed))
            return h @ E.T
        V = self.cfg.vocab
        out = np.empty(h.shape[:-1] + (V,), dtype=np.float64)
        for lo in range(0, V, chunk):
            out[..., lo:lo + chunk] = h @ _f64(self.w.embed[lo:lo + chunk]).T
        return out


# ---------------------------------------------------------------- decoders
class TokenDecoder:
    """Per-token decoder: one position per call, KV cache of fp64 arrays."""

    def __init__(self, model: Fp64Model):
        c = model.cfg
        self.m = model
        self.cfg = c
        self.K = [np.zeros((0, c.n_kv_heads, c.head_dim)) for _ in range(c.n_layers)]
        self.V = [np.zeros((0, c.n_kv_heads, c.head_dim)) for _ in range(c.n_layers)]
        self.tokens: list[int] = []

    @property
    def length(self) -> int:
        return len(self.tokens)

    def decode(self, token: int) -> np.ndarray:
        """Append ``token`` at position ``length``; return fp64 logits for the next id."""
        c, m = self.cfg, self.m
        pos = self.length
        ang = rope_angles(pos, c.head_dim, c.rope_theta)
        x = m.embed_rows([token])[0]
        for l in range(c.n_layers):
            h = rmsnorm(x, m.gain(l, "g_attn"), c.rms_eps)
            q = (m.linear(l, "wq") @ h).reshape(c.n_q_heads, c.head_dim)
            k = (m.linear(l, "wk") @ h).reshape(c.n_kv_heads, c.head_dim)
            v = (m.linear(l, "wv") @ h).reshape(c.n_kv_heads, c.head_dim)
            q, k = rope(q, ang), rope(k, ang)
            self.K[l] = np.concatenate([self.K[l], k[None]], axis=0)
            self.V[l] = np.concatenate([self.V[l], v[None]], axis=0)
            o = attend_one(q, self.K[l], self.V[l], c.group)
            x = x + m.linear(l, "wo") @ o.reshape(-1)
            h = rmsnorm(x, m.gain(l, "g_mlp"), c.rms_eps)
            x = x + mlp(h, m.linear(l, "wg"), m.linear(l, "wu"), m.linear(l, "wd"), c.act)
        self.tokens.append(int(token))
        return m.lm_head(rmsnorm(x, m.gain(0, "g_final"), c.rms_eps))

    def truncate(self, new_len: int) -> None:
        """Forget every position >= new_len (rollback to a committed prefix)."""
        assert 0 <= new_len <= self.length
        for l in range(self.cfg.n_layers):
            self.K[l] = self.K[l][:new_len]
            self.V[l] = self.V[l][:new_len]
        del self.tokens[new_len:]

    def state(self):
        """A copy of everything the cache holds (for exact-restoration checks)."""
        return (list(self.tokens), [k.copy() for k in self.K], [v.copy() for v in self.V])


def forward_cacheless(model: Fp64Model, tokens, positions=None) -> np.ndarray:
    """Recompute the whole causal forward over ``tokens`` with no cache.

    Returns fp64 logits ``[len(positions), V]`` for the requested positions
    (default: every position); row p scores the id after tokens[0..p].
    """
    c, m = model.cfg, model
    T = len(tokens)
    ang = rope_angles(np.arange(T), c.head_dim, c.rope_theta)
    x = m.embed_rows(tokens)
    causal = np.tril(np.ones((T, T), dtype=bool))
    for l in range(c.n_layers):
        h = rmsnorm(x, m.gain(l, "g_attn"), c.rms_eps)
        q = (h @ m.linear(l, "wq").T).reshape(T, c.n_q_heads, c.head_dim)
        k = (h @ m.linear(l, "wk").T).reshape(T, c.n_kv_heads, c.head_dim)
        v = (h @ m.linear(l, "wv").T).reshape(T, c.n_kv_heads, c.head_dim)
        q, k = rope(q, ang), rope(k, ang)
        o = np.empty_like(q)
        for j in range(c.n_q_heads):
            kv = j // c.group
            s = (q[:, j, :] @ k[:, kv, :].T) / math.sqrt(c.head_dim)
            s = np.where(causal, s, -np.inf)
            o[:, j, :] = softmax(s) @ v[:, kv, :]
        x = x + o.reshape(T, -1) @ m.linear(l, "wo").T
        h = rmsnorm(x, m.gain(l, "g_mlp"), c.rms_eps)
        x = x + mlp(h, m.linear(l, "wg"), m.linear(l, "wu"), m.linear(l, "wd"), c.act)
    if positions is None:
        positions = np.arange(T)
    hf = rmsnorm(x[np.asarray(positions)], m.gain(0, "g_final"), c.rms_eps)
    return m.lm_head(hf)
