"""A tiny decoder-only transformer in float64 NumPy over the oracle cache.

Test infrastructure only, like the rest of this package: it is the reference
that the GPU model of the same weights is compared with, and it pins itself
against the figures of "kv-cache-decoding" (the benchmark spec's steps and
"Correctness tests").

The model is the one that page describes: token embedding plus the position
row of each token's absolute position; per layer a pre-norm block (layer norm,
bias-free q/k/v projections split into heads, causal attention over every key
the cache holds, output projection added to the residual) and a pre-norm MLP
(d -> 4d, ReLU, 4d -> d); a final layer norm and the vocabulary projection.
Attention goes through OracleCache (fp32 storage): with a cache, the m new
tokens' keys and values are appended at slots [t, t + m) and their queries
attend to all t + m keys (the mask offset is t); without one, a fresh cache
takes the whole sequence at t = 0. The cache's length moves once per call,
after the last layer.

Work counters (same page, "Correctness tests"): `positions` counts token
positions pushed through the stack, `scores` the attention scores computed
(layers x heads x m x (t + m) per call).
"""
from __future__ import annotations

import numpy as np

from .kvc_oracle import OracleCache


def layer_norm(x: np.ndarray, gain: np.ndarray, bias: np.ndarray, eps: float = 1e-5) -> np.ndarray:
    """Each position normalised on its own (mean 0, variance 1), then scaled."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return gain * (x - mu) / np.sqrt(var + eps) + bias


class OracleTinyDecoder:
    def __init__(self, weights: dict, spec, position_bug: bool = False):
        """`weights` as drawn by workloads.tiny_decoder_weights (float32 arrays,
        used here as float64). position_bug=True plants the classic mistake of
        a decode step taking position row 0 (for tests that must catch it)."""
        self.spec = spec
        f64 = lambda a: np.asarray(a, dtype=np.float64)  # noqa: E731
        self.tok_emb = f64(weights["tok_emb"])
        self.pos_emb = f64(weights["pos_emb"])
        self.layers = [{k: f64(v) for k, v in lw.items()} for lw in weights["layers"]]
        self.g_out, self.b_out, self.w_out = f64(weights["g_out"]), f64(weights["b_out"]), f64(weights["w_out"])
        self.position_bug = position_bug
        self.positions = 0
        self.scores = 0

    def new_cache(self) -> OracleCache:
        s = self.spec
        return OracleCache(s.n_layers, 1, s.n_heads, s.n_heads, s.d_head, s.max_len, "fp32")

    def _heads(self, x: np.ndarray) -> np.ndarray:
        """(m, d_model) -> (1, heads, m, d_head)."""
        m = x.shape[0]
        return x.reshape(m, self.spec.n_heads, self.spec.d_head).transpose(1, 0, 2)[None]

    def forward(self, ids, cache: OracleCache | None = None) -> np.ndarray:
        """Logits (m, vocab) of the m tokens `ids`, placed after the t tokens
        the cache holds (t = 0 without a cache)."""
        s = self.spec
        t = 0 if cache is None else int(cache.seq_len()[0])
        m = len(ids)
        if m < 1 or t + m > s.max_len:
            raise ValueError("need 1 <= m and t + m <= max_len")
        if cache is None:
            cache = self.new_cache()
        p0 = 0 if (self.position_bug and t > 0) else t
        x = self.tok_emb[np.asarray(ids)] + self.pos_emb[p0:p0 + m]
        for layer, p in enumerate(self.layers):
            h = layer_norm(x, p["g1"], p["b1"])
            q, k, v = self._heads(h @ p["w_q"]), self._heads(h @ p["w_k"]), self._heads(h @ p["w_v"])
            cache.append(layer, k, v)
            att = cache.attend(layer, q)[0]                   # (heads, m, d_head)
            x = x + att.transpose(1, 0, 2).reshape(m, s.d_model) @ p["w_o"]
            h = layer_norm(x, p["g2"], p["b2"])
            x = x + np.maximum(h @ p["w_1"], 0.0) @ p["w_2"]
            self.scores += s.n_heads * m * (t + m)
        self.positions += m
        return layer_norm(x, self.g_out, self.b_out) @ self.w_out


def generate_no_cache(model: OracleTinyDecoder, prompt, n_new: int):
    """Greedy: the whole sequence through the model at every step."""
    ids, step_logits = list(prompt), []
    for _ in range(n_new):
        logits = model.forward(ids)[-1]
        step_logits.append(logits)
        ids.append(int(np.argmax(logits)))
    return ids, np.array(step_logits)


def generate_with_cache(model: OracleTinyDecoder, prompt, n_new: int):
    """Greedy: one prefill pass over the prompt, then one token per step."""
    cache = model.new_cache()
    ids, step_logits = list(prompt), []
    new = list(prompt)
    for _ in range(n_new):
        logits = model.forward(new, cache)[-1]
        step_logits.append(logits)
        ids.append(int(np.argmax(logits)))
        new = [ids[-1]]
    return ids, np.array(step_logits), cache
