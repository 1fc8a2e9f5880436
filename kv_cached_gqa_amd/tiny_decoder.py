"""A tiny decoder-only transformer on the GPU whose attention runs through the
KV cache's C ABI ("kv-cache-decoding": the benchmark spec's steps 1-10 and
"Correctness tests"; the model is also the one "KV cache, incremental decode,
..." section 2 drives through its cache).

The dense parts (embeddings, layer norms, projections, MLP, vocabulary
projection) are plain float32 torch operations on the device: plumbing around
the cache. Every key and value goes into a `KVCache` (fp32 storage) with
`append_attend` at the model's own positions (the append, then the attention
over everything stored, in one call: one decode launch for a decode step), so
the cached path (one prefill call, then one token per call) and the uncached
path (the whole sequence at t = 0 each step, in a cache emptied with
`truncate(0)`) exercise append, the committed length, the bottom-right mask
and truncate end to end.

Model: token embedding plus the position row of each token's absolute
position (the cache's committed length t for the first new token); per layer a
pre-norm attention block (bias-free q/k/v/o projections, heads of d_model /
n_heads) and a pre-norm MLP (d -> 4d, ReLU, 4d -> d); a final layer norm and
the vocabulary projection. `positions` and `scores` count the work as the page
does: positions pushed through the stack, and layers x heads x m x (t + m)
attention scores per call.
"""
from __future__ import annotations

import numpy as np

from .kvc import KVCache


class TinyDecoder:
    def __init__(self, weights: dict, spec, device="cuda"):
        import torch
        self.torch = torch
        self.spec = spec
        self.device = torch.device(device)
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(self.device)  # noqa: E731
        self.tok_emb, self.pos_emb = t(weights["tok_emb"]), t(weights["pos_emb"])
        self.layers = [{k: t(v) for k, v in lw.items()} for lw in weights["layers"]]
        self.g_out, self.b_out, self.w_out = t(weights["g_out"]), t(weights["b_out"]), t(weights["w_out"])
        self.positions = 0
        self.scores = 0
        self._scratch = None             # the cache the uncached path reuses

    def new_cache(self) -> KVCache:
        s = self.spec
        return KVCache(s.n_layers, s.n_heads, s.d_head, s.max_len, batch=1, n_q_heads=s.n_heads, dtype="fp32",
                       device=self.device)

    def _heads(self, x):
        """(m, d_model) -> [1, heads, m, d_head], contiguous."""
        m = x.shape[0]
        return x.view(m, self.spec.n_heads, self.spec.d_head).permute(1, 0, 2).contiguous().unsqueeze(0)

    def forward(self, ids, cache: KVCache | None = None):
        """Logits (m, vocab), float32 on the device, of the m tokens `ids`
        placed after the t tokens the cache holds. Without a cache the whole
        sequence runs at t = 0 in an emptied scratch cache."""
        torch, s = self.torch, self.spec
        if cache is None:
            if self._scratch is None:
                self._scratch = self.new_cache()
            cache = self._scratch
            if int(cache.seq_len()[0]) > 0:
                cache.truncate(0)
        t = int(cache.seq_len()[0])
        m = len(ids)
        if m < 1 or t + m > s.max_len:
            raise ValueError("need 1 <= m and t + m <= max_len")
        F = torch.nn.functional
        idx = torch.as_tensor(ids, device=self.device, dtype=torch.long)
        x = self.tok_emb[idx] + self.pos_emb[t:t + m]
        for layer, p in enumerate(self.layers):
            h = F.layer_norm(x, (s.d_model,), p["g1"], p["b1"], 1e-5)
            q, k, v = self._heads(h @ p["w_q"]), self._heads(h @ p["w_k"]), self._heads(h @ p["w_v"])
            att = cache.append_attend(layer, k, v, q)[0]         # [heads, m, d_head] float32
            x = x + att.permute(1, 0, 2).reshape(m, s.d_model) @ p["w_o"]
            h = F.layer_norm(x, (s.d_model,), p["g2"], p["b2"], 1e-5)
            x = x + torch.relu(h @ p["w_1"]) @ p["w_2"]
            self.scores += s.n_heads * m * (t + m)
        self.positions += m
        return F.layer_norm(x, (s.d_model,), self.g_out, self.b_out, 1e-5) @ self.w_out

    def close(self) -> None:
        if self._scratch is not None:
            self._scratch.close()
            self._scratch = None


def generate_no_cache(model: TinyDecoder, prompt, n_new: int):
    """Greedy: the whole sequence through the model at every step. Returns the
    ids and the step logits [n_new, vocab] (float32, on the host)."""
    ids, step_logits = list(prompt), []
    for _ in range(n_new):
        logits = model.forward(ids)[-1]
        step_logits.append(logits)
        ids.append(int(model.torch.argmax(logits)))
    return ids, model.torch.stack(step_logits).cpu().numpy()


def generate_with_cache(model: TinyDecoder, prompt, n_new: int, cache: KVCache | None = None):
    """Greedy: one prefill call over the prompt, then one token per call."""
    cache = cache if cache is not None else model.new_cache()
    ids, step_logits = list(prompt), []
    new = list(prompt)
    for _ in range(n_new):
        logits = model.forward(new, cache)[-1]
        step_logits.append(logits)
        ids.append(int(model.torch.argmax(logits)))
        new = [ids[-1]]
    return ids, model.torch.stack(step_logits).cpu().numpy(), cache
