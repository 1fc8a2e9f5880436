"""A small random-weight decoder-only model whose attention runs through the
C ABI: the workload "kv-cache-decoding" builds (task statement, steps 1-10),
on the GPU.

The dense parts (embedding rows, layer norm, projections, MLP) are float32
torch operations on the device: plumbing around the cache. Every layer's keys
and values go into an fp32 `KVCache` and every attention is the library's
(`kvc_append_attend`: a decode step's append and attention in one launch, a
longer chunk as append then attend). The structure follows the page's steps:
one call for a whole-sequence pass, a prefill or a decode step; new rows take
position rows from the cache length; the cache commits once per call, after
the last layer (the library's committed length is the minimum of the layers'
fills). The counters are the page's: positions processed and attention
scores, m x (t + m) per head and layer.
"""
from __future__ import annotations

from typing import Optional

from .kvc import KVCache

LAYER_NORM_EPS = 1e-5


class GpuDecoder:
    """params: a workloads.DecoderParams; shape: its workloads.DecoderShape."""

    def __init__(self, params, shape, device="cuda"):
        import torch
        self.shape = shape
        self.device = torch.device(device)
        dev = lambda a: torch.as_tensor(a, dtype=torch.float32).to(self.device)  # noqa: E731
        self.token_rows, self.position_rows = dev(params.token_rows), dev(params.position_rows)
        self.blocks = [{name: dev(getattr(b, name)) for name in
                        ("attn_gain", "attn_shift", "qkv", "merge", "mlp_gain", "mlp_shift", "expand", "contract")}
                       for b in params.blocks]
        self.out_gain, self.out_shift, self.readout = dev(params.out_gain), dev(params.out_shift), dev(params.readout)
        self.positions_processed = 0
        self.scores_computed = 0
        self._scratch: Optional[KVCache] = None     # the cache of calls without one

    def new_cache(self) -> KVCache:
        s = self.shape
        return KVCache(s.layers, s.heads, s.head_width, s.positions, batch=1, n_q_heads=s.heads, dtype="fp32",
                       device=self.device)

    def _norm(self, x, gain, shift):
        import torch
        return torch.nn.functional.layer_norm(x, (x.shape[-1],), gain, shift, LAYER_NORM_EPS)

    def _heads(self, x):
        """[m, width] -> [1, heads, m, head_width], contiguous."""
        m = x.shape[0]
        return x.reshape(m, self.shape.heads, self.shape.head_width).transpose(0, 1).unsqueeze(0).contiguous()

    def step(self, token_ids, cache: Optional[KVCache] = None):
        """Logits [m, vocab] (float32, on the device) of the m new tokens; their
        keys and values go into `cache` (into an emptied scratch cache when
        None, so a whole-sequence pass is the same call with t = 0)."""
        import torch
        if cache is None:
            if self._scratch is None:
                self._scratch = self.new_cache()
            cache = self._scratch
            cache.truncate(0)
        ids = torch.as_tensor(list(token_ids), dtype=torch.long, device=self.device)
        m, w = ids.numel(), self.shape.width
        t = int(cache.seq_len()[0])
        rows = self.token_rows[ids] + self.position_rows[t:t + m]
        for layer, blk in enumerate(self.blocks):
            qkv = self._norm(rows, blk["attn_gain"], blk["attn_shift"]) @ blk["qkv"]
            q, k, v = (self._heads(qkv[:, i * w:(i + 1) * w]) for i in range(3))
            ctx = cache.append_attend(layer, k, v, q)[0]             # [heads, m, head_width]
            rows = rows + ctx.transpose(0, 1).reshape(m, w) @ blk["merge"]
            hidden = self._norm(rows, blk["mlp_gain"], blk["mlp_shift"]) @ blk["expand"]
            rows = rows + torch.relu(hidden) @ blk["contract"]
            self.scores_computed += self.shape.heads * m * (t + m)
        self.positions_processed += m
        return self._norm(rows, self.out_gain, self.out_shift) @ self.readout

    def close(self) -> None:
        if self._scratch is not None:
            self._scratch.close()
            self._scratch = None


def greedy_uncached(model: GpuDecoder, prompt, n_new: int):
    """n_new greedy tokens, each step a pass over the whole sequence so far.
    Returns (ids, [n_new, vocab] step logits on the device)."""
    import torch
    seq, per_step = list(prompt), []
    for _ in range(n_new):
        last = model.step(seq)[-1]
        per_step.append(last)
        seq.append(int(torch.argmax(last)))
    return seq, torch.stack(per_step)


def greedy_cached(model: GpuDecoder, prompt, n_new: int):
    """n_new greedy tokens over one cache: prefill, then one call per step
    feeding only the token just chosen. Returns (ids, step logits, cache)."""
    import torch
    cache = model.new_cache()
    seq, feed, per_step = list(prompt), list(prompt), []
    for _ in range(n_new):
        last = model.step(feed, cache)[-1]
        per_step.append(last)
        chosen = int(torch.argmax(last))
        seq.append(chosen)
        feed = [chosen]
    return seq, torch.stack(per_step), cache
