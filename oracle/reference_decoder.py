"""A float64 reference of a small random-weight decoder-only model that keeps
its keys and values in the oracle cache.

TEST INFRASTRUCTURE. Only tests/ may import or run this module; the product
path never does.

"kv-cache-decoding" (task statement, its ten steps and its shapes table) asks
for one model call that serves a whole-sequence pass, a prefill and a decode
step alike. In this file's terms, `ReferenceDecoder.step(token_ids, cache)`:

* takes t = the positions the cache already holds (0 without a cache) and
  m = the new tokens (step 1);
* forms each new row as its token's row plus position row t + i: a new token's
  position is the cache length (step 2);
* in every layer normalises the rows and projects them to queries, keys and
  values (step 4), appends the keys and values at slots t .. t+m-1 and attends
  over all t+m held positions, row i seeing columns 0 .. t+i (steps 3, 5, 6),
  merges the heads, projects and adds the result to the rows; then normalises
  again and adds the MLP's output (step 6);
* commits t + m once, after the last layer (step 7): the oracle cache's
  committed length is the minimum of its layers' fills, so it moves only when
  the last layer has appended;
* counts positions processed and attention scores, m x (t + m) per head and
  layer (step 10);
* returns logits for the m new positions.

Readings where the page is silent: layer norm uses eps 1e-5 and a gain and a
shift per feature; the MLP expands to mlp_ratio x width, applies ReLU and
contracts back; projections carry no bias; the cache stores float32 values
(the GPU model's storage), so the queries the attention uses are float32
too; a call without a cache runs over a fresh, empty cache (t = 0), so the
cached and the uncached path store the same float32 keys and values and
differ only in the order of float64 additions.
"""
from __future__ import annotations

import numpy as np

from .kvc_oracle import OracleCache

LAYER_NORM_EPS = 1e-5


def layer_norm(x: np.ndarray, gain: np.ndarray, shift: np.ndarray) -> np.ndarray:
    """Per row: subtract the mean, divide by sqrt(variance + eps), then scale
    and shift per feature."""
    centred = x - x.mean(axis=-1, keepdims=True)
    spread = np.sqrt((centred * centred).mean(axis=-1, keepdims=True) + LAYER_NORM_EPS)
    return centred / spread * gain + shift


class ReferenceDecoder:
    """The model in float64 NumPy over an `OracleCache` of float32 storage.

    params: a workloads.DecoderParams (float32 arrays, promoted here);
    shape: its workloads.DecoderShape. With restart_positions, every call takes
    position rows from 0 instead of the cache length: the page's pitfall
    "Position restarts at 0", planted for a test that must catch it.
    """

    def __init__(self, params, shape, *, restart_positions: bool = False):
        f64 = lambda a: np.asarray(a, dtype=np.float64)  # noqa: E731
        self.shape = shape
        self.token_rows = f64(params.token_rows)
        self.position_rows = f64(params.position_rows)
        self.blocks = [{name: f64(getattr(b, name)) for name in
                        ("attn_gain", "attn_shift", "qkv", "merge", "mlp_gain", "mlp_shift", "expand", "contract")}
                       for b in params.blocks]
        self.out_gain, self.out_shift = f64(params.out_gain), f64(params.out_shift)
        self.readout = f64(params.readout)
        self.restart_positions = restart_positions
        self.positions_processed = 0
        self.scores_computed = 0

    def empty_cache(self) -> OracleCache:
        s = self.shape
        return OracleCache(s.layers, 1, s.heads, s.heads, s.head_width, s.positions, "fp32")

    def _heads(self, x: np.ndarray) -> np.ndarray:
        """[m, width] -> [1, heads, m, head_width] float32 (the cache's batch of one)."""
        m = x.shape[0]
        return x.reshape(m, self.shape.heads, self.shape.head_width).transpose(1, 0, 2)[None].astype(np.float32)

    def step(self, token_ids, cache: OracleCache | None = None) -> np.ndarray:
        """Logits [m, vocab] of the m new tokens; their keys and values are
        appended to `cache` (to a fresh cache when None)."""
        ids = np.asarray(list(token_ids), dtype=np.int64)
        m, w = len(ids), self.shape.width
        if cache is None:
            cache = self.empty_cache()
        t = int(cache.seq_len()[0])
        first = 0 if self.restart_positions else t
        rows = self.token_rows[ids] + self.position_rows[first:first + m]
        for layer, blk in enumerate(self.blocks):
            qkv = layer_norm(rows, blk["attn_gain"], blk["attn_shift"]) @ blk["qkv"]
            q, k, v = (self._heads(qkv[:, i * w:(i + 1) * w]) for i in range(3))
            cache.append(layer, k, v)
            ctx = cache.attend(layer, q)[0]                        # [heads, m, head_width] float64
            rows = rows + ctx.transpose(1, 0, 2).reshape(m, w) @ blk["merge"]
            hidden = layer_norm(rows, blk["mlp_gain"], blk["mlp_shift"]) @ blk["expand"]
            rows = rows + np.maximum(hidden, 0.0) @ blk["contract"]
            self.scores_computed += self.shape.heads * m * (t + m)
        self.positions_processed += m
        return layer_norm(rows, self.out_gain, self.out_shift) @ self.readout


def greedy_uncached(model: ReferenceDecoder, prompt, n_new: int):
    """n_new greedy tokens, every step a pass over the whole sequence so far
    (step 8). Returns (prompt + new ids, [n_new, vocab] logits of each step)."""
    seq = list(prompt)
    per_step = []
    for _ in range(n_new):
        last = model.step(seq)[-1]
        per_step.append(last)
        seq.append(int(np.argmax(last)))
    return seq, np.stack(per_step)


def greedy_cached(model: ReferenceDecoder, prompt, n_new: int):
    """n_new greedy tokens over one cache: a prefill of the prompt, then one
    call per step that feeds only the token just chosen (step 9); the last
    chosen token is never fed, so the cache ends at P + n_new - 1 positions.
    Returns (ids, [n_new, vocab] step logits, the cache)."""
    cache = model.empty_cache()
    seq, feed, per_step = list(prompt), list(prompt), []
    for _ in range(n_new):
        last = model.step(feed, cache)[-1]
        per_step.append(last)
        chosen = int(np.argmax(last))
        seq.append(chosen)
        feed = [chosen]
    return seq, np.stack(per_step), cache
