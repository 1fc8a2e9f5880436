"""Seeded synthetic workloads: shapes, random draws and call sequences.

This module only draws numbers and lists calls. It holds none of the method's
arithmetic, so both the HIP path and the CPU oracle can consume the same
inputs from it without sharing code.

Every array is drawn with numpy's default_rng(seed) as float32 N(0, 1)
(scaled by 0.5 for the SmolLM2-shaped cache) in the order documented on each
script: per call, q then k then v; the batched-decode lengths and the
speculative rollback counts are drawn where the script says.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Iterator, Optional  # noqa: F401

import numpy as np


@dataclass(frozen=True)
class CacheShape:
    name: str
    n_layers: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    d_head: int
    max_len: int
    dtype: str           # storage dtype: "fp32" | "fp16" | "bf16"
    scale: float = 1.0   # multiplier applied to every N(0, 1) draw (in float32)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


SHAPES = {
    # B=1, L=4, H_q=4, H_kv=2, d_h=32, max_len=128, fp32: prefill 16 then 112 decode steps.
    "tiny_gqa_fp32": CacheShape("tiny_gqa_fp32", 4, 1, 4, 2, 32, 128, "fp32"),
    # SmolLM2-135M-shaped: L=30, H_q=9, H_kv=3, d_h=64, fp16; max_len 2048.
    "smollm2_135m_fp16": CacheShape("smollm2_135m_fp16", 30, 1, 9, 3, 64, 2048, "fp16", 0.5),
    # One Llama-3-8B-shaped layer, batched decode: B=32, H_q=32, H_kv=8, d_h=128, bf16.
    "llama3_8b_layer_decode_bf16": CacheShape("llama3_8b_layer_decode_bf16", 1, 32, 32, 8, 128, 4096, "bf16"),
    # Chunked prefill: B=4, H_q=32, H_kv=8, d_h=128, max_len 16384, chunks of 512.
    "chunked_prefill_bf16": CacheShape("chunked_prefill_bf16", 1, 4, 32, 8, 128, 16384, "bf16"),
    # Long-context decode with speculative rollback: B=8, H_q=64, H_kv=8, s0=32768.
    "long_ctx_spec_bf16": CacheShape("long_ctx_spec_bf16", 1, 8, 64, 8, 128, 32776, "bf16"),
}


@dataclass
class Call:
    """One step of a call script.

    op = "pass":     append(layer, k, v) then attend(layer, q) with the same T.
    op = "append":   append(layer, k, v) only (used to preload a cache).
    op = "truncate": truncate to n (int64 [B]).
    """
    op: str
    layer: int = 0
    T: int = 0
    q: Optional[np.ndarray] = None
    k: Optional[np.ndarray] = None
    v: Optional[np.ndarray] = None
    n: Optional[np.ndarray] = None
    tag: str = ""
    meta: dict = field(default_factory=dict)


def _normal(rng: np.random.Generator, shape, scale: float) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


def draw_qkv(rng: np.random.Generator, shape: CacheShape, T: int):
    """q [B, H_q, T, d_h], then k and v [B, H_kv, T, d_h], in that draw order."""
    q = _normal(rng, (shape.batch, shape.n_q_heads, T, shape.d_head), shape.scale)
    k = _normal(rng, (shape.batch, shape.n_kv_heads, T, shape.d_head), shape.scale)
    v = _normal(rng, (shape.batch, shape.n_kv_heads, T, shape.d_head), shape.scale)
    return q, k, v


def draw_kv(rng: np.random.Generator, shape: CacheShape, T: int):
    """k then v [B, H_kv, T, d_h] (a preload chunk has no queries)."""
    k = _normal(rng, (shape.batch, shape.n_kv_heads, T, shape.d_head), shape.scale)
    v = _normal(rng, (shape.batch, shape.n_kv_heads, T, shape.d_head), shape.scale)
    return k, v


def _passes(rng, shape: CacheShape, T: int, tag: str) -> Iterator[Call]:
    for layer in range(shape.n_layers):
        q, k, v = draw_qkv(rng, shape, T)
        yield Call("pass", layer, T, q, k, v, tag=tag)


def script_tiny_gqa(seed: int = 0, n_decode: int = 112, prefill: int = 16):
    """Prefill T=16 at s=0 over all layers, then n_decode steps of T=1."""
    shape = SHAPES["tiny_gqa_fp32"]

    def calls():
        rng = np.random.default_rng(seed)
        yield from _passes(rng, shape, prefill, "prefill")
        for step in range(n_decode):
            yield from _passes(rng, shape, 1, f"decode{step}")
    return shape, calls()


def script_smollm2(seed: int = 0, prefill: int = 512, n_decode: int = 256,
                   rollback: int = 4, n_layers: Optional[int] = None):
    """Prefill T=512, n_decode steps of T=1, truncate back `rollback`
    positions, then `rollback` fresh T=1 re-decode steps. n_layers can shrink
    the stack for quick runs (the shape otherwise stays SmolLM2's)."""
    shape = SHAPES["smollm2_135m_fp16"]
    if n_layers is not None:
        shape = CacheShape(shape.name, n_layers, shape.batch, shape.n_q_heads, shape.n_kv_heads,
                           shape.d_head, shape.max_len, shape.dtype, shape.scale)

    def calls():
        rng = np.random.default_rng(seed)
        yield from _passes(rng, shape, prefill, "prefill")
        for step in range(n_decode):
            yield from _passes(rng, shape, 1, f"decode{step}")
        s = prefill + n_decode
        yield Call("truncate", n=np.full(shape.batch, s - rollback, dtype=np.int64), tag="rollback")
        for step in range(rollback):
            yield from _passes(rng, shape, 1, f"redecode{step}")
    return shape, calls()


def batched_lengths(rng: np.random.Generator, batch: int, lo: int = 1024, hi: int = 4095) -> np.ndarray:
    """Per-row committed lengths drawn uniformly from {lo, ..., hi}."""
    return rng.integers(lo, hi + 1, size=batch, dtype=np.int64)


def script_batched_decode(seed: int = 0, n_steps: int = 1, batch: Optional[int] = None,
                          max_len: Optional[int] = None):
    """Lengths first, then a preload chunk of max_len-1 positions (k then v),
    then a per-row truncate to the drawn lengths, then n_steps of T=1.
    `batch` and `max_len` can shrink the case for quick runs."""
    base = SHAPES["llama3_8b_layer_decode_bf16"]
    shape = CacheShape(base.name, base.n_layers, batch or base.batch, base.n_q_heads,
                       base.n_kv_heads, base.d_head, max_len or base.max_len, base.dtype)

    def calls():
        rng = np.random.default_rng(seed)
        hi = shape.max_len - 1
        lo = 1024 if max_len is None else max(1, hi // 4)
        lengths = batched_lengths(rng, shape.batch, lo, hi)
        k, v = draw_kv(rng, shape, hi)
        yield Call("append", 0, hi, None, k, v, tag="preload")
        del k, v
        yield Call("truncate", n=lengths, tag="lengths")
        for step in range(n_steps):
            yield from _passes(rng, shape, 1, f"decode{step}")
    return shape, calls()


def script_chunked_prefill(seed: int = 0, chunk: int = 512, n_chunks: int = 32,
                           batch: Optional[int] = None):
    """Chunks of T=chunk appended at s = 0, chunk, 2*chunk, ..."""
    base = SHAPES["chunked_prefill_bf16"]
    shape = CacheShape(base.name, base.n_layers, batch or base.batch, base.n_q_heads,
                       base.n_kv_heads, base.d_head, chunk * n_chunks, base.dtype)

    def calls():
        rng = np.random.default_rng(seed)
        for c in range(n_chunks):
            q, k, v = draw_qkv(rng, shape, chunk)
            yield Call("pass", 0, chunk, q, k, v, tag=f"chunk{c}")
    return shape, calls()


def script_long_ctx_spec(seed: int = 0, n_cycles: int = 64, s0: int = 32768, draft: int = 4,
                         batch: Optional[int] = None):
    """Preload s0 positions (k then v); then per cycle: draw r in {0..draft},
    draw and run a T=draft pass, truncate to s0+draft-r, run (draft-r) T=1
    passes (one per accepted position), and truncate back to s0."""
    base = SHAPES["long_ctx_spec_bf16"]
    shape = CacheShape(base.name, base.n_layers, batch or base.batch, base.n_q_heads,
                       base.n_kv_heads, base.d_head, s0 + 2 * draft, base.dtype)

    def calls():
        rng = np.random.default_rng(seed)
        k, v = draw_kv(rng, shape, s0)
        yield Call("append", 0, s0, None, k, v, tag="preload")
        del k, v
        B = shape.batch
        for c in range(n_cycles):
            r = int(rng.integers(0, draft + 1))
            q, k, v = draw_qkv(rng, shape, draft)
            yield Call("pass", 0, draft, q, k, v, tag=f"draft{c}", meta={"r": r})
            yield Call("truncate", n=np.full(B, s0 + draft - r, dtype=np.int64), tag=f"accept{c}")
            for a in range(draft - r):
                q, k, v = draw_qkv(rng, shape, 1)
                yield Call("pass", 0, 1, q, k, v, tag=f"decode{c}.{a}")
            yield Call("truncate", n=np.full(B, s0, dtype=np.int64), tag=f"reset{c}")
    return shape, calls()


# ---- a random-weight decoder-only model ("kv-cache-decoding": the task
#      statement (vocab 96, width 128, 4 heads, 4 layers, 256 positions, learned
#      position rows) and "Correctness tests" (a 48-token prompt, 160 greedy
#      steps)). Only the shapes and the random draw live here; the model's
#      arithmetic is in its float64 twin (oracle/) and its GPU version. -------

@dataclass(frozen=True)
class DecoderShape:
    vocab: int = 96
    width: int = 128
    heads: int = 4
    layers: int = 4
    positions: int = 256
    mlp_ratio: int = 4

    @property
    def head_width(self) -> int:
        return self.width // self.heads


@dataclass
class BlockParams:
    """One layer: pre-attention norm (gain, shift), the fused query/key/value
    projection [width, 3 width] (columns: queries, keys, values, each head's
    slice contiguous), the head-merge projection [width, width], the pre-MLP
    norm, and the MLP's expand [width, r width] and contract [r width, width]."""
    attn_gain: np.ndarray
    attn_shift: np.ndarray
    qkv: np.ndarray
    merge: np.ndarray
    mlp_gain: np.ndarray
    mlp_shift: np.ndarray
    expand: np.ndarray
    contract: np.ndarray


@dataclass
class DecoderParams:
    token_rows: np.ndarray      # [vocab, width]
    position_rows: np.ndarray   # [positions, width]
    blocks: list
    out_gain: np.ndarray
    out_shift: np.ndarray
    readout: np.ndarray         # [width, vocab]


def decoder_params(seed: int = 0, shape: DecoderShape = DecoderShape()) -> DecoderParams:
    """Random float32 parameters: the readout and both tables first, then each
    layer's matrices in the order qkv, merge, expand, contract. Tables are
    N(0, 1); a matrix with `fan_in` input rows is N(0, 1/fan_in), which keeps
    activations at unit scale through the stack; norm gains 1, shifts 0."""
    rng = np.random.default_rng(seed)
    w, r = shape.width, shape.mlp_ratio

    def matrix(fan_in, fan_out):
        return _normal(rng, (fan_in, fan_out), float(1.0 / np.sqrt(fan_in)))

    readout = matrix(w, shape.vocab)
    tokens = _normal(rng, (shape.vocab, w), 1.0)
    positions = _normal(rng, (shape.positions, w), 1.0)
    ones, zeros = np.ones(w, np.float32), np.zeros(w, np.float32)
    blocks = []
    for _ in range(shape.layers):
        qkv, merge = matrix(w, 3 * w), matrix(w, w)
        expand, contract = matrix(w, r * w), matrix(r * w, w)
        blocks.append(BlockParams(ones.copy(), zeros.copy(), qkv, merge, ones.copy(), zeros.copy(), expand, contract))
    return DecoderParams(tokens, positions, blocks, ones.copy(), zeros.copy(), readout)


def decoder_prompt(seed: int = 1, length: int = 48, shape: DecoderShape = DecoderShape()) -> list:
    """A prompt of `length` token ids drawn uniformly from the vocabulary."""
    return [int(x) for x in np.random.default_rng(seed).integers(0, shape.vocab, size=length)]
