"""Algorithmic work of each call: the bytes and flops the method must move or
compute, independent of how a kernel does it (workspace traffic and masked
tile waste are not counted).

* Attention scores per call: a chunk of T queries at offset s against s + T
  keys computes H * T * (s + T) scores when the whole rectangle is evaluated
  (the work counter of "kv-cache-decoding", "Prefill and decode" and its
  correctness tests), of which H * (T*s + T*(T+1)/2) are visible under the
  bottom-right causal mask ("KV cache, incremental decode, ...", section 2.3).
* Flops: 2*d_h for q.k and 2*d_h for p*v per visible pair and query head.
* Bytes: K and V of every visible position of every KV head read once, q read
  once, the float32 output written once; append reads its input and writes
  the storage dtype.
"""
from __future__ import annotations

from typing import Iterable

ITEMSIZE = {"fp32": 4, "fp16": 2, "bf16": 2}


def rectangle_scores(n_heads: int, T: int, s: int) -> int:
    return n_heads * T * (s + T)


def visible_pairs(T: int, s: int) -> int:
    return T * s + T * (T + 1) // 2


def attend_flops(offsets: Iterable[int], T: int, n_q_heads: int, d_head: int) -> int:
    """4 * d_h * H_q * visible pairs, summed over rows with query offsets s_b."""
    return sum(4 * d_head * n_q_heads * visible_pairs(T, int(s)) for s in offsets)


def attend_bytes(offsets: Iterable[int], T: int, n_q_heads: int, n_kv_heads: int, d_head: int,
                 dtype: str, q_dtype: str) -> int:
    """K+V of the s_b + T cached positions per row and KV head, plus q in and fp32 out."""
    offs = [int(s) for s in offsets]
    kv = sum((s + T) for s in offs) * n_kv_heads * d_head * ITEMSIZE[dtype] * 2
    B = len(offs)
    q = B * n_q_heads * T * d_head * ITEMSIZE[q_dtype]
    out = B * n_q_heads * T * d_head * 4
    return kv + q + out


def append_bytes(batch: int, n_kv_heads: int, T: int, d_head: int, in_dtype: str, dtype: str) -> int:
    """k and v: read in_dtype, write the storage dtype."""
    return batch * n_kv_heads * T * d_head * (ITEMSIZE[in_dtype] + ITEMSIZE[dtype]) * 2
