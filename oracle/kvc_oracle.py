"""Plain float64 CPU oracle for KV-cached grouped-query attention.

TEST INFRASTRUCTURE. Only tests/, the package smoke check and the CPU-baseline
leg of bench.py may import or run this module. It shares no code with the HIP
path (no kernels, headers, helpers or tables) and imports nothing from it.

What it computes, and where the pages define it:

* Storage. A preallocated cache of shape (L, B, H_kv, max_len, d_h) for K and
  for V, zero before anything is written ("kv-cache-decoding", shapes table:
  unfilled slots are zeros; "Generation and the KV Cache", the KVCache
  paragraph: k, v of shape (L, B, H, max_len, d_head)).
* Per-layer fill counts and the committed length s = min over layers
  ("KV cache, incremental decode, ...", section 2.3). Rows of a batch carry
  their own counts (the per-request length of "kv-cache-decoding",
  "Batching caches of different lengths").
* append: write a chunk of T positions at slots [fill, fill+T) after
  rounding to the storage dtype, and advance that layer's fill
  ("KV cache, ...", sections 2.5 and 4, update; "kv-cache-decoding", step 5).
  On any error nothing changes ("KV cache, ...", section 4 test table,
  test_update_copies_and_checks).
* attend: softmax(q K^T / sqrt(d_h)) V for every query head h of every row,
  over the keys that head's K/V head g = h // G holds, with query i of the
  chunk at absolute position s + i seeing keys j <= s + i
  ("KV cache, ...", section 2.3, the mask equation; "Heads, GQA and K/V
  cache", "Four queries, two sets of K/V": heads map in order [0,0,1,1];
  "kv-cache-decoding", shapes table: scores = q k^T / sqrt(d_head)).
  It is the definition written out: every call recomputes from storage,
  in float64, with masked keys excluded from the sum.
* truncate(n): every layer's fill becomes n; storage is untouched
  ("KV cache, ...", section 2.4).
* nbytes = 2 L B H_kv max_len d_h itemsize ("KV cache, ...", section 2.5;
  "Heads, GQA and K/V cache", "Memory and the window limit").
* append_rope / rope_rotate: keys stored after the rotary embedding at their
  absolute positions ("Generation and the KV Cache", "What the cache
  stores": K is stored after RoPE; "kv-cache-decoding", "Position
  information with a cache": a query and a key are rotated by angles of
  their absolute positions, so scores depend only on the distance). The
  pages leave the variant open; the reading here pairs element i with
  i + d_h/2, frequency base^(-2i/d_h), computed in float64 and rounded to
  float32 before the storage rounding.

Readings where the pages are silent (each one is listed with its reason in the
design notes of the repository):

* Rounding to fp16/bf16 is IEEE round-to-nearest-even from the float32 value
  the caller hands in. NaN becomes a canonical quiet NaN that keeps the sign
  (fp16: 0x7E00, bf16: 0x7FC0); overflow rounds to infinity.
* The query is rounded to the storage dtype before the product when the
  cache is fp16/bf16 and q arrives as float32 (a 16-bit q is used as is).
* Truncating to n > s (extending) or n < 0 is an error; appending past
  max_len is an error that changes nothing; T < 1 is an error; attend
  needs fill >= T for every row.
"""
from __future__ import annotations

import math

import numpy as np

DTYPES = ("fp32", "fp16", "bf16")
_ITEMSIZE = {"fp32": 4, "fp16": 2, "bf16": 2}


class OracleError(ValueError):
    """A call the cache contract rejects; the oracle state is unchanged."""


class OracleCapacityError(OracleError):
    """An append that would run past max_len."""


# ---------------------------------------------------------------------------
# Rounding to the storage dtype ("KV cache, ...", section 2.5: values are
# converted on the way in and the stored values are what is returned).
# ---------------------------------------------------------------------------

def round_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round-to-nearest-even.

    bfloat16 keeps the top 16 bits of the float32 pattern; rounding to nearest
    with ties to even adds 0x7FFF plus the lowest kept bit before the shift.
    Overflow carries into the exponent and gives infinity, as IEEE asks.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    is_nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    # only NaN patterns can wrap around 2^32 here, and those are replaced below
    r = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)
    r = r.astype(np.uint16)
    if is_nan.any():
        sign = (u[is_nan] >> np.uint32(31)).astype(np.uint16)
        r[is_nan] = (sign << np.uint16(15)) | np.uint16(0x7FC0)
    return r


def round_f16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> IEEE binary16 bit patterns (uint16), round-to-nearest-even.

    NumPy's float32 -> float16 cast is RNE with subnormals and overflow to
    infinity; NaN is replaced by the canonical quiet NaN of the same sign.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    with np.errstate(over="ignore"):
        h = x.astype(np.float16).view(np.uint16).astype(np.uint32)
    sign = (x.view(np.uint32) >> 31).astype(np.uint32)
    h = np.where(np.isnan(x), (sign << 15) | 0x7E00, h)
    return h.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> the float32 values they denote (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """binary16 bit patterns -> the float32 values they denote (exact)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


def round_to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """The float32 array of values a cache of `dtype` stores for input x."""
    if dtype == "fp32":
        return np.array(x, dtype=np.float32, copy=True)
    if dtype == "fp16":
        return f16_bits_to_f32(round_f16_bits(x))
    if dtype == "bf16":
        return bf16_bits_to_f32(round_bf16_bits(x))
    raise OracleError(f"unknown dtype {dtype!r}")


def storage_bits(values_f32: np.ndarray, dtype: str) -> np.ndarray:
    """Raw storage pattern of already-rounded values (uint32 for fp32, uint16 else)."""
    v = np.ascontiguousarray(values_f32, dtype=np.float32)
    if dtype == "fp32":
        return v.view(np.uint32).copy()
    if dtype == "bf16":
        return (v.view(np.uint32) >> 16).astype(np.uint16)
    if dtype == "fp16":
        return v.astype(np.float16).view(np.uint16).copy()
    raise OracleError(f"unknown dtype {dtype!r}")


# ---------------------------------------------------------------------------
# Mask and byte count, as closed forms.
# ---------------------------------------------------------------------------

def rope_freqs(d_head: int, base: float) -> np.ndarray:
    """Frequencies of the rotary pairs (i, i + d_head/2): base^(-2i / d_head)."""
    return np.float64(base) ** (-2.0 * np.arange(d_head // 2) / d_head)


def rope_rotate64(x: np.ndarray, positions: np.ndarray, base: float) -> np.ndarray:
    """Rotate head vectors x [..., T, d_head] at positions [..., T] (broadcast):
    each pair (x_i, x_{i + d/2}) turns by the angle position * f_i. float64."""
    x = np.asarray(x, dtype=np.float64)
    half = x.shape[-1] // 2
    ang = np.asarray(positions, dtype=np.int64).astype(np.float64)[..., None] * rope_freqs(x.shape[-1], base)
    c, sn = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * sn, x2 * c + x1 * sn], axis=-1)


def rope_rotate(x: np.ndarray, positions: np.ndarray, base: float) -> np.ndarray:
    """rope_rotate64 rounded to float32 (round to nearest even)."""
    return rope_rotate64(x, positions, base).astype(np.float32)


def causal_mask(T: int, n_keys: int, q_offset: int) -> np.ndarray:
    """Boolean [T, n_keys]: query i (absolute position q_offset + i) may see key j
    exactly when j <= q_offset + i ("KV cache, ...", section 2.3 equation;
    "kv-cache-decoding", step 3)."""
    i = np.arange(T)[:, None]
    j = np.arange(n_keys)[None, :]
    return j <= q_offset + i


def storage_bytes(n_layers: int, n_rows: int, n_kv_heads: int, n_positions: int, d_head: int,
                  itemsize: int) -> int:
    """Bytes of a cache's K and V: two tensors of n_layers x n_rows x n_kv_heads
    x n_positions x d_head values ("kv-cache-decoding", "What is cached, what is
    not, and what it costs"; "Heads, GQA and K/V cache", "Memory and the window
    limit"; with grouped-query attention only the KV heads count)."""
    return 2 * n_layers * n_rows * n_kv_heads * n_positions * d_head * itemsize


# ---------------------------------------------------------------------------
# The cache.
# ---------------------------------------------------------------------------

class OracleCache:
    """Float64 reference of the KV-cache contract (append / attend / seq_len /
    truncate / nbytes), with its own bookkeeping and its own rounding.

    K and V hold the dtype-rounded values as float32 (every fp16/bf16 value
    is exact in float32); arithmetic upcasts them to float64.
    """

    def __init__(self, n_layers: int, batch: int, n_q_heads: int, n_kv_heads: int,
                 d_head: int, max_len: int, dtype: str = "fp32"):
        for name, val in (("n_layers", n_layers), ("batch", batch), ("n_q_heads", n_q_heads),
                          ("n_kv_heads", n_kv_heads), ("d_head", d_head), ("max_len", max_len)):
            if int(val) < 1:
                raise OracleError(f"{name} must be positive, got {val}")
        if n_q_heads % n_kv_heads:
            raise OracleError("n_q_heads must be a multiple of n_kv_heads")
        if dtype not in DTYPES:
            raise OracleError(f"unknown dtype {dtype!r}")
        self.L, self.B = int(n_layers), int(batch)
        self.Hq, self.Hkv, self.D = int(n_q_heads), int(n_kv_heads), int(d_head)
        self.G = self.Hq // self.Hkv
        self.max_len = int(max_len)
        self.dtype = dtype
        shape = (self.L, self.B, self.Hkv, self.max_len, self.D)
        self.K = np.zeros(shape, dtype=np.float32)
        self.V = np.zeros(shape, dtype=np.float32)
        self.fill = np.zeros((self.L, self.B), dtype=np.int64)

    # -- bookkeeping ("KV cache, ...", sections 2.3 and 2.4) ---------------

    def seq_len(self, layer: int = -1) -> np.ndarray:
        """Per-row committed length min over layers (layer = -1), or one layer's fill."""
        if layer == -1:
            return self.fill.min(axis=0).copy()
        if not 0 <= layer < self.L:
            raise OracleError(f"layer {layer} out of range")
        return self.fill[layer].copy()

    def positions(self, T: int) -> np.ndarray:
        """[B, T] absolute positions s_b + i of the next chunk (what RoPE rotates by)."""
        s = self.seq_len(-1)
        return s[:, None] + np.arange(T)[None, :]

    def mask(self, T: int, row: int = 0) -> np.ndarray:
        """causal_mask(T, s + T, q_offset=s) for one row of the batch."""
        s = int(self.seq_len(-1)[row])
        return causal_mask(T, s + T, s)

    def truncate(self, n) -> None:
        """Set every layer's fill of each row to n (scalar: all rows). Storage is
        not touched; the next append overwrites from n."""
        n = np.asarray(n, dtype=np.int64)
        if n.ndim == 0:
            n = np.full(self.B, int(n), dtype=np.int64)
        if n.shape != (self.B,):
            raise OracleError("truncate takes one length or one per row")
        s = self.seq_len(-1)
        if (n < 0).any() or (n > s).any():
            raise OracleError("truncate length must lie in [0, committed length]")
        self.fill[:, :] = n[None, :]

    def nbytes(self) -> int:
        return storage_bytes(self.L, self.B, self.Hkv, self.max_len, self.D, _ITEMSIZE[self.dtype])

    # -- append ("KV cache, ...", sections 2.5 and 4; "kv-cache-decoding", step 5)

    def append(self, layer: int, k_new: np.ndarray, v_new: np.ndarray) -> None:
        """Store k_new, v_new [B, H_kv, T, d_h] (float32 or an already 16-bit
        array's float32 values) at slots [fill, fill + T) of `layer`."""
        if not 0 <= layer < self.L:
            raise OracleError(f"layer {layer} out of range")
        k_new = np.asarray(k_new)
        v_new = np.asarray(v_new)
        if k_new.ndim != 4 or k_new.shape != v_new.shape or k_new.shape[:2] != (self.B, self.Hkv) \
                or k_new.shape[3] != self.D:
            raise OracleError(f"k/v must be [B={self.B}, H_kv={self.Hkv}, T, d_h={self.D}]")
        T = k_new.shape[2]
        if T < 1:
            raise OracleError("T must be at least 1")
        f = self.fill[layer]
        if (f + T > self.max_len).any():
            raise OracleCapacityError("append would run past max_len")
        kr = round_to_storage(k_new.astype(np.float32), self.dtype)
        vr = round_to_storage(v_new.astype(np.float32), self.dtype)
        for b in range(self.B):
            fb = int(f[b])
            self.K[layer, b, :, fb:fb + T] = kr[b]
            self.V[layer, b, :, fb:fb + T] = vr[b]
        self.fill[layer] += T

    def append_rope(self, layer: int, k_new: np.ndarray, v_new: np.ndarray, base: float) -> None:
        """append with the keys rotated at their slots fill + t first."""
        k_new = np.asarray(k_new)
        if k_new.ndim != 4 or k_new.shape[:2] != (self.B, self.Hkv):
            raise OracleError(f"k/v must be [B={self.B}, H_kv={self.Hkv}, T, d_h={self.D}]")
        if not (np.isfinite(base) and base > 0):
            raise OracleError("rope base must be finite and positive")
        T = k_new.shape[2]
        pos = self.fill[layer][:, None, None] + np.arange(T)[None, None, :]        # [B, 1, T]
        self.append(layer, rope_rotate(k_new.astype(np.float32), pos, base), v_new)

    def rope_query(self, layer: int, q: np.ndarray, base: float, q_dtype: str = "fp32") -> np.ndarray:
        """q [B, H_q, T, d_h] rotated at the positions the next attend of
        `layer` gives it (s_b + t, s_b = fill - T), rounded to float32 and then
        to q_dtype. Returns float32 values."""
        q = np.asarray(q, dtype=np.float32)
        T = q.shape[2]
        if (self.fill[layer] < T).any():
            raise OracleError("rope_query needs the chunk appended first (fill >= T)")
        pos = (self.fill[layer] - T)[:, None, None] + np.arange(T)[None, None, :]
        return round_to_storage(rope_rotate(q, pos, base), q_dtype)

    # -- attend (the plain definition) --------------------------------------

    def query_values(self, q: np.ndarray) -> np.ndarray:
        """The values of q the product uses: rounded to the storage dtype when
        the cache is 16-bit and q is float32 (a 16-bit q is already exact)."""
        q = np.asarray(q)
        if self.dtype != "fp32" and q.dtype == np.float32:
            return round_to_storage(q, self.dtype)
        return q.astype(np.float32)

    def attend(self, layer: int, q: np.ndarray, rows=None) -> np.ndarray:
        """out[b, h, i] = sum_j w_j V[g, j] / sum_j w_j over visible keys j,
        w_j = exp(z_j - max z), z_j = q[b, h, i] . K[g, j] / sqrt(d_h), g = h // G.

        q is [B, H_q, T, d_h]; the chunk is the last T slots of the layer, so row
        b's query offset is s_b = fill[layer][b] - T. Returns float64
        [B, H_q, T, d_h]; with rows = [(b, h, i), ...] only those are computed
        (others stay NaN).
        """
        if not 0 <= layer < self.L:
            raise OracleError(f"layer {layer} out of range")
        q = np.asarray(q)
        if q.ndim != 4 or q.shape[:2] != (self.B, self.Hq) or q.shape[3] != self.D:
            raise OracleError(f"q must be [B={self.B}, H_q={self.Hq}, T, d_h={self.D}]")
        T = q.shape[2]
        if T < 1:
            raise OracleError("T must be at least 1")
        if (self.fill[layer] < T).any():
            raise OracleError("attend needs the chunk appended first (fill >= T)")
        qv = self.query_values(q).astype(np.float64)
        out = np.full((self.B, self.Hq, T, self.D), np.nan)
        inv_sqrt_d = 1.0 / math.sqrt(self.D)
        wanted = None
        if rows is not None:
            wanted = {}
            for (b, h, i) in rows:
                wanted.setdefault((int(b), int(h) // self.G), set()).add((int(h), int(i)))
        for b in range(self.B):
            n = int(self.fill[layer, b])
            s = n - T
            visible = causal_mask(T, n, s)
            for g in range(self.Hkv):
                if wanted is not None and (b, g) not in wanted:
                    continue
                Kg = self.K[layer, b, g, :n].astype(np.float64)
                Vg = self.V[layer, b, g, :n].astype(np.float64)
                for h in range(g * self.G, (g + 1) * self.G):
                    if wanted is not None:
                        idx = sorted(i for (hh, i) in wanted[(b, g)] if hh == h)
                        if not idx:
                            continue
                    else:
                        idx = list(range(T))
                    z = (qv[b, h, idx] @ Kg.T) * inv_sqrt_d          # [len(idx), n]
                    vis = visible[idx]
                    z = np.where(vis, z, -np.inf)                     # masked keys drop out
                    m = z.max(axis=1, keepdims=True)
                    w = np.where(vis, np.exp(z - m), 0.0)
                    out[b, h, idx] = (w @ Vg) / w.sum(axis=1, keepdims=True)
        return out

    # -- raw views for bit-exact comparison ---------------------------------

    def stored_bits(self, which: str = "K") -> np.ndarray:
        arr = self.K if which == "K" else self.V
        return storage_bits(arr, self.dtype)


class OracleLatentCache:
    """The latent cache of multi-head latent attention ("KV cache, incremental
    decode, ...", section 2.6): one latent c (rank r) and one shared rotary key
    k_R (d_R) per position, under the K/V cache's rules (per-layer fill,
    committed length = min over layers, metadata-only truncate). Storage
    C (L, B, max_len, r) and KR (L, B, max_len, d_R) holds the values rounded
    to the storage dtype (as float32), zero before anything is written."""

    def __init__(self, n_layers: int, batch: int, rank: int, rope_dim: int, max_len: int, dtype: str):
        if dtype not in DTYPES:
            raise OracleError(f"dtype {dtype!r}")
        if min(n_layers, batch, rank, rope_dim, max_len) < 1:
            raise OracleError("dimensions must be positive")
        self.L, self.B, self.r, self.dR, self.max_len, self.dtype = n_layers, batch, rank, rope_dim, max_len, dtype
        self.C = np.zeros((n_layers, batch, max_len, rank), np.float32)
        self.KR = np.zeros((n_layers, batch, max_len, rope_dim), np.float32)
        self.fill = np.zeros((n_layers, batch), np.int64)

    def seq_len(self, layer: int = -1) -> np.ndarray:
        return self.fill.min(axis=0).copy() if layer < 0 else self.fill[layer].copy()

    def append(self, layer: int, c_new: np.ndarray, kr_new: np.ndarray) -> None:
        """c_new [B, T, r], kr_new [B, T, d_R] (float32 values) at slots
        [fill, fill + T) of `layer`, rounded; nothing changes on an error."""
        if not 0 <= layer < self.L:
            raise OracleError(f"layer {layer} out of range")
        c_new, kr_new = np.asarray(c_new), np.asarray(kr_new)
        if c_new.shape[:1] != (self.B,) or c_new.ndim != 3 or c_new.shape[2] != self.r \
                or kr_new.shape != (self.B, c_new.shape[1], self.dR):
            raise OracleError(f"c_new [B={self.B}, T, {self.r}] and kr_new [B, T, {self.dR}] expected")
        T = c_new.shape[1]
        if T < 1:
            raise OracleError("T must be at least 1")
        if (self.fill[layer] + T > self.max_len).any():
            raise OracleCapacityError("append would run past max_len")
        cr = round_to_storage(c_new.astype(np.float32), self.dtype)
        kr = round_to_storage(kr_new.astype(np.float32), self.dtype)
        for b in range(self.B):
            f = int(self.fill[layer, b])
            self.C[layer, b, f:f + T] = cr[b]
            self.KR[layer, b, f:f + T] = kr[b]
        self.fill[layer] += T

    def truncate(self, n) -> None:
        n = np.broadcast_to(np.asarray(n, dtype=np.int64), (self.B,))
        if (n < 0).any() or (n > self.seq_len()).any():
            raise OracleError("truncate needs 0 <= n <= committed length")
        self.fill[:] = n[None, :]

    def nbytes(self) -> int:
        return self.L * self.B * self.max_len * (self.r + self.dR) * _ITEMSIZE[self.dtype]
