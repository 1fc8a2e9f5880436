"""Thin ctypes binding of libkvc (include/kvc.h).

Argument marshalling only: every step of append and attention runs in the
HIP kernels of libkvc.so. PyTorch supplies device memory and streams.
Importing this module loads the library and raises ImportError when it has
not been built (there is no fallback).

    cache = KVCache(n_layers, n_kv_heads, d_head, max_len, batch=B,
                    n_q_heads=Hq, dtype="bf16")
    cache.append(layer, k, v)        # k, v: [B, H_kv, T, d_h] device tensors
    out = cache.attend(layer, q)     # q: [B, H_q, T, d_h] -> float32 [B, H_q, T, d_h]
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvc.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -m kv_cached_gqa_amd.build` "
                      "(or __graft_entry__.build()) first")

_lib = ctypes.CDLL(LIB_PATH)

# ---- dtypes and status codes (kvc.h) --------------------------------------
F32, F16, BF16 = 0, 1, 2
DTYPE_CODES = {"fp32": F32, "fp16": F16, "bf16": BF16}
ITEMSIZE = {"fp32": 4, "fp16": 2, "bf16": 2}

PREFILL_P_ROUNDED, PREFILL_P_SPLIT = 0, 1      # kvc_prefill_precision
PREFILL_PRECISION = {"rounded": PREFILL_P_ROUNDED, "split": PREFILL_P_SPLIT}

OK = 0
ERR_ARG, ERR_CAPACITY, ERR_STATE, ERR_DTYPE = -1, -2, -3, -4
ERR_STORAGE, ERR_HIP, ERR_NOMEM, ERR_UNSUPPORTED, ERR_SCRATCH = -5, -6, -7, -8, -9

EXPORTED = ("kvc_create", "kvc_destroy", "kvc_append", "kvc_append_rope", "kvc_rope_q", "kvc_attend",
            "kvc_append_attend", "kvc_gather", "kvc_attend_static", "kvc_set_prefill_precision",
            "kvc_seq_len", "kvc_truncate", "kvc_nbytes", "kvc_strerror",
            "kvc_create_paged", "kvc_paged_blocks", "kvc_block_table",
            "kvc_latent_create", "kvc_latent_destroy", "kvc_latent_append", "kvc_latent_seq_len",
            "kvc_latent_truncate", "kvc_latent_nbytes")


class KVCConfig(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("d_head", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("max_len", ctypes.c_int64)]


_vp, _i32, _i64, _u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
_lib.kvc_create.argtypes = [ctypes.POINTER(KVCConfig), _vp, _vp, _u64, ctypes.POINTER(_vp)]
_lib.kvc_create.restype = ctypes.c_int
_lib.kvc_create_paged.argtypes = [ctypes.POINTER(KVCConfig), _i32, _i32, _vp, _vp, _u64, ctypes.POINTER(_vp)]
_lib.kvc_create_paged.restype = ctypes.c_int
_lib.kvc_paged_blocks.argtypes = [_vp, ctypes.POINTER(_i32), ctypes.POINTER(_i32)]
_lib.kvc_paged_blocks.restype = ctypes.c_int
_lib.kvc_block_table.argtypes = [_vp, ctypes.POINTER(_i32), _i64]
_lib.kvc_block_table.restype = ctypes.c_int
_lib.kvc_destroy.argtypes = [_vp]
_lib.kvc_destroy.restype = None
_lib.kvc_append.argtypes = [_vp, _i32, _vp, _vp, _i32, _i32, _vp]
_lib.kvc_append.restype = ctypes.c_int
_lib.kvc_append_rope.argtypes = [_vp, _i32, _vp, _vp, _i32, _i32, ctypes.c_double, _vp]
_lib.kvc_append_rope.restype = ctypes.c_int
_lib.kvc_rope_q.argtypes = [_vp, _i32, _vp, _i32, _i32, ctypes.c_double, _vp]
_lib.kvc_rope_q.restype = ctypes.c_int
_lib.kvc_attend.argtypes = [_vp, _i32, _vp, _i32, _i32, _vp, _vp]
_lib.kvc_attend.restype = ctypes.c_int
_lib.kvc_append_attend.argtypes = [_vp, _i32, _vp, _vp, _i32, _vp, _i32, _i32, _vp, _vp]
_lib.kvc_append_attend.restype = ctypes.c_int
_lib.kvc_attend_static.argtypes = [_vp, _i32, _vp, _i32, _i32, _vp, _vp]
_lib.kvc_attend_static.restype = ctypes.c_int
_lib.kvc_set_prefill_precision.argtypes = [_vp, _i32]
_lib.kvc_set_prefill_precision.restype = ctypes.c_int
_lib.kvc_gather.argtypes = [_vp, _i32, _i64, _vp, _vp, _vp]
_lib.kvc_gather.restype = ctypes.c_int
_lib.kvc_seq_len.argtypes = [_vp, _i32, ctypes.POINTER(_i64)]
_lib.kvc_seq_len.restype = ctypes.c_int
_lib.kvc_truncate.argtypes = [_vp, _vp, _i32]        # int64 lengths, by address
_lib.kvc_truncate.restype = ctypes.c_int
_lib.kvc_nbytes.argtypes = [_vp, ctypes.POINTER(_u64)]
_lib.kvc_nbytes.restype = ctypes.c_int
_lib.kvc_latent_create.argtypes = [_vp, _vp, _vp, _u64, _u64, ctypes.POINTER(_vp)]
_lib.kvc_latent_create.restype = ctypes.c_int
_lib.kvc_latent_destroy.argtypes = [_vp]
_lib.kvc_latent_destroy.restype = None
_lib.kvc_latent_append.argtypes = [_vp, _i32, _vp, _vp, _i32, _i32, _vp]
_lib.kvc_latent_append.restype = ctypes.c_int
_lib.kvc_latent_seq_len.argtypes = [_vp, _i32, ctypes.POINTER(_i64)]
_lib.kvc_latent_seq_len.restype = ctypes.c_int
_lib.kvc_latent_truncate.argtypes = [_vp, _vp, _i32]
_lib.kvc_latent_truncate.restype = ctypes.c_int
_lib.kvc_latent_nbytes.argtypes = [_vp, ctypes.POINTER(_u64)]
_lib.kvc_latent_nbytes.restype = ctypes.c_int
_lib.kvc_strerror.argtypes = [ctypes.c_int]
_lib.kvc_strerror.restype = ctypes.c_char_p


class KVCError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call}: {strerror(status)} ({status})")


class KVCArgumentError(KVCError, ValueError):
    """Bad argument, dtype, storage or unsupported shape."""


class ContextLimitError(KVCError):
    """An append would run past max_len (the cache is unchanged)."""


class KVCStateError(KVCError):
    """Attend before append, or truncate past the committed length."""


def strerror(status: int) -> str:
    return _lib.kvc_strerror(int(status)).decode()


def _check(status: int, call: str) -> None:
    if status == OK:
        return
    if status == ERR_CAPACITY:
        raise ContextLimitError(status, call)
    if status == ERR_STATE:
        raise KVCStateError(status, call)
    if status in (ERR_ARG, ERR_DTYPE, ERR_STORAGE, ERR_UNSUPPORTED):
        raise KVCArgumentError(status, call)
    raise KVCError(status, call)


def lib() -> ctypes.CDLL:
    """The loaded libkvc (for tests that call the C ABI directly)."""
    return _lib


# ---- torch plumbing ----------------------------------------------------------

def _torch():
    import torch
    return torch


def torch_dtype(name: str):
    torch = _torch()
    return {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}[name]


_DTYPE_NAMES = {}     # torch dtype -> name, filled at the first call (torch is imported lazily)


def dtype_name(t) -> str:
    if not _DTYPE_NAMES:
        torch = _torch()
        _DTYPE_NAMES.update({torch.float32: "fp32", torch.float16: "fp16", torch.bfloat16: "bf16"})
    name = _DTYPE_NAMES.get(t.dtype)
    if name is None:
        raise KVCArgumentError(ERR_DTYPE, f"dtype {t.dtype}")
    return name


def _dtype_code(t) -> int:
    return DTYPE_CODES[dtype_name(t)]


def _stream_ptr(stream, device=None) -> Optional[int]:
    """The HIP stream to enqueue on: `stream`, else the current stream of
    `device` (read directly: building a torch Stream object per call costs
    microseconds, which a launch-bound caller pays on every call)."""
    if stream is not None:
        return stream.cuda_stream
    torch = _torch()
    idx = device.index if device is not None and device.index is not None else torch.cuda.current_device()
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return raw(idx)
    return torch.cuda.current_stream(idx).cuda_stream


def _lengths(n) -> tuple:
    """(address, count, keep-alive) of n as contiguous int64."""
    arr = np.ascontiguousarray(np.atleast_1d(np.asarray(n, dtype=np.int64)))
    return arr.__array_interface__["data"][0], int(arr.size), arr


class KVCache:
    """Owns zero-filled device storage (two torch tensors shaped
    (L, B, H_kv, max_len, d_h)) and a libkvc handle over it.

    The method names follow the KVCache interface of "KV cache, incremental
    decode, incremental UTF-8 detokenizer, generate" (section 4).
    """

    def __init__(self, n_layers: int, n_kv_heads: int, d_head: int, max_len: int, batch: int = 1,
                 n_q_heads: Optional[int] = None, dtype: str = "fp32", device=None):
        torch = _torch()
        if dtype not in DTYPE_CODES:
            raise KVCArgumentError(ERR_DTYPE, f"dtype {dtype!r}")
        self.n_layers, self.batch = int(n_layers), int(batch)
        self.n_kv_heads, self.d_head, self.max_len = int(n_kv_heads), int(d_head), int(max_len)
        self.n_q_heads = int(n_q_heads if n_q_heads is not None else n_kv_heads)
        self.dtype = dtype
        self.device = torch.device(device if device is not None else "cuda")
        shape = (self.n_layers, self.batch, self.n_kv_heads, self.max_len, self.d_head)
        tdt = torch_dtype(dtype)
        self.k_storage = torch.zeros(shape, dtype=tdt, device=self.device)
        self.v_storage = torch.zeros(shape, dtype=tdt, device=self.device)
        self._dev = self.k_storage.device
        cfg = KVCConfig(self.n_layers, self.batch, self.n_q_heads, self.n_kv_heads, self.d_head,
                        DTYPE_CODES[dtype], self.max_len)
        h = _vp()
        each = self.k_storage.numel() * self.k_storage.element_size()
        _check(_lib.kvc_create(ctypes.byref(cfg), self.k_storage.data_ptr(), self.v_storage.data_ptr(),
                               each, ctypes.byref(h)), "kvc_create")
        self._h = h

    # -- lifetime --
    def close(self) -> None:
        if getattr(self, "_h", None):
            _lib.kvc_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def handle(self):
        return self._h

    # -- the contract --
    def append(self, layer: int, k_new, v_new, stream=None, rope_base: Optional[float] = None) -> None:
        """Store k_new, v_new [B, H_kv, T, d_h] (device, contiguous) at slots
        [fill, fill + T) of `layer`, rounded to the storage dtype. With
        rope_base, K is stored rotated at its positions (kvc_append_rope)."""
        self._check_chunk(k_new, self.n_kv_heads, "k_new")
        self._check_chunk(v_new, self.n_kv_heads, "v_new")
        if k_new.shape != v_new.shape or k_new.dtype != v_new.dtype:
            raise KVCArgumentError(ERR_ARG, "k_new and v_new differ in shape or dtype")
        if rope_base is None:
            _check(_lib.kvc_append(self._h, int(layer), k_new.data_ptr(), v_new.data_ptr(),
                                   _dtype_code(k_new), int(k_new.shape[2]), _stream_ptr(stream, self._dev)),
                   "kvc_append")
        else:
            _check(_lib.kvc_append_rope(self._h, int(layer), k_new.data_ptr(), v_new.data_ptr(),
                                        _dtype_code(k_new), int(k_new.shape[2]), float(rope_base),
                                        _stream_ptr(stream, self._dev)), "kvc_append_rope")

    def rope_q(self, layer: int, q, rope_base: float, stream=None):
        """Rotate q [B, H_q, T, d_h] (device, contiguous) in place at the
        positions the next attend of `layer` gives the chunk; returns q."""
        self._check_chunk(q, self.n_q_heads, "q")
        _check(_lib.kvc_rope_q(self._h, int(layer), q.data_ptr(), _dtype_code(q), int(q.shape[2]),
                               float(rope_base), _stream_ptr(stream, self._dev)), "kvc_rope_q")
        return q

    def attend(self, layer: int, q, out=None, stream=None):
        """softmax(q K^T / sqrt(d_h)) V over everything `layer` holds, with the
        chunk's queries at positions [s, s + T). Returns float32 [B, H_q, T, d_h]."""
        torch = _torch()
        self._check_chunk(q, self.n_q_heads, "q")
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        elif out.shape != q.shape or out.dtype != torch.float32 or not out.is_contiguous():
            raise KVCArgumentError(ERR_ARG, "out must be contiguous float32 shaped like q")
        _check(_lib.kvc_attend(self._h, int(layer), q.data_ptr(), _dtype_code(q),
                               int(q.shape[2]), out.data_ptr(), _stream_ptr(stream, self._dev)), "kvc_attend")
        return out

    def append_attend(self, layer: int, k_new, v_new, q, out=None, stream=None):
        """append(layer, k_new, v_new) then attend(layer, q) in one call
        (kvc_append_attend: one decode launch for a decode step whose input
        already has the storage dtype). Returns float32 [B, H_q, T, d_h]."""
        torch = _torch()
        self._check_chunk(k_new, self.n_kv_heads, "k_new")
        self._check_chunk(v_new, self.n_kv_heads, "v_new")
        self._check_chunk(q, self.n_q_heads, "q")
        if k_new.shape != v_new.shape or k_new.dtype != v_new.dtype or q.shape[2] != k_new.shape[2]:
            raise KVCArgumentError(ERR_ARG, "k_new, v_new and q differ in T or dtype")
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        elif out.shape != q.shape or out.dtype != torch.float32 or not out.is_contiguous():
            raise KVCArgumentError(ERR_ARG, "out must be contiguous float32 shaped like q")
        _check(_lib.kvc_append_attend(self._h, int(layer), k_new.data_ptr(), v_new.data_ptr(),
                                      _dtype_code(k_new), q.data_ptr(), _dtype_code(q),
                                      int(q.shape[2]), out.data_ptr(), _stream_ptr(stream, self._dev)), "kvc_append_attend")
        return out

    def update(self, layer: int, k_new, v_new, stream=None):
        """Append, then return views of everything the layer stores (the pages'
        update): [B, H_kv, n, d_h] up to the longest row's fill."""
        self.append(layer, k_new, v_new, stream)
        n = int(self.seq_len(layer).max())
        return self.k_storage[layer, :, :, :n], self.v_storage[layer, :, :, :n]

    def seq_len(self, layer: Optional[int] = None) -> np.ndarray:
        """Per-row committed length (layer None) or one layer's fill count."""
        out = (_i64 * self.batch)()
        _check(_lib.kvc_seq_len(self._h, -1 if layer is None else int(layer), out), "kvc_seq_len")
        return np.frombuffer(out, dtype=np.int64).copy()

    def positions(self, t_new: int) -> np.ndarray:
        """[B, T] absolute positions s_b + i of the next chunk."""
        s = self.seq_len()
        return s[:, None] + np.arange(int(t_new))[None, :]

    def mask(self, t_new: int, row: int = 0) -> np.ndarray:
        """causal_mask(T, s + T, q_offset=s) for one row (boolean [T, s + T])."""
        s = int(self.seq_len()[row])
        i = np.arange(int(t_new))[:, None]
        j = np.arange(s + int(t_new))[None, :]
        return j <= s + i

    def truncate(self, n) -> None:
        ptr, count, _keep = _lengths(n)
        _check(_lib.kvc_truncate(self._h, ptr, count),
               "kvc_truncate")

    def nbytes(self) -> int:
        out = _u64()
        _check(_lib.kvc_nbytes(self._h, ctypes.byref(out)), "kvc_nbytes")
        return int(out.value)

    def set_prefill_precision(self, mode: str) -> None:
        """"rounded" (the default: P rounded once to the storage type) or
        "split" (P as a hi + lo pair) for this cache's prefill chunks."""
        if mode not in PREFILL_PRECISION:
            raise KVCArgumentError(ERR_ARG, f"prefill precision must be one of {sorted(PREFILL_PRECISION)}")
        _check(_lib.kvc_set_prefill_precision(self._h, PREFILL_PRECISION[mode]), "kvc_set_prefill_precision")

    def attend_static(self, layer: int, q, out, stream=None):
        """attend() through kvc_attend_static: split-K scratch from the library's
        static device array, nothing allocated (out must be given)."""
        torch = _torch()
        self._check_chunk(q, self.n_q_heads, "q")
        if out.shape != q.shape or out.dtype != torch.float32 or not out.is_contiguous():
            raise KVCArgumentError(ERR_ARG, "out must be contiguous float32 shaped like q")
        _check(_lib.kvc_attend_static(self._h, int(layer), q.data_ptr(), _dtype_code(q),
                                      int(q.shape[2]), out.data_ptr(), _stream_ptr(stream, self._dev)),
               "kvc_attend_static")
        return out

    def gather(self, layer: int, n: Optional[int] = None, stream=None):
        """Copies [B, H_kv, n, d_h] of K and V of `layer` in position order
        (kvc_gather; n defaults to the longest row's fill; positions at or past
        a row's fill read as zero)."""
        torch = _torch()
        n = int(self.seq_len(layer).max()) if n is None else int(n)
        shape = (self.batch, self.n_kv_heads, max(n, 1), self.d_head)
        k = torch.empty(shape, dtype=torch_dtype(self.dtype), device=self._dev)
        v = torch.empty_like(k)
        if n < 1:
            return k[:, :, :0], v[:, :, :0]
        _check(_lib.kvc_gather(self._h, int(layer), n, k.data_ptr(), v.data_ptr(), _stream_ptr(stream, self._dev)),
               "kvc_gather")
        return k, v

    # -- helpers --
    def _check_chunk(self, t, heads: int, name: str) -> None:
        sh = t.shape          # read once: every access builds a new size object
        if len(sh) != 4 or sh[0] != self.batch or sh[1] != heads or sh[3] != self.d_head:
            raise KVCArgumentError(ERR_ARG, f"{name} must be [B={self.batch}, H={heads}, T, d_h={self.d_head}], "
                                            f"got {tuple(sh)}")
        if not t.is_contiguous() or t.device != self._dev:
            raise KVCArgumentError(ERR_ARG, f"{name} must be contiguous and on {self._dev}")


class PagedKVCache(KVCache):
    """The same cache over block pools (kvc_create_paged): k_pool and v_pool
    shaped (L, n_blocks, H_kv, block_size, d_h), one block table for all
    layers, blocks taken on growth and given back on truncate ("kv-cache-
    decoding", "Batching caches of different lengths"). Every call of KVCache
    works unchanged; `update` returns gathered copies instead of views."""

    def __init__(self, n_layers: int, n_kv_heads: int, d_head: int, max_len: int, batch: int = 1,
                 n_q_heads: Optional[int] = None, dtype: str = "fp32", device=None, block_size: int = 128,
                 n_blocks: Optional[int] = None):
        torch = _torch()
        if dtype not in DTYPE_CODES:
            raise KVCArgumentError(ERR_DTYPE, f"dtype {dtype!r}")
        self.n_layers, self.batch = int(n_layers), int(batch)
        self.n_kv_heads, self.d_head, self.max_len = int(n_kv_heads), int(d_head), int(max_len)
        self.n_q_heads = int(n_q_heads if n_q_heads is not None else n_kv_heads)
        self.dtype = dtype
        self.device = torch.device(device if device is not None else "cuda")
        self.block_size = int(block_size)
        self.width = -(-self.max_len // self.block_size)
        self.n_blocks = int(n_blocks if n_blocks is not None else self.batch * self.width)
        shape = (self.n_layers, self.n_blocks, self.n_kv_heads, self.block_size, self.d_head)
        tdt = torch_dtype(dtype)
        self.k_pool = torch.empty(shape, dtype=tdt, device=self.device)
        self.v_pool = torch.empty(shape, dtype=tdt, device=self.device)
        self._dev = self.k_pool.device
        cfg = KVCConfig(self.n_layers, self.batch, self.n_q_heads, self.n_kv_heads, self.d_head,
                        DTYPE_CODES[dtype], self.max_len)
        h = _vp()
        each = self.k_pool.numel() * self.k_pool.element_size()
        _check(_lib.kvc_create_paged(ctypes.byref(cfg), self.block_size, self.n_blocks, self.k_pool.data_ptr(),
                                     self.v_pool.data_ptr(), each, ctypes.byref(h)), "kvc_create_paged")
        self._h = h

    def block_table(self) -> np.ndarray:
        """The host block table, int32 [B, ceil(max_len / block_size)], -1 = none."""
        out = np.empty((self.batch, self.width), dtype=np.int32)
        _check(_lib.kvc_block_table(self._h, out.ctypes.data_as(ctypes.POINTER(_i32)), int(out.size)),
               "kvc_block_table")
        return out

    def blocks(self) -> tuple:
        """(blocks in use, blocks in the pool)."""
        used, total = _i32(), _i32()
        _check(_lib.kvc_paged_blocks(self._h, ctypes.byref(used), ctypes.byref(total)), "kvc_paged_blocks")
        return int(used.value), int(total.value)

    def update(self, layer: int, k_new, v_new, stream=None):
        """Append, then return copies of everything the layer stores."""
        self.append(layer, k_new, v_new, stream)
        return self.gather(layer)


class KVCLatentConfig(ctypes.Structure):
    _fields_ = [("n_layers", _i32), ("batch", _i32), ("rank", _i32), ("rope_dim", _i32), ("dtype", _i32),
                ("max_len", _i64)]


class LatentCache:
    """Latent cache of multi-head latent attention ("KV cache, incremental
    decode, ...", section 2.6): zero-filled device storage c (L, B, max_len, r)
    and k_rope (L, B, max_len, d_R) and a libkvc handle over it, with the K/V
    cache's rules (per-layer fill, committed length, truncate)."""

    def __init__(self, n_layers: int, rank: int, rope_dim: int, max_len: int, batch: int = 1,
                 dtype: str = "fp32", device=None):
        torch = _torch()
        if dtype not in DTYPE_CODES:
            raise KVCArgumentError(ERR_DTYPE, f"dtype {dtype!r}")
        self.n_layers, self.batch, self.max_len = int(n_layers), int(batch), int(max_len)
        self.rank, self.rope_dim, self.dtype = int(rank), int(rope_dim), dtype
        self.device = torch.device(device if device is not None else "cuda")
        tdt = torch_dtype(dtype)
        self.c_storage = torch.zeros((self.n_layers, self.batch, self.max_len, self.rank), dtype=tdt,
                                     device=self.device)
        self.kr_storage = torch.zeros((self.n_layers, self.batch, self.max_len, self.rope_dim), dtype=tdt,
                                      device=self.device)
        self._dev = self.c_storage.device
        cfg = KVCLatentConfig(self.n_layers, self.batch, self.rank, self.rope_dim, DTYPE_CODES[dtype], self.max_len)
        h = _vp()
        nb = lambda t: t.numel() * t.element_size()  # noqa: E731
        _check(_lib.kvc_latent_create(ctypes.byref(cfg), self.c_storage.data_ptr(), self.kr_storage.data_ptr(),
                                      nb(self.c_storage), nb(self.kr_storage), ctypes.byref(h)), "kvc_latent_create")
        self._h = h

    def close(self) -> None:
        if getattr(self, "_h", None):
            _lib.kvc_latent_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def append(self, layer: int, c_new, kr_new, stream=None) -> None:
        """Store c_new [B, T, r] and kr_new [B, T, d_R] (device, contiguous, one
        dtype) at slots [fill, fill + T) of `layer`, rounded to the storage dtype."""
        for t, w, name in ((c_new, self.rank, "c_new"), (kr_new, self.rope_dim, "kr_new")):
            if t.dim() != 3 or t.shape[0] != self.batch or t.shape[2] != w:
                raise KVCArgumentError(ERR_ARG, f"{name} must be [B={self.batch}, T, {w}], got {tuple(t.shape)}")
            if not t.is_contiguous() or t.device != self.c_storage.device:
                raise KVCArgumentError(ERR_ARG, f"{name} must be contiguous and on {self.c_storage.device}")
        if c_new.shape[1] != kr_new.shape[1] or c_new.dtype != kr_new.dtype:
            raise KVCArgumentError(ERR_ARG, "c_new and kr_new differ in T or dtype")
        _check(_lib.kvc_latent_append(self._h, int(layer), c_new.data_ptr(), kr_new.data_ptr(),
                                      _dtype_code(c_new), int(c_new.shape[1]), _stream_ptr(stream, self._dev)),
               "kvc_latent_append")

    def seq_len(self, layer: Optional[int] = None) -> np.ndarray:
        out = (_i64 * self.batch)()
        _check(_lib.kvc_latent_seq_len(self._h, -1 if layer is None else int(layer), out), "kvc_latent_seq_len")
        return np.frombuffer(out, dtype=np.int64).copy()

    def truncate(self, n) -> None:
        ptr, count, _keep = _lengths(n)
        _check(_lib.kvc_latent_truncate(self._h, ptr, count),
               "kvc_latent_truncate")

    def nbytes(self) -> int:
        out = _u64()
        _check(_lib.kvc_latent_nbytes(self._h, ctypes.byref(out)), "kvc_latent_nbytes")
        return int(out.value)


def exported_symbols(names: Sequence[str] = EXPORTED) -> dict:
    """Which of the C ABI's names the loaded library exports."""
    found = {}
    for n in names:
        try:
            getattr(_lib, n)
            found[n] = True
        except AttributeError:
            found[n] = False
    return found
