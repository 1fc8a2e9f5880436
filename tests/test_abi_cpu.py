"""The C ABI on the CPU: the library loads, exports every call include/kvc.h
declares, and rejects bad arguments before any device work (an error leaves
the cache unchanged). No call here reaches a kernel launch."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvc.h")


@pytest.fixture(scope="module")
def kvc():
    from kv_cached_gqa_amd import kvc as mod
    return mod


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvc_[a-z_]+)\s*\(", text)))


def test_header_declares_the_contract():
    names = declared_functions()
    for n in ("kvc_create", "kvc_destroy", "kvc_append", "kvc_attend", "kvc_seq_len", "kvc_truncate",
              "kvc_nbytes", "kvc_strerror"):
        assert n in names


def test_library_exports_every_declared_symbol(kvc):
    found = kvc.exported_symbols(declared_functions())
    assert all(found.values()), found


def test_strerror(kvc):
    assert kvc.strerror(0) == "ok"
    for code in range(-9, 0):
        assert kvc.strerror(code) and kvc.strerror(code) != "unknown status"
    assert kvc.strerror(-99) == "unknown status"


# A 256-byte-aligned host buffer stands in for device storage: kvc_create only
# records the pointers and never dereferences them.
_BUF = np.zeros(1 << 16, dtype=np.uint8)
_BASE = (_BUF.ctypes.data + 255) & ~255


def _create(kvc, L=2, B=3, Hq=4, Hkv=2, D=32, max_len=8, dtype=0, store=None, kptr=_BASE, vptr=_BASE):
    cfg = kvc.KVCConfig(L, B, Hq, Hkv, D, dtype, max_len)
    nb = 2 * L * B * Hkv * max_len * D * (4 if dtype == 0 else 2)
    h = ctypes.c_void_p()
    rc = kvc.lib().kvc_create(ctypes.byref(cfg), kptr, vptr, nb // 2 if store is None else store, ctypes.byref(h))
    return rc, h


def test_create_validation(kvc):
    assert _create(kvc, L=0)[0] == kvc.ERR_ARG
    assert _create(kvc, B=-1)[0] == kvc.ERR_ARG
    assert _create(kvc, Hq=3, Hkv=2)[0] == kvc.ERR_ARG
    assert _create(kvc, max_len=0)[0] == kvc.ERR_ARG
    assert _create(kvc, D=128, max_len=1 << 24)[0] == kvc.ERR_ARG      # max_len * d_head >= 2^31
    assert _create(kvc, dtype=7)[0] == kvc.ERR_DTYPE
    assert _create(kvc, D=48)[0] == kvc.ERR_UNSUPPORTED
    assert _create(kvc, kptr=None)[0] == kvc.ERR_STORAGE
    assert _create(kvc, vptr=_BASE + 8)[0] == kvc.ERR_STORAGE            # not 16-byte aligned
    assert _create(kvc, store=100)[0] == kvc.ERR_STORAGE
    h = ctypes.c_void_p()
    assert kvc.lib().kvc_create(None, _BASE, _BASE, 1 << 20, ctypes.byref(h)) == kvc.ERR_ARG


@pytest.mark.parametrize("dtype,itemsize", [(0, 4), (1, 2), (2, 2)])
def test_fresh_handle_metadata(kvc, dtype, itemsize):
    rc, h = _create(kvc, L=2, B=3, Hkv=2, D=32, max_len=8, dtype=dtype)
    assert rc == kvc.OK
    lib = kvc.lib()
    try:
        nb = ctypes.c_uint64()
        assert lib.kvc_nbytes(h, ctypes.byref(nb)) == kvc.OK
        assert nb.value == 2 * 2 * 3 * 2 * 8 * 32 * itemsize
        lens = (ctypes.c_int64 * 3)()
        for layer in (-1, 0, 1):
            assert lib.kvc_seq_len(h, layer, lens) == kvc.OK
            assert list(lens) == [0, 0, 0]
        assert lib.kvc_seq_len(h, 2, lens) == kvc.ERR_ARG
        assert lib.kvc_seq_len(h, -2, lens) == kvc.ERR_ARG
        zero = (ctypes.c_int64 * 1)(0)
        assert lib.kvc_truncate(h, zero, 1) == kvc.OK                      # n = s is a no-op
        one = (ctypes.c_int64 * 1)(1)
        assert lib.kvc_truncate(h, one, 1) == kvc.ERR_STATE                # cannot extend
        assert lib.kvc_truncate(h, zero, 2) == kvc.ERR_ARG                 # count is 1 or batch
        neg = (ctypes.c_int64 * 3)(0, -1, 0)
        assert lib.kvc_truncate(h, neg, 3) == kvc.ERR_STATE
    finally:
        lib.kvc_destroy(h)


def test_append_and_attend_reject_before_any_launch(kvc):
    rc, h = _create(kvc, L=2, B=3, Hq=4, Hkv=2, D=32, max_len=8, dtype=2)
    assert rc == kvc.OK
    lib = kvc.lib()
    p = _BASE
    try:
        assert lib.kvc_append(h, 2, p, p, 0, 1, None) == kvc.ERR_ARG         # layer out of range
        assert lib.kvc_append(h, -1, p, p, 0, 1, None) == kvc.ERR_ARG
        assert lib.kvc_append(h, 0, p, p, 0, 0, None) == kvc.ERR_ARG         # T < 1
        assert lib.kvc_append(h, 0, None, p, 0, 1, None) == kvc.ERR_ARG
        assert lib.kvc_append(h, 0, p + 4, p, 0, 1, None) == kvc.ERR_ARG     # misaligned input
        assert lib.kvc_append(h, 0, p, p, 5, 1, None) == kvc.ERR_DTYPE
        assert lib.kvc_append(h, 0, p, p, 0, 9, None) == kvc.ERR_CAPACITY    # 0 + 9 > max_len 8
        out = p
        assert lib.kvc_attend(h, 0, p, 2, 1, out, None) == kvc.ERR_STATE     # nothing appended yet
        assert lib.kvc_attend(h, 3, p, 2, 1, out, None) == kvc.ERR_ARG
        assert lib.kvc_attend(h, 0, p, 2, 0, out, None) == kvc.ERR_ARG
        assert lib.kvc_attend(h, 0, p, 9, 1, out, None) == kvc.ERR_DTYPE
        assert lib.kvc_attend(h, 0, None, 2, 1, out, None) == kvc.ERR_ARG
        lens = (ctypes.c_int64 * 3)()
        assert lib.kvc_seq_len(h, 0, lens) == kvc.OK and list(lens) == [0, 0, 0]   # nothing changed
    finally:
        lib.kvc_destroy(h)


def test_rope_calls_reject_before_any_launch(kvc):
    rc, h = _create(kvc, L=2, B=3, Hq=4, Hkv=2, D=32, max_len=8, dtype=2)
    assert rc == kvc.OK
    lib = kvc.lib()
    p = _BASE
    try:
        for base in (0.0, -10.0, float("inf"), float("nan")):
            assert lib.kvc_append_rope(h, 0, p, p, 0, 1, base, None) == kvc.ERR_ARG
            assert lib.kvc_rope_q(h, 0, p, 0, 1, base, None) == kvc.ERR_ARG
        assert lib.kvc_append_rope(h, 2, p, p, 0, 1, 1e4, None) == kvc.ERR_ARG       # layer out of range
        assert lib.kvc_append_rope(h, 0, p, p, 0, 9, 1e4, None) == kvc.ERR_CAPACITY
        assert lib.kvc_append_rope(h, 0, p, p, 7, 1, 1e4, None) == kvc.ERR_DTYPE
        assert lib.kvc_rope_q(h, 0, p, 2, 1, 1e4, None) == kvc.ERR_STATE             # nothing appended yet
        assert lib.kvc_rope_q(h, 0, None, 2, 1, 1e4, None) == kvc.ERR_ARG
        assert lib.kvc_rope_q(h, 0, p + 2, 2, 1, 1e4, None) == kvc.ERR_ARG           # misaligned
        assert lib.kvc_rope_q(h, 0, p, 2, 0, 1e4, None) == kvc.ERR_ARG               # T < 1
        assert lib.kvc_rope_q(None, 0, p, 2, 1, 1e4, None) == kvc.ERR_ARG
        lens = (ctypes.c_int64 * 3)()
        assert lib.kvc_seq_len(h, 0, lens) == kvc.OK and list(lens) == [0, 0, 0]
    finally:
        lib.kvc_destroy(h)


def test_null_handles(kvc):
    lib = kvc.lib()
    lens = (ctypes.c_int64 * 1)()
    nb = ctypes.c_uint64()
    assert lib.kvc_seq_len(None, -1, lens) == kvc.ERR_ARG
    assert lib.kvc_nbytes(None, ctypes.byref(nb)) == kvc.ERR_ARG
    assert lib.kvc_truncate(None, lens, 1) == kvc.ERR_ARG
    assert lib.kvc_append(None, 0, _BASE, _BASE, 0, 1, None) == kvc.ERR_ARG
    assert lib.kvc_attend(None, 0, _BASE, 0, 1, _BASE, None) == kvc.ERR_ARG
    lib.kvc_destroy(None)


def test_nbytes_matches_page_figures(kvc):
    """256 KiB for B=1, L=4, 128 positions, 2 KV heads of width 32 in fp32
    ("Heads, GQA and K/V cache", Memory and the window limit); 64 bytes for the
    worked example would need d_head 2, which the kernels do not take."""
    rc, h = _create(kvc, L=4, B=1, Hq=4, Hkv=2, D=32, max_len=128, dtype=0, store=1 << 17)
    assert rc == kvc.OK
    nb = ctypes.c_uint64()
    assert kvc.lib().kvc_nbytes(h, ctypes.byref(nb)) == kvc.OK
    assert nb.value == 262144
    kvc.lib().kvc_destroy(h)


def _latent_create(kvc, L=2, B=3, r=64, dR=16, max_len=8, dtype=2, c_bytes=None, kr_bytes=None, base=None):
    lib = kvc.lib()
    cfg = kvc.KVCLatentConfig(L, B, r, dR, dtype, max_len)
    item = 4 if dtype == 0 else 2
    cb = c_bytes if c_bytes is not None else L * B * max_len * r * item
    kb = kr_bytes if kr_bytes is not None else L * B * max_len * dR * item
    h = ctypes.c_void_p()
    p = _BASE if base is None else base
    rc = lib.kvc_latent_create(ctypes.byref(cfg), p, p, cb, kb, ctypes.byref(h))
    return rc, h


def test_latent_cache_abi(kvc):
    """Creation checks, nbytes = L B N_max (r + d_R) itemsize ("KV cache, ...",
    section 2.6), per-layer lengths, truncate bounds, append errors before any
    launch."""
    lib = kvc.lib()
    assert _latent_create(kvc, r=60)[0] == kvc.ERR_ARG            # not a multiple of 8
    assert _latent_create(kvc, dR=0)[0] == kvc.ERR_ARG
    assert _latent_create(kvc, dtype=9)[0] == kvc.ERR_DTYPE
    assert _latent_create(kvc, c_bytes=10)[0] == kvc.ERR_STORAGE
    assert _latent_create(kvc, base=_BASE + 4)[0] == kvc.ERR_STORAGE
    rc, h = _latent_create(kvc, L=60, B=1, r=512, dR=64, max_len=4096, dtype=1)
    assert rc == kvc.OK
    nb = ctypes.c_uint64()
    assert lib.kvc_latent_nbytes(h, ctypes.byref(nb)) == kvc.OK and nb.value == 283115520
    lib.kvc_latent_destroy(h)
    rc, h = _latent_create(kvc)
    assert rc == kvc.OK
    p = _BASE
    try:
        assert lib.kvc_latent_append(h, 2, p, p, 0, 1, None) == kvc.ERR_ARG       # layer out of range
        assert lib.kvc_latent_append(h, 0, p, p, 0, 0, None) == kvc.ERR_ARG       # T < 1
        assert lib.kvc_latent_append(h, 0, p + 4, p, 0, 1, None) == kvc.ERR_ARG   # misaligned
        assert lib.kvc_latent_append(h, 0, p, p, 6, 1, None) == kvc.ERR_DTYPE
        assert lib.kvc_latent_append(h, 0, p, p, 0, 9, None) == kvc.ERR_CAPACITY
        lens = (ctypes.c_int64 * 3)()
        assert lib.kvc_latent_seq_len(h, -1, lens) == kvc.OK and list(lens) == [0, 0, 0]
        assert lib.kvc_latent_seq_len(h, 2, lens) == kvc.ERR_ARG
        one = (ctypes.c_int64 * 1)(1)
        assert lib.kvc_latent_truncate(h, one, 1) == kvc.ERR_STATE                # beyond the committed length
        zero = (ctypes.c_int64 * 1)(0)
        assert lib.kvc_latent_truncate(h, zero, 1) == kvc.OK
        assert lib.kvc_latent_truncate(h, zero, 2) == kvc.ERR_ARG                 # count neither 1 nor B
        assert lib.kvc_latent_nbytes(None, ctypes.byref(nb)) == kvc.ERR_ARG
    finally:
        lib.kvc_latent_destroy(h)
    lib.kvc_latent_destroy(None)


def test_paged_create_validation(kvc):
    """kvc_create_paged rejects bad shapes, block sizes and pools before it
    touches the device; the paged queries reject a contiguous-less call."""
    lib = kvc.lib()
    h = ctypes.c_void_p()
    buf = ctypes.create_string_buffer(64)
    p = (ctypes.addressof(buf) + 15) & ~15          # aligned, never dereferenced

    def create(block_size, n_blocks, D=128, dtype=kvc.BF16, nbytes=1 << 40, pool=p, cfg=True):
        c = kvc.KVCConfig(2, 4, 8, 2, D, dtype, 1000)
        return lib.kvc_create_paged(ctypes.byref(c) if cfg else None, block_size, n_blocks, pool, pool,
                                    nbytes, ctypes.byref(h))

    assert create(128, 8, cfg=False) == kvc.ERR_ARG
    for bs in (0, 32, 96, 100, 8192):                 # below 64, not a power of two, above 4096
        assert create(bs, 8) == kvc.ERR_ARG, bs
    assert create(128, 0) == kvc.ERR_ARG
    assert create(128, 8, dtype=7) == kvc.ERR_DTYPE
    assert create(128, 8, D=48) == kvc.ERR_UNSUPPORTED
    # the decode kernels read at most 32 keys per batch at d_head 32 (16-bit
    # caches: 32-key tiles; fp32: 4 waves x 8 keys), so 64-position blocks pass
    # the shape checks; the host buffer then fails as a pool
    for dt in (kvc.F32, kvc.F16, kvc.BF16):
        assert create(64, 8, D=32, dtype=dt) == kvc.ERR_STORAGE
    # max_len * d_head must stay below 2^31, as for a contiguous cache
    def create_long(max_len, D):
        c = kvc.KVCConfig(1, 1, 2, 2, D, kvc.BF16, max_len)
        return lib.kvc_create_paged(ctypes.byref(c), 4096, 8, p, p, 1 << 40, ctypes.byref(h))
    assert create_long((1 << 24), 128) == kvc.ERR_ARG
    assert create_long((1 << 24) - 1, 128) == kvc.ERR_STORAGE
    assert create(128, 8, pool=None) == kvc.ERR_STORAGE
    assert create(128, 8, pool=p + 4) == kvc.ERR_STORAGE
    need_each = 2 * 8 * 2 * 128 * 128 * 2               # L * n_blocks * H_kv * block * d_head * 2 bytes
    assert create(128, 8, nbytes=need_each - 1) == kvc.ERR_STORAGE
    used, total = ctypes.c_int32(), ctypes.c_int32()
    assert lib.kvc_paged_blocks(None, ctypes.byref(used), ctypes.byref(total)) == kvc.ERR_ARG
    tab = (ctypes.c_int32 * 4)()
    assert lib.kvc_block_table(None, tab, 4) == kvc.ERR_ARG


def test_append_attend_rejects_before_any_launch(kvc):
    """kvc_append_attend checks every argument of both halves first."""
    rc, h = _create(kvc, dtype=2)
    assert rc == kvc.OK
    lib = kvc.lib()
    p = _BASE
    out = ctypes.c_void_p(_BASE)
    assert lib.kvc_append_attend(None, 0, p, p, 2, p, 2, 1, out, None) == kvc.ERR_ARG
    assert lib.kvc_append_attend(h, 0, None, p, 2, p, 2, 1, out, None) == kvc.ERR_ARG
    assert lib.kvc_append_attend(h, 0, p, p, 2, None, 2, 1, out, None) == kvc.ERR_ARG
    assert lib.kvc_append_attend(h, 2, p, p, 2, p, 2, 1, out, None) == kvc.ERR_ARG       # layer out of range
    assert lib.kvc_append_attend(h, 0, p, p, 2, p, 2, 0, out, None) == kvc.ERR_ARG       # T < 1
    assert lib.kvc_append_attend(h, 0, p, p, 9, p, 2, 1, out, None) == kvc.ERR_DTYPE
    assert lib.kvc_append_attend(h, 0, p, p, 2, p, 9, 1, out, None) == kvc.ERR_DTYPE
    assert lib.kvc_append_attend(h, 0, p + 8, p, 2, p, 2, 1, out, None) == kvc.ERR_ARG   # misaligned
    assert lib.kvc_append_attend(h, 0, p, p, 2, p, 2, 9, out, None) == kvc.ERR_CAPACITY  # max_len 8
    lens = (ctypes.c_int64 * 3)()
    assert lib.kvc_seq_len(h, 0, lens) == kvc.OK and list(lens) == [0, 0, 0]
    lib.kvc_destroy(h)


def test_host_storage_launches_nothing(kvc):
    """A handle over storage that is not device memory keeps metadata but every
    call that would enqueue device work returns KVC_ERR_STORAGE, after its
    argument checks, and changes nothing (no kernel can touch host memory)."""
    rc, h = _create(kvc, L=2, B=3, Hq=4, Hkv=2, D=32, max_len=8, dtype=2)
    assert rc == kvc.OK
    lib = kvc.lib()
    p = _BASE
    lens = (ctypes.c_int64 * 3)()
    try:
        assert lib.kvc_append(h, 0, p, p, 2, 1, None) == kvc.ERR_STORAGE
        assert lib.kvc_append(h, 0, p, p, 2, 9, None) == kvc.ERR_CAPACITY     # argument checks come first
        assert lib.kvc_append_rope(h, 0, p, p, 2, 1, ctypes.c_double(1e4), None) == kvc.ERR_STORAGE
        assert lib.kvc_append_attend(h, 0, p, p, 2, p, 2, 1, ctypes.c_void_p(p), None) == kvc.ERR_STORAGE
        assert lib.kvc_append_attend(h, 0, p, p, 0, p, 2, 1, ctypes.c_void_p(p), None) == kvc.ERR_STORAGE
        assert lib.kvc_gather(h, 0, 4, p, p, None) == kvc.ERR_STORAGE
        assert lib.kvc_seq_len(h, 0, lens) == kvc.OK and list(lens) == [0, 0, 0]
        used = ctypes.c_uint64()
        assert lib.kvc_nbytes(h, ctypes.byref(used)) == kvc.OK
        n0 = (ctypes.c_int64 * 1)(0)
        assert lib.kvc_truncate(h, n0, 1) == kvc.OK
    finally:
        lib.kvc_destroy(h)


def test_gather_rejects_bad_arguments(kvc):
    rc, h = _create(kvc, L=2, B=3, Hq=4, Hkv=2, D=32, max_len=8, dtype=2)
    assert rc == kvc.OK
    lib = kvc.lib()
    p = _BASE
    try:
        assert lib.kvc_gather(None, 0, 4, p, p, None) == kvc.ERR_ARG
        assert lib.kvc_gather(h, 2, 4, p, p, None) == kvc.ERR_ARG          # layer out of range
        assert lib.kvc_gather(h, -1, 4, p, p, None) == kvc.ERR_ARG
        assert lib.kvc_gather(h, 0, 0, p, p, None) == kvc.ERR_ARG          # n < 1
        assert lib.kvc_gather(h, 0, 9, p, p, None) == kvc.ERR_ARG          # n > max_len
        assert lib.kvc_gather(h, 0, 4, None, p, None) == kvc.ERR_ARG
        assert lib.kvc_gather(h, 0, 4, p, p + 8, None) == kvc.ERR_ARG      # misaligned
    finally:
        lib.kvc_destroy(h)


def test_prefill_precision_setting(kvc):
    """kvc_set_prefill_precision takes the two declared modes on any handle
    (host state only) and rejects a null handle or an unknown mode, leaving the
    setting as it was."""
    lib = kvc.lib()
    assert (kvc.PREFILL_P_ROUNDED, kvc.PREFILL_P_SPLIT) == (0, 1)
    text = open(HEADER).read()
    assert re.search(r"KVC_PREFILL_P_ROUNDED\s*=\s*0", text) and re.search(r"KVC_PREFILL_P_SPLIT\s*=\s*1", text)
    rc, h = _create(kvc)
    assert rc == kvc.OK
    try:
        assert lib.kvc_set_prefill_precision(h, kvc.PREFILL_P_SPLIT) == kvc.OK
        assert lib.kvc_set_prefill_precision(h, kvc.PREFILL_P_ROUNDED) == kvc.OK
        for bad in (2, -1, 99):
            assert lib.kvc_set_prefill_precision(h, bad) == kvc.ERR_ARG
        assert lib.kvc_set_prefill_precision(None, kvc.PREFILL_P_SPLIT) == kvc.ERR_ARG
    finally:
        lib.kvc_destroy(h)
