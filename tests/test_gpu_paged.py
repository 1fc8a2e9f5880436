"""The paged cache (kvc_create_paged) on the GPU.

"KV cache, incremental decode, ..." (Key takeaways) makes the point of the
rounding contract that a float16 paged cache compares exactly with the
contiguous one; "kv-cache-decoding" ("Batching caches of different lengths")
describes the paged layout: fixed-size blocks, a table per request, a block
taken when a sequence grows into it and freed when it ends.

Bars: with the same calls, a paged and a contiguous cache hold the same bits at
every filled position, and attention outputs are bit-identical, since both
run the same kernel with a work split that depends only on the lengths.
Every shape against the oracle is held to the oracle's tolerances. Block accounting is exact: blocks in use = sum over rows of
ceil(held length / block_size), no block in two places.
"""
import numpy as np
import pytest

from oracle import OracleCache, storage_bits
from tests.harness import FP32_MAX_ABS, HALF_REL_FROB, compare_out, gpu_bits, log, to_device

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_cached_gqa_amd import kvc  # noqa: F401  (fails loudly if libkvc.so is missing)
    yield
    torch.cuda.synchronize()


def _pair(L, B, Hq, Hkv, D, max_len, dtype, block_size, n_blocks=None):
    from kv_cached_gqa_amd.kvc import KVCache, PagedKVCache
    return (KVCache(L, Hkv, D, max_len, batch=B, n_q_heads=Hq, dtype=dtype, device=DEV),
            PagedKVCache(L, Hkv, D, max_len, batch=B, n_q_heads=Hq, dtype=dtype, device=DEV,
                         block_size=block_size, n_blocks=n_blocks))


def _check_table(pc):
    """Held blocks are distinct, in range, a prefix of each row's table, and
    exactly as many as the longest layer fill needs."""
    tab = pc.block_table()
    used, total = pc.blocks()
    held = tab[tab >= 0]
    assert len(np.unique(held)) == held.size and held.size == used
    assert held.min(initial=0) >= 0 and held.max(initial=0) < total
    fills = np.max([pc.seq_len(layer) for layer in range(pc.n_layers)], axis=0)
    for b in range(pc.batch):
        n = int((tab[b] >= 0).sum())
        assert (tab[b, :n] >= 0).all() and (tab[b, n:] < 0).all()
        assert n == -(-int(fills[b]) // pc.block_size), (b, n, fills[b])


def _same_storage(cc, pc, layers):
    import torch
    torch.cuda.synchronize()
    for layer in layers:
        lens = cc.seq_len(layer)
        kp, vp = pc.gather(layer)
        for b, n in enumerate(lens):
            n = int(n)
            assert np.array_equal(gpu_bits(kp[b, :, :n]), gpu_bits(cc.k_storage[layer, b, :, :n])), (layer, b)
            assert np.array_equal(gpu_bits(vp[b, :, :n]), gpu_bits(cc.v_storage[layer, b, :, :n])), (layer, b)


def _both_append(cc, pc, layer, k, v, inp="fp32"):
    kd, vd = to_device(k, inp, DEV), to_device(v, inp, DEV)
    cc.append(layer, kd, vd)
    pc.append(layer, kd, vd)


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("D", [32, 64, 128])
def test_paged_equals_contiguous_bit_exact(dtype, D):
    """Ragged rows across block edges, decode steps, chunks, truncates that free
    and regrow blocks: the same stored bits and bit-identical attention outputs
    on every kernel (16-bit storage: vector, matrix-core decode and prefill;
    fp32: vector and row-split)."""
    import torch
    rng = np.random.default_rng(900 + D)
    for G in ((8,) if dtype == "fp32" else (4, 8)):
        # 64-position blocks at d_head 32: one block per stage of the fp32
        # row-split kernel (T=3 x G=8 = 24 rows) and two matrix-core tiles
        for bs in ((64, 128, 256) if D == 32 else (128, 256)):
            log(f"paged vs contiguous dtype={dtype} D={D} G={G} block={bs}")
            L, B, Hkv, max_len = 2, 5, 2, 1500
            Hq = G * Hkv
            cc, pc = _pair(L, B, Hq, Hkv, D, max_len, dtype, bs)
            # fill, then give blocks back so the free list comes out of order
            for layer in range(L):
                k, v = (rng.standard_normal((B, Hkv, 700, D), dtype=np.float32) for _ in range(2))
                _both_append(cc, pc, layer, k, v)
            lens = np.array([0, 1, bs - 1, bs, 2 * bs + 1])
            cc.truncate(lens)
            pc.truncate(lens)
            _check_table(pc)
            for step, T in enumerate((1, 1, bs, 1, 3)):
                for layer in range(L):
                    k, v = (rng.standard_normal((B, Hkv, T, D), dtype=np.float32) for _ in range(2))
                    _both_append(cc, pc, layer, k, v, inp="fp32" if step % 2 else "bf16")
                    q = to_device(rng.standard_normal((B, Hq, T, D), dtype=np.float32), "fp32", DEV)
                    oc, op = cc.attend(layer, q), pc.attend(layer, q)
                    torch.cuda.synchronize()
                    assert torch.equal(oc.view(torch.int32), op.view(torch.int32)), (bs, step, layer)
                _check_table(pc)
                if step == 2:
                    cut = np.array([3, 0, bs + 5, 1, 2 * bs])
                    cc.truncate(cut)
                    pc.truncate(cut)
                    _check_table(pc)
            _same_storage(cc, pc, range(L))
            assert pc.nbytes() == 2 * L * pc.n_blocks * Hkv * bs * D * (4 if dtype == "fp32" else 2)
            cc.close()
            pc.close()


def test_paged_long_context_and_prefill_chunks_bit_exact():
    """Matrix-core paths on a paged bf16 cache: 2 rows of 8192 keys with
    H_q=64, H_kv=8 (T=1 and a T=4 draft: 8 and 32 query rows per KV head),
    then four prefill chunks of 512 with H_q=32 (the chunked-prefill shape at
    B=2): bit-identical to the contiguous cache."""
    import torch
    rng = np.random.default_rng(990)
    for (B, Hq, Hkv, D, s0, chunks) in ((2, 64, 8, 128, 8192, (1, 4)), (2, 32, 8, 128, 0, (512,) * 4)):
        log(f"paged matrix-core paths: B={B} Hq={Hq} s0={s0} chunks={chunks}")
        max_len = s0 + sum(chunks)
        cc, pc = _pair(1, B, Hq, Hkv, D, max_len, "bf16", 128)
        if s0:
            k, v = (rng.standard_normal((B, Hkv, s0, D), dtype=np.float32) for _ in range(2))
            _both_append(cc, pc, 0, k, v)
        for T in chunks:
            k, v = (rng.standard_normal((B, Hkv, T, D), dtype=np.float32) for _ in range(2))
            _both_append(cc, pc, 0, k, v)
            q = to_device(rng.standard_normal((B, Hq, T, D), dtype=np.float32), "bf16", DEV)
            oc, op = cc.attend(0, q), pc.attend(0, q)
            torch.cuda.synchronize()
            assert torch.equal(oc.view(torch.int32), op.view(torch.int32)), T
        _check_table(pc)
        _same_storage(cc, pc, [0])
        cc.close()
        pc.close()


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_paged_rows_that_reach_the_last_table_entry(dtype):
    """Rows whose last key sits in the last entry of their table row, rows that
    end exactly at a block edge, one-block rows, and long rows over many small
    blocks: the decode kernels read each block's entry ahead of time (the block
    after next, clamped to the row's table, -1 past the held blocks), which must
    change nothing. Attention outputs bit-identical to the contiguous cache for
    T = 1 and 3 and for 4 and 8 query heads per KV head."""
    import torch
    rng = np.random.default_rng(4242)
    D, Hkv, bs = 128, 2, 64
    for max_len, lens in ((4 * bs, [4 * bs - 1, 2 * bs - 1, bs - 1, 199]), (4096, [4095, 4032, 2049, 64])):
        for G in (4, 8):
            for T in (1, 3):
                log(f"paged table edges dtype={dtype} max_len={max_len} G={G} T={T}")
                B, Hq = len(lens), G * Hkv
                cc, pc = _pair(1, B, Hq, Hkv, D, max_len, dtype, bs)
                k, v = (rng.standard_normal((B, Hkv, max_len - T, D), dtype=np.float32) for _ in range(2))
                _both_append(cc, pc, 0, k, v, inp="bf16")
                cut = np.minimum(np.array(lens) + 1 - T, max_len - T)
                cc.truncate(cut)
                pc.truncate(cut)
                k, v = (rng.standard_normal((B, Hkv, T, D), dtype=np.float32) for _ in range(2))
                _both_append(cc, pc, 0, k, v)
                _check_table(pc)
                q = to_device(rng.standard_normal((B, Hq, T, D), dtype=np.float32), "bf16", DEV)
                oc, op = cc.attend(0, q), pc.attend(0, q)
                torch.cuda.synchronize()
                assert torch.equal(oc.view(torch.int32), op.view(torch.int32)), (max_len, G, T)
                assert np.isfinite(oc.cpu().numpy()).all()
                cc.close()
                pc.close()


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_paged_groups_and_chunks_against_the_oracle(dtype):
    """Group sizes 1..16 and chunks T = 1..9 (slabs of up to 8 query rows per
    KV head, several slabs per call) on a paged cache, against the oracle."""
    rng = np.random.default_rng(950)
    D, B, max_len, bs = 64, 4, 700, 128
    for (Hq, Hkv) in ((2, 2), (6, 2), (16, 1), (24, 3)):
        log(f"paged vs oracle dtype={dtype} Hq={Hq} Hkv={Hkv}")
        from kv_cached_gqa_amd.kvc import PagedKVCache
        pc = PagedKVCache(1, Hkv, D, max_len, batch=B, n_q_heads=Hq, dtype=dtype, device=DEV, block_size=bs)
        orc = OracleCache(1, B, Hq, Hkv, D, max_len, dtype)
        k, v = (rng.standard_normal((B, Hkv, 600, D), dtype=np.float32) for _ in range(2))
        pc.append(0, to_device(k, "fp32", DEV), to_device(v, "fp32", DEV))
        orc.append(0, k, v)
        pre = np.array([0, 127, 128, 555])
        pc.truncate(pre)
        orc.truncate(pre)
        for T in (1, 3, 9, 1, 40):
            q, k, v = (rng.standard_normal(s, dtype=np.float32) for s in
                       ((B, Hq, T, D), (B, Hkv, T, D), (B, Hkv, T, D)))
            pc.append(0, to_device(k, "fp32", DEV), to_device(v, "fp32", DEV))
            orc.append(0, k, v)
            got = pc.attend(0, to_device(q, "fp32", DEV)).cpu().numpy()
            want = orc.attend(0, q)
            mabs, rel = compare_out(got, want, dtype)
            assert np.isfinite(got).all()
            if dtype == "fp32":
                assert mabs <= FP32_MAX_ABS, (Hq, Hkv, T, mabs)
            else:
                assert rel <= HALF_REL_FROB, (Hq, Hkv, T, rel)
        kp, vp = pc.gather(0)
        lens = orc.seq_len(0)
        for b in range(B):
            n = int(lens[b])
            assert np.array_equal(gpu_bits(kp[b, :, :n]), storage_bits(orc.K[0, b, :, :n], dtype))
            assert np.array_equal(gpu_bits(vp[b, :, :n]), storage_bits(orc.V[0, b, :, :n], dtype))
        _check_table(pc)
        pc.close()


def test_paged_blocks_are_taken_on_growth_and_given_back():
    """A pool smaller than B * max_len: a finished row's blocks go to a growing
    one; an append the pool cannot cover fails with nothing changed."""
    import torch
    from kv_cached_gqa_amd.kvc import ContextLimitError, PagedKVCache
    log("paged block accounting")
    rng = np.random.default_rng(970)
    L, B, Hq, Hkv, D, max_len, bs = 2, 3, 4, 2, 128, 2048, 128
    pc = PagedKVCache(L, Hkv, D, max_len, batch=B, n_q_heads=Hq, dtype="bf16", device=DEV, block_size=bs,
                      n_blocks=10)
    orc = OracleCache(L, B, Hq, Hkv, D, max_len, "bf16")
    assert pc.blocks() == (0, 10)

    def app(T):
        for layer in range(L):
            k, v = (rng.standard_normal((B, Hkv, T, D), dtype=np.float32) for _ in range(2))
            pc.append(layer, to_device(k, "fp32", DEV), to_device(v, "fp32", DEV))
            orc.append(layer, k, v)

    app(300)                                  # 3 blocks per row
    assert pc.blocks() == (9, 10)
    pc.truncate(np.array([300, 0, 129]))      # row 1 ends: its 3 blocks return; row 2 keeps 2
    orc.truncate(np.array([300, 0, 129]))
    assert pc.blocks() == (5, 10)
    _check_table(pc)
    app(100)                                  # rows: 400 (4), 100 (1), 229 (2) = 7 blocks
    assert pc.blocks() == (7, 10)
    _check_table(pc)
    before = (pc.block_table().copy(), pc.seq_len().copy(), pc.blocks())
    k = to_device(rng.standard_normal((B, Hkv, 300, D), dtype=np.float32), "fp32", DEV)
    with pytest.raises(ContextLimitError):
        pc.append(0, k, k)                    # needs 2 + 3 + 3 = 8 more blocks, 3 free
    assert np.array_equal(pc.block_table(), before[0]) and np.array_equal(pc.seq_len(), before[1])
    assert pc.blocks() == before[2]
    q = rng.standard_normal((B, Hq, 1, D), dtype=np.float32)
    app(1)
    for layer in range(L):
        got = pc.attend(layer, to_device(q, "fp32", DEV)).cpu().numpy()
        _, rel = compare_out(got, orc.attend(layer, q), "bf16")
        assert rel <= HALF_REL_FROB
    torch.cuda.synchronize()
    pc.truncate(0)
    assert pc.blocks() == (0, 10)
    pc.close()


@pytest.mark.parametrize("st", ["fp16", "bf16"])
def test_paged_rope_equals_contiguous(st):
    """Keys stored rotated at their slots: the same bits in a paged cache."""
    import torch
    rng = np.random.default_rng(980)
    L, B, Hq, Hkv, D, max_len = 1, 3, 8, 2, 128, 900
    cc, pc = _pair(L, B, Hq, Hkv, D, max_len, st, 128)
    for T in (200, 1, 130):
        k, v = (rng.standard_normal((B, Hkv, T, D), dtype=np.float32) for _ in range(2))
        kd, vd = to_device(k, "fp32", DEV), to_device(v, "fp32", DEV)
        cc.append(0, kd, vd, rope_base=10000.0)
        pc.append(0, kd, vd, rope_base=10000.0)
    q = to_device(rng.standard_normal((B, Hq, 1, D), dtype=np.float32), st, DEV)
    oc = cc.attend(0, cc.rope_q(0, q.clone(), 10000.0))
    op = pc.attend(0, pc.rope_q(0, q.clone(), 10000.0))
    torch.cuda.synchronize()
    assert torch.equal(oc.view(torch.int32), op.view(torch.int32))
    _same_storage(cc, pc, [0])
    cc.close()
    pc.close()


def test_paged_batched_decode_full_size():
    """B=32, H_q=32, H_kv=8, d_h=128, bf16, lengths U{1024..4095}, T=1, blocks of
    128: a decode step on the paged cache is bit-identical to the contiguous
    cache's and both hold the same bits."""
    import torch
    from kv_cached_gqa_amd import workloads as W
    log("paged batched decode bf16 B=32, full size")
    shape, calls = W.script_batched_decode(n_steps=1)
    cc, pc = _pair(shape.n_layers, shape.batch, shape.n_q_heads, shape.n_kv_heads, shape.d_head, shape.max_len,
                   shape.dtype, 128)
    for call in calls:
        if call.op in ("append", "pass"):
            _both_append(cc, pc, call.layer, call.k, call.v)
        if call.op == "pass":
            q = to_device(call.q, "bf16", DEV)
            oc, op = cc.attend(call.layer, q), pc.attend(call.layer, q)
            torch.cuda.synchronize()
            assert torch.equal(oc.view(torch.int32), op.view(torch.int32)), call.tag
        if call.op == "truncate":
            cc.truncate(call.n)
            pc.truncate(call.n)
    _check_table(pc)
    _same_storage(cc, pc, range(shape.n_layers))
    cc.close()
    pc.close()


def test_paged_batch_wider_than_one_launch():
    """B=300 rows (two launches of at most 256 rows; the second launch's table
    starts at row 256), ragged lengths: the vector kernel (2 rows per KV head),
    the matrix-core decode kernel (8 rows) and the prefill kernel (a 24-position
    chunk at 8 heads per group) give the contiguous cache's bits."""
    import torch
    log("paged B=300 rows")
    rng = np.random.default_rng(995)
    B, Hkv, D, max_len = 300, 2, 64, 330
    for G in (2, 8):
        cc, pc = _pair(1, B, G * Hkv, Hkv, D, max_len, "bf16", 64)
        k, v = (rng.standard_normal((B, Hkv, 290, D), dtype=np.float32) for _ in range(2))
        _both_append(cc, pc, 0, k, v)
        lens = rng.integers(0, 291, size=B)
        cc.truncate(lens)
        pc.truncate(lens)
        for T in (1, 24, 1):
            k, v = (rng.standard_normal((B, Hkv, T, D), dtype=np.float32) for _ in range(2))
            _both_append(cc, pc, 0, k, v)
            q = to_device(rng.standard_normal((B, G * Hkv, T, D), dtype=np.float32), "bf16", DEV)
            oc, op = cc.attend(0, q), pc.attend(0, q)
            torch.cuda.synchronize()
            assert torch.equal(oc.view(torch.int32), op.view(torch.int32)), (G, T)
        _check_table(pc)
        _same_storage(cc, pc, [0])
        cc.close()
        pc.close()
