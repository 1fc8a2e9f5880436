"""Parity of the HIP path (through the C ABI binding) with the CPU oracle.

Run on an MI355X: python -u -m pytest tests -m gpu -x -v --timeout 120 --timeout-method thread
"""
import numpy as np
import pytest

from oracle import OracleCache, round_to_storage
from kv_cached_gqa_amd import workloads as W
from tests.harness import (FP32_MAX_ABS, HALF_REL_FROB, cache_bits_equal, compare_out, gpu_bits,
                           input_values, log, run_script, to_device)

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


def _new(shape_args, dtype):
    from kv_cached_gqa_amd.kvc import KVCache
    L, B, Hq, Hkv, D, max_len = shape_args
    return (KVCache(L, Hkv, D, max_len, batch=B, n_q_heads=Hq, dtype=dtype, device=DEV),
            OracleCache(L, B, Hq, Hkv, D, max_len, dtype))


def _edge_values(rng, n):
    special = np.array([0.0, -0.0, 65504.0, 65519.0, 65520.0, -7e4, 1e-8, -6e-8, 3e-5, 1.0 + 2 ** -9,
                        1.0 + 3 * 2 ** -9, 3.3e38, -3.4e38, np.inf, -np.inf, np.nan, 2.0 ** -130],
                       dtype=np.float32)
    bits = rng.integers(0, 2 ** 32, size=n, dtype=np.uint64).astype(np.uint32).view(np.float32)
    x = np.concatenate([special, bits, rng.standard_normal(n, dtype=np.float32)])
    return x


@pytest.mark.parametrize("st", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("inp", ["fp32", "fp16", "bf16"])
def test_append_bit_exact(st, inp):
    log(f"append bit-exact st={st} in={inp}")
    rng = np.random.default_rng(100)
    L, B, Hq, Hkv, D, max_len = 2, 3, 4, 2, 64, 40
    cache, orc = _new((L, B, Hq, Hkv, D, max_len), st)
    for T in (5, 1, 16, 3):
        for layer in range(L):
            n = B * Hkv * T * D
            vals = _edge_values(rng, n)[:n]
            k = rng.permutation(vals).reshape(B, Hkv, T, D).astype(np.float32)
            v = rng.permutation(vals).reshape(B, Hkv, T, D).astype(np.float32)
            cache.append(layer, to_device(k, inp, DEV), to_device(v, inp, DEV))
            orc.append(layer, input_values(k, inp), input_values(v, inp))
    import torch
    torch.cuda.synchronize()
    assert cache_bits_equal(cache, orc)
    assert np.array_equal(cache.seq_len(), orc.seq_len())


def test_append_touches_only_its_slots_and_attend_reads_only_filled():
    """Canaries: every slot not yet appended holds NaN; an append changes only
    [fill, fill + T) and attention stays finite (nothing reads past the fill)."""
    import torch
    log("canary append/attend")
    rng = np.random.default_rng(101)
    L, B, Hq, Hkv, D, max_len = 2, 4, 8, 2, 128, 96
    cache, orc = _new((L, B, Hq, Hkv, D, max_len), "bf16")
    cache.k_storage.fill_(float("nan"))
    cache.v_storage.fill_(float("nan"))
    torch.cuda.synchronize()
    canary = gpu_bits(cache.k_storage).copy()
    for step, T in enumerate((7, 1, 1, 13, 2)):
        for layer in range(L):
            q, k, v = (rng.standard_normal(s, dtype=np.float32) for s in
                       ((B, Hq, T, D), (B, Hkv, T, D), (B, Hkv, T, D)))
            cache.append(layer, to_device(k, "fp32", DEV), to_device(v, "fp32", DEV))
            orc.append(layer, k, v)
            out = cache.attend(layer, to_device(q, "bf16", DEV)).cpu().numpy()
            assert np.isfinite(out).all()
            want = orc.attend(layer, input_values(q, "bf16"))
            assert compare_out(out, want, "bf16")[1] <= HALF_REL_FROB
    torch.cuda.synchronize()
    kb = gpu_bits(cache.k_storage)
    fill = int(orc.seq_len()[0])
    assert np.array_equal(kb[:, :, :, fill:], canary[:, :, :, fill:])     # untouched past the fill
    assert cache_bits_equal(cache, orc, layer_slice=(slice(None), slice(None), slice(None), slice(0, fill)))


def test_tiny_gqa_fp32_full_script():
    """B=1, L=4, H_q=4, H_kv=2, d_h=32, max_len=128, fp32: prefill 16 then 112
    decode steps to exactly max_len; max-abs <= 1e-5 on every call."""
    log("tiny GQA fp32: 16 + 112 steps x 4 layers")
    shape, calls = W.script_tiny_gqa()
    rep, cache, orc = run_script(shape, calls)
    log(f"  attends={rep.attends} worst abs={rep.worst_abs:.3e}")
    assert rep.ok(), rep.failures[:5]
    assert rep.worst_abs <= FP32_MAX_ABS
    assert int(cache.seq_len()[0]) == 128
    assert cache.nbytes() == 262144
    from kv_cached_gqa_amd.kvc import ContextLimitError
    with pytest.raises(ContextLimitError):
        k = to_device(np.zeros((1, 2, 1, 32), np.float32), "fp32", DEV)
        cache.append(0, k, k)
    assert int(cache.seq_len(0)[0]) == 128


def test_smollm2_fp16_full_script_with_rollback():
    """L=30, H_q=9, H_kv=3, d_h=64, fp16 (x0.5 draws): prefill 512, 256 decode
    steps, truncate back 4, 4 fresh re-decode steps; then a replay check."""
    import torch
    log("SmolLM2-shaped fp16: 512 + 256 steps x 30 layers, rollback 4")
    shape, calls = W.script_smollm2()
    calls = list(calls)
    rep, cache, orc = run_script(shape, calls, check_every_call=False)
    log(f"  attends={rep.attends} worst rel={rep.worst_rel:.3e} ({rep.worst_tag}) abs={rep.worst_abs:.3e}")
    assert rep.ok(), rep.failures[:5]
    assert cache.seq_len().tolist() == [768]
    assert cache.nbytes() == 47185920
    # (i) replay: truncate again and feed the same 4 re-decode chunks: identical bytes and outputs
    before_k = gpu_bits(cache.k_storage).copy()
    redecode = [c for c in calls if c.tag.startswith("redecode")]
    first = []
    cache.truncate(764)
    for c in redecode:
        cache.append(c.layer, to_device(c.k, "fp32", DEV), to_device(c.v, "fp32", DEV))
        first.append(cache.attend(c.layer, to_device(c.q, "fp32", DEV)).cpu().numpy())
    torch.cuda.synchronize()
    assert np.array_equal(gpu_bits(cache.k_storage), before_k)
    cache.truncate(764)
    for c, o in zip(redecode, first):
        cache.append(c.layer, to_device(c.k, "fp32", DEV), to_device(c.v, "fp32", DEV))
        o2 = cache.attend(c.layer, to_device(c.q, "fp32", DEV)).cpu().numpy()
        assert np.array_equal(o, o2)
    # (ii) the rolled-back cache equals one that never saw positions 764..767
    never = OracleCache(shape.n_layers, 1, shape.n_q_heads, shape.n_kv_heads, shape.d_head, shape.max_len, "fp16")
    keep = [c for c in calls if c.op == "pass"]
    pre = [c for c in keep if not c.tag.startswith("redecode")]
    pre = pre[: len(pre) - 4 * shape.n_layers]
    for c in pre:
        never.append(c.layer, c.k, c.v)
    for c in redecode:
        never.append(c.layer, c.k, c.v)
    assert cache_bits_equal(cache, never, layer_slice=(slice(None), slice(None), slice(None), slice(0, 768)))


def test_batched_decode_bf16_full_size():
    """B=32, H_q=32, H_kv=8, d_h=128, bf16, lengths U{1024..4095}, T=1: every
    output row against the oracle."""
    log("batched decode bf16 B=32 ctx U[1024,4095], full size")
    shape, calls = W.script_batched_decode(n_steps=2)
    rep, cache, orc = run_script(shape, calls, kv_dtype="fp32", q_dtype="bf16", compare_cache=True)
    log(f"  attends={rep.attends} worst rel={rep.worst_rel:.3e} abs={rep.worst_abs:.3e}")
    assert rep.ok(), rep.failures[:5]


@pytest.mark.parametrize("D, B", [(64, 64), (32, 128)])
def test_batched_decode_small_heads_full_size(D, B):
    """Batched decode at head dimensions 64 and 32 with the batch scaled so a
    call moves the bytes of the d_h 128 workload (H_q=32, H_kv=8, bf16, lengths
    U{1024..4095}, T=1): the split over every work-group these head dimensions
    run per CU. One step as append + attend and one as the fused call, every
    output row against the oracle, the per-row worst error reported."""
    import torch
    log(f"batched decode bf16 D={D} B={B} ctx U[1024,4095], all rows")
    rng = np.random.default_rng(900 + D)
    Hq, Hkv, max_len = 32, 8, 4096
    lens = W.batched_lengths(rng, B)
    cache, orc = _new((1, B, Hq, Hkv, D, max_len), "bf16")
    k, v = (rng.standard_normal((B, Hkv, max_len - 2, D), dtype=np.float32) for _ in range(2))
    cache.append(0, to_device(k, "fp32", DEV), to_device(v, "fp32", DEV))
    orc.append(0, k, v)
    del k, v
    cache.truncate(lens)
    orc.truncate(lens)
    for step in range(2):
        q, k, v = (rng.standard_normal(s, dtype=np.float32) for s in ((B, Hq, 1, D), (B, Hkv, 1, D), (B, Hkv, 1, D)))
        qv = input_values(q, "bf16")
        qd = torch.from_numpy(qv).to(torch.bfloat16).to(DEV)
        kd, vd = to_device(k, "fp32", DEV), to_device(v, "fp32", DEV)
        if step == 0:
            cache.append(0, kd, vd)
            got = cache.attend(0, qd).cpu().numpy()
        else:
            got = cache.append_attend(0, kd, vd, qd).cpu().numpy()
        orc.append(0, k, v)
        want = orc.attend(0, qv)
        mabs, rel = compare_out(got, want, "bf16")
        diff = (got.astype(np.float64) - want).reshape(B * Hq, D)
        row_rel = np.linalg.norm(diff, axis=1) / np.linalg.norm(want.reshape(B * Hq, D), axis=1)
        log(f"  step {step} ({'append + attend' if step == 0 else 'fused'}): rel {rel:.2e}, "
            f"worst row {row_rel.max():.2e}, max abs {mabs:.2e}")
        assert np.isfinite(got).all() and np.isfinite(want).all()
        assert rel <= HALF_REL_FROB, (D, B, step, rel)
    assert cache_bits_equal(cache, orc)


def test_chunked_prefill_bf16_reduced():
    """B=4, H_q=32, H_kv=8, d_h=128, bf16: four chunks of 512 with the bottom-right mask."""
    log("chunked prefill bf16: 4 chunks of 512")
    shape, calls = W.script_chunked_prefill(n_chunks=4)
    rep, cache, orc = run_script(shape, calls, sample=48)
    log(f"  attends={rep.attends} worst rel={rep.worst_rel:.3e}")
    assert rep.ok(), rep.failures[:5]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_prefill_split_precision(dtype):
    """kvc_set_prefill_precision: the first two chunks of the chunked-prefill
    workload (B=4, H_q=32, H_kv=8, d_h=128, T=512), every row, with P as a hi +
    lo pair, within 1e-4 of the float64 oracle per call (the once-rounded P of
    the default is ~1e-3 on bf16); the paged cache, in the same mode, gives the
    same bits; switching back restores the default kernel's result."""
    import torch
    from kv_cached_gqa_amd.kvc import KVCache, PagedKVCache
    log(f"prefill split precision {dtype}")
    shape, calls = W.script_chunked_prefill(n_chunks=2)
    mk = dict(batch=shape.batch, n_q_heads=shape.n_q_heads, dtype=dtype, device="cuda")
    cache = KVCache(1, shape.n_kv_heads, shape.d_head, shape.max_len, **mk)
    paged = PagedKVCache(1, shape.n_kv_heads, shape.d_head, shape.max_len, block_size=128, **mk)
    orc = OracleCache(1, shape.batch, shape.n_q_heads, shape.n_kv_heads, shape.d_head, shape.max_len, dtype)
    cache.set_prefill_precision("split")
    paged.set_prefill_precision("split")
    for n, call in enumerate(c for c in calls if c.op == "pass"):
        kd, vd = to_device(call.k, "fp32", "cuda"), to_device(call.v, "fp32", "cuda")
        cache.append(0, kd, vd)
        paged.append(0, kd, vd)
        orc.append(0, input_values(call.k, "fp32"), input_values(call.v, "fp32"))
        q = to_device(call.q, dtype, "cuda")
        got = cache.attend(0, q)
        got_paged = paged.attend(0, q)
        cache.set_prefill_precision("rounded")
        got_rounded = cache.attend(0, q)
        cache.set_prefill_precision("split")
        torch.cuda.synchronize()
        want = orc.attend(0, input_values(call.q, dtype))
        _, rel = compare_out(got.cpu().numpy(), want, dtype)
        _, rel_rounded = compare_out(got_rounded.cpu().numpy(), want, dtype)
        log(f"  chunk {n}: split rel {rel:.3e}, rounded rel {rel_rounded:.3e}")
        assert rel <= 1e-4, (n, rel)
        assert rel_rounded <= HALF_REL_FROB and rel < rel_rounded, (n, rel, rel_rounded)
        assert torch.equal(got.view(torch.int32), got_paged.view(torch.int32)), n
    cache.close()
    paged.close()


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("D", [32, 64])
def test_prefill_split_precision_small_heads(dtype, D):
    """The split prefill precision at head dimensions 32 and 64 (the
    SmolLM2-shaped cache's): ragged rows (fills 0, 37 and 300), two chunks of
    T=96 with 3 query heads per KV head, every row within 1e-4 of the oracle."""
    from kv_cached_gqa_amd.kvc import KVCache
    log(f"prefill split precision D={D} {dtype}")
    rng = np.random.default_rng(4100 + D)
    B, Hq, Hkv, T, max_len = 3, 9, 3, 96, 600
    cache = KVCache(1, Hkv, D, max_len, batch=B, n_q_heads=Hq, dtype=dtype, device=DEV)
    orc = OracleCache(1, B, Hq, Hkv, D, max_len, dtype)
    cache.set_prefill_precision("split")
    k, v = (rng.standard_normal((B, Hkv, 300, D), dtype=np.float32) for _ in range(2))
    cache.append(0, to_device(k, "fp32", DEV), to_device(v, "fp32", DEV))
    orc.append(0, k, v)
    fills = np.array([0, 37, 300])
    cache.truncate(fills)
    orc.truncate(fills)
    for n in range(2):
        k, v, q = (rng.standard_normal(s, dtype=np.float32) for s in ((B, Hkv, T, D), (B, Hkv, T, D), (B, Hq, T, D)))
        cache.append(0, to_device(k, "fp32", DEV), to_device(v, "fp32", DEV))
        orc.append(0, k, v)
        got = cache.attend(0, to_device(q, dtype, DEV)).cpu().numpy()
        _, rel = compare_out(got, orc.attend(0, input_values(q, dtype)), dtype)
        log(f"  chunk {n}: split rel {rel:.3e}")
        assert rel <= 1e-4, (n, rel)
    cache.close()


@pytest.mark.timeout(1200)
def test_long_context_speculative_cycles():
    """B=8, H_q=64, H_kv=8, d_h=128, bf16, s0=32768: all 64 draft / accept /
    reset cycles of the configuration. Every row of every call of the first
    and the last cycle, 24 sampled rows (in 4 (row, KV head) units) of every
    other call, fills after every call, and the whole cache bit for bit at the
    end (every slot a cycle wrote past s0 included)."""
    log("long context bf16 s0=32768: 64 speculative cycles")
    shape, calls = W.script_long_ctx_spec(n_cycles=64)
    def first_or_last_cycle(tag):
        return tag in ("draft0", "draft63") or tag.startswith(("decode0.", "decode63."))

    full = lambda n, call: first_or_last_cycle(call.tag)  # noqa: E731
    per_call = []
    rep, cache, orc = run_script(shape, calls, sample=24, sample_groups=4, full_rows_at=full, compare_cache=True,
                                 out_log=per_call, row_errors=True)
    fulls = [c for c in per_call if first_or_last_cycle(c[0])]
    log(f"  attends={rep.attends} (all rows on {len(fulls)}) worst rel={rep.worst_rel:.3e} ({rep.worst_tag}); "
        f"worst per-row rel={max(e for _, _, e in rep.row_errors):.3e}")
    assert rep.ok(), rep.failures[:5]
    assert rep.attends == sum(1 for _ in W.script_long_ctx_spec(n_cycles=64)[1] if _.op == "pass")
    assert cache.seq_len().tolist() == [32768] * 8
    assert len(fulls) >= 4


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("D", [32, 64, 128])
def test_ragged_rows_groups_and_chunks(dtype, D):
    """Rows of lengths 1..300, group sizes 1..16 (slabs across heads), chunks
    T = 1..9 (slabs across positions)."""
    log(f"ragged dtype={dtype} D={D}")
    rng = np.random.default_rng(200 + D)
    for (Hq, Hkv) in ((2, 2), (6, 2), (9, 3), (16, 1), (24, 3)):
        B, max_len = 6, 320
        cache, orc = _new((1, B, Hq, Hkv, D, max_len), dtype)
        pre = np.array([0, 1, 63, 64, 65, 299])
        k, v = (rng.standard_normal((B, Hkv, 300, D), dtype=np.float32) for _ in range(2))
        cache.append(0, to_device(k, "fp32", DEV), to_device(v, "fp32", DEV))
        orc.append(0, k, v)
        cache.truncate(pre)
        orc.truncate(pre)
        for T in (1, 3, 9, 1):
            q, k, v = (rng.standard_normal(s, dtype=np.float32) for s in
                       ((B, Hq, T, D), (B, Hkv, T, D), (B, Hkv, T, D)))
            cache.append(0, to_device(k, "fp32", DEV), to_device(v, "fp32", DEV))
            orc.append(0, k, v)
            got = cache.attend(0, to_device(q, "fp32", DEV)).cpu().numpy()
            want = orc.attend(0, q)
            mabs, rel = compare_out(got, want, dtype)
            if dtype == "fp32":
                assert mabs <= FP32_MAX_ABS, (Hq, Hkv, T, mabs)
            else:
                assert rel <= HALF_REL_FROB, (Hq, Hkv, T, rel)
        assert cache_bits_equal(cache, orc)


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("D", [32, 64, 128])
def test_decode_slabs_split_over_many_work_groups(dtype, D):
    """Decode slabs of 4..32 query rows per KV head over contexts of thousands of
    keys, so that one (row, KV head) spans many work-groups and one work-group's
    slice crosses unit boundaries: 16-bit caches take the matrix-core decode
    kernel from 5 rows on, fp32 caches the row-split kernel above 8 rows. A row
    that starts empty gets only the chunk's own keys."""
    log(f"decode split slabs dtype={dtype} D={D}")
    rng = np.random.default_rng(700 + D)
    #          B  Hq  Hkv T   context lengths before the chunk
    cases = ((2, 8, 1, 4, (9001, 2999)),        # 32 rows
             (3, 10, 2, 1, (4096, 1, 6143)),    # 5 rows
             (4, 12, 4, 2, (0, 2050, 3333, 777)),  # 6 rows
             (1, 32, 2, 1, (12000,)),           # 16 rows, two long units
             (3, 4, 4, 9, (1500, 31, 2600)),     # 9 rows = 1 head x 9 positions
             (2, 4, 2, 2, (5000, 64)))          # 4 rows (vector kernel)
    for (B, Hq, Hkv, T, lens) in cases:
        lens = np.array(lens)
        max_len = int(lens.max()) + T
        cache, orc = _new((1, B, Hq, Hkv, D, max_len), dtype)
        n0 = int(lens.max())
        k, v = (rng.standard_normal((B, Hkv, n0, D), dtype=np.float32) for _ in range(2))
        cache.append(0, to_device(k, "fp32", DEV), to_device(v, "fp32", DEV))
        orc.append(0, k, v)
        cache.truncate(lens)
        orc.truncate(lens)
        q, k, v = (rng.standard_normal(s, dtype=np.float32) for s in ((B, Hq, T, D), (B, Hkv, T, D), (B, Hkv, T, D)))
        # a slightly peaked softmax: scores spread over several units of log-weight
        q *= 2.0
        cache.append(0, to_device(k, "fp32", DEV), to_device(v, "fp32", DEV))
        orc.append(0, k, v)
        got = cache.attend(0, to_device(q, "fp32", DEV)).cpu().numpy()
        want = orc.attend(0, q)
        mabs, rel = compare_out(got, want, dtype)
        log(f"  B={B} Hq={Hq} Hkv={Hkv} T={T}: rel {rel:.2e} max abs {mabs:.2e}")
        assert np.isfinite(got).all()
        if dtype == "fp32":
            assert mabs <= FP32_MAX_ABS, (Hq, Hkv, T, mabs)
        else:
            assert rel <= HALF_REL_FROB, (Hq, Hkv, T, rel)


@pytest.mark.parametrize("B, dtype", [(300, "bf16"), (300, "fp32"), (33, "bf16"), (33, "fp32")])
def test_batch_wider_than_one_launch(B, dtype):
    """B=300 rows (two launches of at most 256 rows each) and B=33 (one launch
    just past the 32 rows whose arguments carry the short row table): the
    vector (2 and 8 query rows per KV head) and matrix-core (6 rows) decode
    kernels on bf16, the vector and both row-split kernels (10 and 24 rows) on
    fp32."""
    log(f"B={B} rows {dtype}")
    rng = np.random.default_rng(300 + B)
    Hq, Hkv, D, max_len = 4, 2, 64, 80
    cache, orc = _new((1, B, Hq, Hkv, D, max_len), dtype)
    lens = rng.integers(0, 40, size=B)
    k, v = (rng.standard_normal((B, Hkv, 40, D), dtype=np.float32) for _ in range(2))
    cache.append(0, to_device(k, "fp32", DEV), to_device(v, "fp32", DEV))
    orc.append(0, k, v)
    cache.truncate(lens)
    orc.truncate(lens)
    for T in ((1, 4, 3) if dtype == "bf16" else (1, 4, 5, 12)):
        q, k, v = (rng.standard_normal(s, dtype=np.float32) for s in ((B, Hq, T, D), (B, Hkv, T, D), (B, Hkv, T, D)))
        cache.append(0, to_device(k, "fp32", DEV), to_device(v, "fp32", DEV))
        orc.append(0, k, v)
        got = cache.attend(0, to_device(q, "fp32", DEV)).cpu().numpy()
        want = orc.attend(0, input_values(q, dtype) if dtype != "fp32" else q)
        if dtype == "fp32":
            assert compare_out(got, want, dtype)[0] <= FP32_MAX_ABS, T
        else:
            assert compare_out(got, want, dtype)[1] <= HALF_REL_FROB, T
    assert cache_bits_equal(cache, orc)


def test_decode_more_kv_heads_than_a_wave_has_lanes():
    """80 and 130 KV heads: a decode work-group finds the KV head of its first
    key by a division instead of a ballot over the wave's 64 lanes (1 and 8
    query rows per KV head on the matrix-core kernel, 1 row on the vector
    kernel of an fp32 cache), on a contiguous and a paged cache (bit-identical
    to each other), and through the fused call (bit-identical to the two calls)."""
    from kv_cached_gqa_amd.kvc import KVCache, PagedKVCache
    rng = np.random.default_rng(1300)
    #        dtype   D   B  Hq   Hkv  T  context lengths before the chunk
    cases = (("bf16", 64, 3, 80, 80, 1, (700, 64, 1500)),
             ("fp16", 64, 2, 260, 130, 4, (900, 333)),
             ("fp32", 32, 2, 80, 80, 1, (500, 1200)))
    for (dtype, D, B, Hq, Hkv, T, lens) in cases:
        log(f"  {dtype} D={D} B={B} Hq={Hq} Hkv={Hkv} T={T}")
        lens = np.array(lens)
        max_len = int(lens.max()) + 2 * T
        n0 = int(lens.max())
        caches = [KVCache(1, Hkv, D, max_len, batch=B, n_q_heads=Hq, dtype=dtype, device=DEV),
                  PagedKVCache(1, Hkv, D, max_len, batch=B, n_q_heads=Hq, dtype=dtype, device=DEV, block_size=64),
                  KVCache(1, Hkv, D, max_len, batch=B, n_q_heads=Hq, dtype=dtype, device=DEV)]
        orc = OracleCache(1, B, Hq, Hkv, D, max_len, dtype)
        k, v = (rng.standard_normal((B, Hkv, n0, D), dtype=np.float32) for _ in range(2))
        for c in caches:
            c.append(0, to_device(k, "fp32", DEV), to_device(v, "fp32", DEV))
            c.truncate(lens)
        orc.append(0, k, v)
        orc.truncate(lens)
        q, k, v = (rng.standard_normal(sh, dtype=np.float32) for sh in ((B, Hq, T, D), (B, Hkv, T, D), (B, Hkv, T, D)))
        q *= 2.0
        outs = []
        for c in caches[:2]:
            c.append(0, to_device(k, "fp32", DEV), to_device(v, "fp32", DEV))
            outs.append(c.attend(0, to_device(q, "fp32", DEV)).cpu().numpy())
        # the fused call takes the chunk in the storage type
        fused = caches[2].append_attend(0, to_device(round_to_storage(k, dtype), dtype, DEV),
                                        to_device(round_to_storage(v, dtype), dtype, DEV),
                                        to_device(q, "fp32", DEV)).cpu().numpy()
        orc.append(0, k, v)
        want = orc.attend(0, q)
        mabs, rel = compare_out(outs[0], want, dtype)
        log(f"    rel {rel:.2e} max abs {mabs:.2e}")
        assert np.isfinite(outs[0]).all()
        if dtype == "fp32":
            assert mabs <= FP32_MAX_ABS, mabs
        else:
            assert rel <= HALF_REL_FROB, rel
        assert np.array_equal(outs[0], outs[1]), "paged differs from contiguous"
        assert np.array_equal(outs[0], fused), "fused call differs from the two calls"
        assert cache_bits_equal(caches[0], orc) and cache_bits_equal(caches[2], orc)


@pytest.mark.parametrize("st", ["fp16", "bf16"])
def test_q_dtype_rule(st):
    """An fp32 q for a 16-bit cache is rounded to the storage type first: the
    same output as a q passed in that type (read as stored), on the vector
    decode kernel (T=1, 4 rows), the matrix-core decode kernel (T=3, 12 rows)
    and the prefill kernel (T=16, 64 rows)."""
    log(f"q dtype rule {st}")
    rng = np.random.default_rng(400)
    cache, orc = _new((1, 2, 8, 2, 128, 64), st)
    k, v = (rng.standard_normal((2, 2, 50, 128), dtype=np.float32) for _ in range(2))
    cache.append(0, to_device(k, "fp32", DEV), to_device(v, "fp32", DEV))
    for T in (1, 3, 16):
        q = rng.standard_normal((2, 8, T, 128), dtype=np.float32)
        a = cache.attend(0, to_device(q, "fp32", DEV)).cpu().numpy()
        b = cache.attend(0, to_device(q, st, DEV)).cpu().numpy()
        assert np.array_equal(a, b), T


def test_errors_leave_gpu_state_unchanged():
    import torch
    from kv_cached_gqa_amd.kvc import ContextLimitError, KVCArgumentError, KVCStateError
    log("errors leave state unchanged")
    rng = np.random.default_rng(500)
    cache, _ = _new((2, 2, 4, 2, 32, 10), "fp16")
    k = to_device(rng.standard_normal((2, 2, 8, 32), dtype=np.float32), "fp32", DEV)
    cache.append(0, k, k)
    torch.cuda.synchronize()
    snap = gpu_bits(cache.k_storage).copy()
    fills = [cache.seq_len(layer).tolist() for layer in range(2)]
    with pytest.raises(ContextLimitError):
        k3 = to_device(np.ones((2, 2, 3, 32), np.float32), "fp32", DEV)
        cache.append(0, k3, k3)
    with pytest.raises(KVCStateError):
        cache.attend(1, to_device(np.ones((2, 4, 1, 32), np.float32), "fp32", DEV))
    with pytest.raises(KVCStateError):
        cache.truncate(1)            # layer 1 is empty, the committed length is 0
    with pytest.raises(KVCArgumentError):
        cache.append(2, k, k)
    torch.cuda.synchronize()
    assert np.array_equal(gpu_bits(cache.k_storage), snap)
    assert [cache.seq_len(layer).tolist() for layer in range(2)] == fills


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("D", [32, 64, 128])
def test_prefill_chunks_matrix_core_path(dtype, D):
    """Chunks with more than 32 query rows per KV head (the matrix-core kernel):
    group sizes 1..40 (40 > 32 splits the group), chunk lengths that leave ragged
    query blocks, rows with different offsets, and offsets that are not multiples
    of the key tile."""
    log(f"prefill matrix-core path dtype={dtype} D={D}")
    rng = np.random.default_rng(600 + D)
    for (Hq, Hkv, T) in ((2, 2, 40), (4, 1, 33), (9, 3, 100), (32, 8, 64), (16, 2, 17), (40, 1, 9), (8, 8, 300)):
        B, max_len = 3, 700
        cache, orc = _new((1, B, Hq, Hkv, D, max_len), dtype)
        pre = np.array([0, 17, 301])
        k, v = (rng.standard_normal((B, Hkv, 301, D), dtype=np.float32) for _ in range(2))
        cache.append(0, to_device(k, "fp32", DEV), to_device(v, "fp32", DEV))
        orc.append(0, k, v)
        cache.truncate(pre)
        orc.truncate(pre)
        q, k, v = (rng.standard_normal(s, dtype=np.float32) for s in ((B, Hq, T, D), (B, Hkv, T, D), (B, Hkv, T, D)))
        cache.append(0, to_device(k, "fp32", DEV), to_device(v, "fp32", DEV))
        orc.append(0, k, v)
        for q_in in ("fp32", dtype):
            got = cache.attend(0, to_device(q, q_in, DEV)).cpu().numpy()
            want = orc.attend(0, input_values(q, q_in))
            mabs, rel = compare_out(got, want, dtype)
            log(f"  Hq={Hq} Hkv={Hkv} T={T} q={q_in}: rel {rel:.2e} max abs {mabs:.2e}")
            assert np.isfinite(got).all()
            assert rel <= HALF_REL_FROB, (Hq, Hkv, T, rel)


@pytest.mark.timeout(900)
def test_chunked_prefill_bf16_full_size():
    """All 32 chunks of T=512 (offsets 0 .. 15872) at B=4, H_q=32, H_kv=8, d_h=128:
    every query row of chunks 0, 15 and 31, sampled rows of two (row, head)
    pairs per other chunk; the per-call Frobenius bound and the worst per-row
    error reported."""
    from tests.harness import worst_row_error
    log("chunked prefill bf16 full size: 32 chunks of 512")
    shape, calls = W.script_chunked_prefill()
    from kv_cached_gqa_amd.kvc import KVCache
    cache = KVCache(shape.n_layers, shape.n_kv_heads, shape.d_head, shape.max_len, batch=shape.batch,
                    n_q_heads=shape.n_q_heads, dtype=shape.dtype, device=DEV)
    orc = OracleCache(shape.n_layers, shape.batch, shape.n_q_heads, shape.n_kv_heads, shape.d_head,
                      shape.max_len, shape.dtype)
    rng = np.random.default_rng(7)
    worst, worst_row = 0.0, 0.0
    for n, call in enumerate(calls):
        cache.append(0, to_device(call.k, "fp32", DEV), to_device(call.v, "fp32", DEV))
        orc.append(0, call.k, call.v)
        got = cache.attend(0, to_device(call.q, "bf16", DEV)).cpu().numpy()
        if n in (0, 15, 31):
            rows = None
        else:
            pairs = [(int(rng.integers(shape.batch)), int(rng.integers(shape.n_q_heads))) for _ in range(2)]
            rows = sorted({(b, h, int(i)) for (b, h) in pairs for i in rng.integers(0, call.T, 24)} |
                          {(b, h, call.T - 1) for (b, h) in pairs})
        want = orc.attend(0, input_values(call.q, "bf16"), rows=rows)
        mabs, rel = compare_out(got, want, "bf16", rows)
        row_err = worst_row_error(got, want, rows)
        worst, worst_row = max(worst, rel), max(worst_row, row_err)
        if rows is None:
            log(f"  chunk {n}: all rows, rel {rel:.3e}, worst row {row_err:.3e}")
        assert rel <= HALF_REL_FROB, (n, rel)
        sel = tuple(np.array(rows).T) if rows is not None else slice(None)
        assert np.isfinite(got[sel]).all() and np.isfinite(want[sel]).all()
    log(f"  worst rel {worst:.3e}, worst per-row rel {worst_row:.3e}")


def _ulp_gap(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """Distance in representable steps between equal-signed stored values."""
    return np.abs(a_bits.astype(np.int64) - b_bits.astype(np.int64))


@pytest.mark.parametrize("st", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("D", [32, 64, 128])
def test_append_rope_and_rope_q(st, D):
    """Keys stored rotated at per-row positions (fills 2000, 1 and 777, then
    chunks of 1, 5 and 16), values unrotated, queries rotated in place; against
    the oracle's append_rope / rope_query. Both sides compute the rotation in
    float64 with the same operation order and round to float32 and then to
    the storage type, so the stored bits agree except where the two sine and
    cosine implementations round an angle differently and the float32 result
    lands on the other side of a rounding boundary: at most one storage step,
    and rare (asserted below 1 in 10^4 elements). Attention of rotated queries
    over the rotated keys is then held to the usual bound."""
    from oracle import storage_bits
    import torch
    log(f"rope append/q st={st} D={D}")
    rng = np.random.default_rng(800 + D)
    B, Hq, Hkv, max_len, base = 3, 4, 2, 2100, 10000.0
    cache, orc = _new((1, B, Hq, Hkv, D, max_len), st)
    k0, v0 = (rng.standard_normal((B, Hkv, 2000, D), dtype=np.float32) for _ in range(2))
    cache.append(0, to_device(k0, "fp32", DEV), to_device(v0, "fp32", DEV))
    orc.append(0, k0, v0)
    lens = np.array([2000, 1, 777])
    cache.truncate(lens)
    orc.truncate(lens)
    q_in = "fp32" if st == "fp32" else st
    for T in (1, 5, 16):
        k, v, q = (rng.standard_normal(s, dtype=np.float32) for s in ((B, Hkv, T, D), (B, Hkv, T, D), (B, Hq, T, D)))
        f0 = orc.seq_len(0).copy()
        cache.append(0, to_device(k, "fp32", DEV), to_device(v, "fp32", DEV), rope_base=base)
        orc.append_rope(0, k, v, base)
        qd = to_device(q, q_in, DEV)
        cache.rope_q(0, qd, base)
        qr_ref = orc.rope_query(0, input_values(q, q_in), base, q_in)
        torch.cuda.synchronize()
        kb, vb = gpu_bits(cache.k_storage), gpu_bits(cache.v_storage)
        ko, vo = storage_bits(orc.K, st), storage_bits(orc.V, st)
        for b in range(B):
            sl = (0, b, slice(None), slice(int(f0[b]), int(f0[b]) + T))
            gap = _ulp_gap(kb[sl], ko[sl])
            assert gap.max() <= 1 and (gap > 0).mean() <= 1e-4, (b, T, gap.max(), (gap > 0).mean())
            assert np.array_equal(vb[sl], vo[sl])
        qgap = _ulp_gap(gpu_bits(qd), storage_bits(qr_ref, q_in))
        assert qgap.max() <= 1 and (qgap > 0).mean() <= 1e-4
        got = cache.attend(0, qd).cpu().numpy()
        want = orc.attend(0, np.asarray(qr_ref, dtype=np.float32))
        mabs, rel = compare_out(got, want, st)
        log(f"  T={T}: key steps off {int((gap > 0).sum())}, attention rel {rel:.2e} abs {mabs:.2e}")
        if st == "fp32":
            assert mabs <= FP32_MAX_ABS
        else:
            assert rel <= HALF_REL_FROB


def test_append_rope_at_large_positions():
    """Positions 32760..32775 (angles up to 3.3e4 rad at the first frequency):
    the float64 angle keeps the rotation exact to float32 rounding."""
    from oracle import storage_bits
    import torch
    log("rope at positions near 32768")
    rng = np.random.default_rng(900)
    cache, orc = _new((1, 1, 2, 1, 128, 32776), "fp32")
    k0 = rng.standard_normal((1, 1, 32760, 128), dtype=np.float32)
    cache.append(0, to_device(k0, "fp32", DEV), to_device(k0, "fp32", DEV))
    orc.append(0, k0, k0)
    k = rng.standard_normal((1, 1, 16, 128), dtype=np.float32)
    cache.append(0, to_device(k, "fp32", DEV), to_device(k, "fp32", DEV), rope_base=500000.0)
    orc.append_rope(0, k, k, 500000.0)
    torch.cuda.synchronize()
    gap = _ulp_gap(gpu_bits(cache.k_storage)[0, 0, 0, 32760:], storage_bits(orc.K, "fp32")[0, 0, 0, 32760:])
    assert gap.max() <= 1 and (gap > 0).mean() <= 1e-3


@pytest.mark.parametrize("st", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("inp", ["fp32", "bf16"])
def test_latent_cache_append_bit_exact(st, inp):
    """The latent cache ("KV cache, incremental decode, ...", section 2.6):
    latents (r = 512) and rotary keys (d_R = 64) with edge values, chunks of
    1, 7 and 33 positions over 3 layers, a per-row rollback and fresh chunks;
    storage bits, fills and nbytes equal the oracle's. Also B = 300 (two
    launches of rows)."""
    from oracle import OracleLatentCache, storage_bits
    from kv_cached_gqa_amd.kvc import LatentCache
    import torch
    log(f"latent cache st={st} in={inp}")
    rng = np.random.default_rng(1000)
    for (L, B, r, dR, max_len) in ((3, 3, 512, 64, 64), (1, 300, 32, 8, 12)):
        lc = LatentCache(L, r, dR, max_len, batch=B, dtype=st, device=DEV)
        orc = OracleLatentCache(L, B, r, dR, max_len, st)
        steps = (1, 7, 33) if max_len == 64 else (1, 3)
        for T in steps:
            for layer in range(L):
                c = _edge_values(rng, B * T * r)[:B * T * r].reshape(B, T, r).astype(np.float32)
                kr = _edge_values(rng, B * T * dR)[:B * T * dR].reshape(B, T, dR).astype(np.float32)
                lc.append(layer, to_device(c, inp, DEV), to_device(kr, inp, DEV))
                orc.append(layer, input_values(c, inp), input_values(kr, inp))
        n = rng.integers(0, int(orc.seq_len()[0]) + 1, size=B)
        lc.truncate(n)
        orc.truncate(n)
        for layer in range(L):
            c, kr = (rng.standard_normal((B, 2, w), dtype=np.float32) for w in (r, dR))
            lc.append(layer, to_device(c, inp, DEV), to_device(kr, inp, DEV))
            orc.append(layer, input_values(c, inp), input_values(kr, inp))
        torch.cuda.synchronize()
        assert np.array_equal(gpu_bits(lc.c_storage), storage_bits(orc.C, st))
        assert np.array_equal(gpu_bits(lc.kr_storage), storage_bits(orc.KR, st))
        assert np.array_equal(lc.seq_len(), orc.seq_len())
        assert lc.nbytes() == orc.nbytes()
        lc.close()


def test_longest_row_the_layout_allows():
    """max_len * d_head just below 2^31 (16,777,215 positions at d_h=128, bf16,
    one row and one KV head: 4 GiB per tensor). The far end of the row is
    stored bit for bit by the fused call, and a T=1 query over all 16.7M keys
    returns the value vector when every position holds the same one: the
    softmax weights sum to 1 (a property that holds at any size, so no oracle
    pass over the row is needed)."""
    import torch
    from kv_cached_gqa_amd.kvc import KVCache
    ml = (1 << 24) - 1
    log(f"longest row: max_len {ml}, d_h 128, bf16")
    gen = torch.Generator(device=DEV)
    gen.manual_seed(5)
    cache = KVCache(1, 1, 128, ml, batch=1, n_q_heads=4, dtype="bf16", device=DEV)
    vrow = torch.randn((128,), generator=gen, device=DEV).to(torch.bfloat16)
    k = torch.randn((1, 1, ml - 1, 128), generator=gen, device=DEV, dtype=torch.bfloat16)
    v = vrow.view(1, 1, 1, 128).expand(1, 1, ml - 1, 128).contiguous()
    cache.append(0, k, v)
    k_prev = k[0, 0, -1].clone()
    del k, v
    kn = torch.randn((1, 1, 1, 128), generator=gen, device=DEV, dtype=torch.bfloat16)
    vn = vrow.view(1, 1, 1, 128).contiguous()
    q = torch.randn((1, 4, 1, 128), generator=gen, device=DEV, dtype=torch.bfloat16)
    out = cache.append_attend(0, kn, vn, q)
    torch.cuda.synchronize()
    assert cache.seq_len().tolist() == [ml]
    assert np.array_equal(gpu_bits(cache.k_storage[0, 0, 0, ml - 1]), gpu_bits(kn[0, 0, 0]))
    assert np.array_equal(gpu_bits(cache.k_storage[0, 0, 0, ml - 2]), gpu_bits(k_prev))
    assert np.array_equal(gpu_bits(cache.v_storage[0, 0, 0, ml - 1]), gpu_bits(vrow))
    want = vrow.float().cpu().numpy()
    got = out[0, :, 0].cpu().numpy()
    err = float(np.abs(got - want[None, :]).max() / np.abs(want).max())
    log(f"  relative error against the value vector {err:.2e}")
    assert np.isfinite(got).all() and err <= 1e-4
    cache.close()
