"""kvc_attend_static, the allocation-free attention call, against kvc_attend
through the C ABI: the same results on two calls in a row (the second over
shorter rows and fewer query positions, so a smaller split-K job reuses the
static scratch the first one left behind), on the matrix-core decode kernel
(16-bit cache, split units), the fp32 vector kernel with its merge pass, and a
prefill-sized chunk; and a shape whose records exceed the static array is
refused before anything runs."""
import ctypes

import numpy as np
import pytest

from tests.harness import log

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


@pytest.mark.parametrize("dtype, D", [("bf16", 128), ("fp32", 128), ("bf16", 64), ("bf16", 32)])
def test_attend_static_equals_attend_on_two_calls(dtype, D):
    import torch
    from kv_cached_gqa_amd.kvc import KVCache
    log(f"attend_static vs attend dtype={dtype} D={D}")
    gen = torch.Generator(device=DEV)
    gen.manual_seed(31)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    # d_head 64 and 32 run more decode work-groups per CU: a finer split
    B, Hq, Hkv, max_len = 8, 32, 8, 3000
    cache = KVCache(1, Hkv, D, max_len, batch=B, n_q_heads=Hq, dtype=dtype, device=DEV)
    k = torch.randn((B, Hkv, 2900, D), generator=gen, device=DEV, dtype=tdt)
    v = torch.randn((B, Hkv, 2900, D), generator=gen, device=DEV, dtype=tdt)
    cache.append(0, k, v)
    # first call: long ragged rows, a 4-token chunk (16 rows per KV head)
    cache.truncate(np.array([2896, 1000, 2500, 17, 2896, 640, 1999, 2222]))
    calls = [(4, None), (1, np.array([300, 5, 290, 1, 64, 299, 100, 250]))]   # second: shorter rows, T=1
    for n, (T, cut) in enumerate(calls):
        if cut is not None:
            cache.truncate(cut)
            cache.append(0, k[:, :, :T].contiguous(), v[:, :, :T].contiguous())
        q = torch.randn((B, Hq, T, D), generator=gen, device=DEV, dtype=tdt)
        ref = cache.attend(0, q)
        got = torch.full_like(ref, float("nan"))
        cache.attend_static(0, q, out=got)
        torch.cuda.synchronize()
        assert torch.isfinite(got).all(), n
        # the same kernels with the same work split: bit for bit
        assert torch.equal(got.view(torch.int32), ref.view(torch.int32)), n
        log(f"  call {n}: T={T}, bit-identical to kvc_attend")
    # a prefill-sized chunk (16-bit storage: the matrix-core prefill, no
    # scratch; fp32: several decode slabs through the scratch)
    cache.truncate(np.full(B, 2))
    cache.append(0, k[:, :, :40].contiguous(), v[:, :, :40].contiguous())
    q = torch.randn((B, Hq, 40, D), generator=gen, device=DEV, dtype=tdt)
    ref = cache.attend(0, q)
    got = cache.attend_static(0, q, out=torch.empty_like(ref))
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int32), ref.view(torch.int32))
    cache.close()


def test_attend_static_refuses_a_job_larger_than_its_scratch():
    """256 rows x 64 KV heads of 32-row records at d_head 128 need ~272 MB of
    scratch: KVC_ERR_SCRATCH, nothing changes, kvc_attend still works."""
    import torch
    from kv_cached_gqa_amd import kvc
    B, Hq, Hkv, D = 256, 64, 64, 128
    cache = kvc.KVCache(1, Hkv, D, 4, batch=B, n_q_heads=Hq, dtype="bf16", device=DEV)
    kv = torch.randn((B, Hkv, 1, D), device=DEV, dtype=torch.bfloat16)
    cache.append(0, kv, kv)
    q = torch.randn((B, Hq, 1, D), device=DEV, dtype=torch.bfloat16)
    out = torch.empty((B, Hq, 1, D), device=DEV, dtype=torch.float32)
    rc = kvc.lib().kvc_attend_static(cache.handle, 0, ctypes.c_void_p(q.data_ptr()), kvc.BF16, 1,
                                     ctypes.c_void_p(out.data_ptr()), None)
    assert rc == kvc.ERR_SCRATCH
    assert cache.seq_len().tolist() == [1] * B
    ref = cache.attend(0, q)
    torch.cuda.synchronize()
    assert torch.isfinite(ref).all()
    cache.close()
