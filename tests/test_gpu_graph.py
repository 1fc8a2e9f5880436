"""Attention calls captured in a HIP graph (torch.cuda.graph): kvc_attend and
kvc_attend_static enqueue kernels only (the split-K workspace is allocated at
create, the static scratch is looked up without allocating), so a call can be
captured and replayed. A replay repeats the call as captured, with the
lengths of that moment: a graph serves repeated calls over the same cache
state (re-scoring, a fixed-size verification step), not a growing cache.
Every replay is checked against the eager result, with eager work and
synchronisations between replays; the graph holds no memset node."""
import numpy as np
import pytest

from tests.harness import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_cached_gqa_amd import kvc  # noqa: F401  (fails loudly if libkvc.so is missing)
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("kind", ["contiguous", "paged", "static"])
@pytest.mark.parametrize("shape", [(32, 32, 8, 128, 4096, 1, "bf16"), (1, 9, 3, 64, 700, 1, "fp16"),
                                   (2, 8, 2, 128, 1500, 64, "bf16")])
def test_attention_call_replays_from_a_graph(kind, shape):
    import torch
    from kv_cached_gqa_amd.kvc import KVCache, PagedKVCache
    B, Hq, Hkv, D, max_len, T, dtype = shape
    log(f"graph capture {kind} B={B} Hq={Hq} Hkv={Hkv} D={D} T={T} {dtype}")
    dev = torch.device("cuda")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    gen = torch.Generator(device=dev)
    gen.manual_seed(2024)
    mk = dict(batch=B, n_q_heads=Hq, dtype=dtype, device=dev)
    cache = PagedKVCache(1, Hkv, D, max_len, block_size=128, **mk) if kind == "paged" else \
        KVCache(1, Hkv, D, max_len, **mk)
    k = torch.randn((B, Hkv, max_len - 1, D), generator=gen, device=dev, dtype=tdt)
    cache.append(0, k, k)
    lengths = np.random.default_rng(7).integers(T, max_len - 1, size=B)
    cache.truncate(lengths)
    kv = torch.randn((B, Hkv, T, D), generator=gen, device=dev, dtype=tdt)
    cache.append(0, kv, kv)
    q = torch.randn((B, Hq, T, D), generator=gen, device=dev, dtype=tdt)
    out = torch.empty((B, Hq, T, D), device=dev, dtype=torch.float32)
    call = (lambda: cache.attend_static(0, q, out)) if kind == "static" else (lambda: cache.attend(0, q, out=out))
    call()
    torch.cuda.synchronize()
    eager = out.clone()

    side = torch.cuda.Stream()          # default priority
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        call()
    other = torch.empty_like(out)
    for rep in range(3):
        out.fill_(float("nan"))
        cache.attend(0, q, out=other)   # eager work on the same cache between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), eager.view(torch.int32)), (kind, shape, rep)
        assert torch.equal(other.view(torch.int32), eager.view(torch.int32)), (kind, shape, rep)
    del graph
    cache.close()
