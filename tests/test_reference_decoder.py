"""Pins of the float64 reference decoder (oracle/reference_decoder.py) against
what "kv-cache-decoding" fixes ("Correctness tests", "Prefill and decode",
"What is cached, what is not, and what it costs", the pitfall list): cached
and uncached greedy runs agree, the work counters equal the page's figures and
formulas, chunked prefills build the same cache, a prefix is never rewritten,
and the position pitfall is caught."""
import json
import os

import numpy as np
import pytest

from kv_cached_gqa_amd.workloads import DecoderShape, decoder_params, decoder_prompt
from oracle.reference_decoder import ReferenceDecoder, greedy_cached, greedy_uncached, layer_norm

SHAPE = DecoderShape()
P, N = 48, 160


@pytest.fixture(scope="module")
def params():
    return decoder_params(0, SHAPE)


@pytest.fixture(scope="module")
def runs(params):
    prompt = decoder_prompt(1, P, SHAPE)
    cached, uncached = ReferenceDecoder(params, SHAPE), ReferenceDecoder(params, SHAPE)
    ids_c, logits_c, cache = greedy_cached(cached, prompt, N)
    ids_u, logits_u = greedy_uncached(uncached, prompt, N)
    return dict(prompt=prompt, cached=cached, uncached=uncached, ids_c=ids_c, logits_c=logits_c, cache=cache,
                ids_u=ids_u, logits_u=logits_u)


def test_layer_norm_closed_form():
    """Unit gain and zero shift give rows of mean 0 and variance v / (v + eps);
    a constant row maps to the shift."""
    rng = np.random.default_rng(4)
    x = rng.standard_normal((5, 64)) * 3 + 7
    y = layer_norm(x, np.ones(64), np.zeros(64))
    var = x.var(axis=1)
    assert np.allclose(y.mean(axis=1), 0, atol=1e-12)
    assert np.allclose(y.var(axis=1), var / (var + 1e-5), atol=1e-12)
    assert np.allclose(layer_norm(np.full((2, 8), 3.0), np.full(8, 2.0), np.arange(8.0)), np.arange(8.0))


def test_cached_equals_uncached(runs):
    """160 greedy steps after a 48-token prompt: identical ids, logits equal to
    below 1e-9, and a logit spread wide enough for the comparison to mean
    something (the page prints the spread for the same reason)."""
    assert runs["ids_c"] == runs["ids_u"]
    assert np.abs(runs["logits_c"] - runs["logits_u"]).max() < 1e-9
    assert runs["logits_c"].std() > 0.5


def test_work_counters_equal_the_page(runs, golden_dir):
    """Attention scores 47,077,120 without the cache and 362,496 with it (the
    page's figures for L = 4, h = 4, P = 48, N = 160), and positions
    sum(P + i) against P + N - 1."""
    g = json.load(open(os.path.join(golden_dir, "work_counters.json")))
    assert (g["layers"], g["heads"], g["prompt"], g["new_tokens"]) == (SHAPE.layers, SHAPE.heads, P, N)
    assert runs["uncached"].scores_computed == g["scores_uncached"] == 47077120
    assert runs["cached"].scores_computed == g["scores_cached"] == 362496
    assert runs["uncached"].positions_processed == sum(P + i for i in range(N))
    assert runs["cached"].positions_processed == P + N - 1
    # the page's formulas: L h sum (P + i)^2 and L h (P^2 + sum (P + i)), i >= 1
    assert runs["uncached"].scores_computed == SHAPE.layers * SHAPE.heads * sum((P + i) ** 2 for i in range(N))
    assert runs["cached"].scores_computed == SHAPE.layers * SHAPE.heads * (P * P + sum(P + i for i in range(1, N)))


def test_cache_fill_bytes_and_zeros(runs):
    """The cache holds P + N - 1 positions (the last chosen token is never
    fed); its filled part is 2 L h d_head (P + N - 1) values, 8,192 bytes per
    position in float64 as the page counts; unfilled slots are zero."""
    cache = runs["cache"]
    fill = P + N - 1
    assert cache.seq_len().tolist() == [fill]
    per_position = 2 * SHAPE.layers * SHAPE.heads * SHAPE.head_width
    assert cache.K[:, 0, :, :fill].size + cache.V[:, 0, :, :fill].size == per_position * fill
    assert per_position * 8 == 8192
    assert not cache.K[:, :, :, fill:].any() and not cache.V[:, :, :, fill:].any()


def test_prefill_in_chunks_builds_the_same_cache(params):
    """One pass over the prompt, 30 + 18, and 48 single-token passes: the same
    cache and the same logits for the prompt's last token."""
    prompt = decoder_prompt(1, P, SHAPE)
    built = []
    for chunks in ([P], [30, 18], [1] * P):
        model = ReferenceDecoder(params, SHAPE)
        cache = model.empty_cache()
        at = 0
        for c in chunks:
            last = model.step(prompt[at:at + c], cache)[-1]
            at += c
        built.append((cache.K.copy(), cache.V.copy(), last))
    for K, V, last in built[1:]:
        assert np.abs(K - built[0][0]).max() <= 1e-6       # float32 storage of float64 projections
        assert np.abs(V - built[0][1]).max() <= 1e-6
        assert np.abs(last - built[0][2]).max() < 1e-9


def test_prefix_keys_and_values_never_change(params):
    """Appending 20 more tokens leaves the keys and values of the first 48
    unchanged (bit for bit here; the page asks for 1e-12)."""
    prompt = decoder_prompt(1, P, SHAPE)
    model = ReferenceDecoder(params, SHAPE)
    cache = model.empty_cache()
    model.step(prompt, cache)
    K0, V0 = cache.K[:, :, :, :P].copy(), cache.V[:, :, :, :P].copy()
    model.step(decoder_prompt(2, 20, SHAPE), cache)
    assert np.array_equal(cache.K[:, :, :, :P], K0) and np.array_equal(cache.V[:, :, :, :P], V0)


def test_position_restarting_at_zero_is_caught(params):
    """The planted pitfall: decode steps take position row 0. The prefill is
    still right, every later step's logits are wrong, and the equality pin
    fails."""
    prompt = decoder_prompt(1, P, SHAPE)
    _, bad, _ = greedy_cached(ReferenceDecoder(params, SHAPE, restart_positions=True), prompt, 8)
    _, good = greedy_uncached(ReferenceDecoder(params, SHAPE), prompt, 8)
    assert np.abs(bad[0] - good[0]).max() < 1e-9
    assert np.abs(bad[1:] - good[1:]).max() > 1e-3
