"""Pins of the float64 tiny decoder (oracle/tiny_decoder.py) against what
"kv-cache-decoding" ("Correctness tests", "Prefill and decode", "What is
cached") fixes: cached and uncached greedy runs agree, the work counters equal
the page's figures, chunked prefills build the same cache, a prefix is never
rewritten, and the classic position bug is caught."""
import json
import os

import numpy as np
import pytest

from kv_cached_gqa_amd.workloads import TinyDecoderSpec, tiny_decoder_prompt, tiny_decoder_weights
from oracle.tiny_decoder import OracleTinyDecoder, generate_no_cache, generate_with_cache

SPEC = TinyDecoderSpec()
P, N = 48, 160


@pytest.fixture(scope="module")
def weights():
    return tiny_decoder_weights(0, SPEC)


@pytest.fixture(scope="module")
def runs(weights):
    prompt = tiny_decoder_prompt(1, P, SPEC)
    mc, mn = OracleTinyDecoder(weights, SPEC), OracleTinyDecoder(weights, SPEC)
    ids_c, lc, cache = generate_with_cache(mc, prompt, N)
    ids_n, ln = generate_no_cache(mn, prompt, N)
    return dict(prompt=prompt, mc=mc, mn=mn, ids_c=ids_c, lc=lc, cache=cache, ids_n=ids_n, ln=ln)


def test_cached_equals_uncached(runs):
    """160 greedy steps after a 48-token prompt: identical ids, logits equal to
    below 1e-9, and a logit spread that makes the comparison meaningful."""
    assert runs["ids_c"] == runs["ids_n"]
    assert np.abs(runs["lc"] - runs["ln"]).max() < 1e-9
    assert runs["lc"].std() > 0.5


def test_work_counters_equal_the_page(runs, golden_dir):
    g = json.load(open(os.path.join(golden_dir, "work_counters.json")))
    assert (g["layers"], g["heads"], g["prompt"], g["new_tokens"]) == (SPEC.n_layers, SPEC.n_heads, P, N)
    assert runs["mn"].scores == g["scores_uncached"] == 47077120
    assert runs["mc"].scores == g["scores_cached"] == 362496
    assert runs["mn"].positions == sum(P + i for i in range(N))
    assert runs["mc"].positions == P + N - 1


def test_cache_fill_bytes_and_zeros(runs):
    """The cache holds P + N - 1 positions (the last sampled token is not fed);
    its filled part is 2 L h d_head (P + N - 1) values; unfilled slots are zero."""
    cache = runs["cache"]
    fill = P + N - 1
    assert cache.seq_len().tolist() == [fill]
    filled = cache.K[:, 0, :, :fill].size + cache.V[:, 0, :, :fill].size
    assert filled == 2 * SPEC.n_layers * SPEC.n_heads * SPEC.d_head * fill
    assert not cache.K[:, :, :, fill:].any() and not cache.V[:, :, :, fill:].any()


def test_prefill_in_chunks_builds_the_same_cache(weights):
    """One pass over the prompt, 30 + 18, and 48 single-token passes: the same
    cache and the same logits for the prompt's last token."""
    prompt = tiny_decoder_prompt(1, P, SPEC)
    results = []
    for chunks in ([P], [30, 18], [1] * P):
        m = OracleTinyDecoder(weights, SPEC)
        cache = m.new_cache()
        at = 0
        for c in chunks:
            last = m.forward(prompt[at:at + c], cache)[-1]
            at += c
        results.append((cache.K.copy(), cache.V.copy(), last))
    for K, V, last in results[1:]:
        assert np.abs(K - results[0][0]).max() <= 1e-6       # fp32 storage of float64 projections
        assert np.abs(V - results[0][1]).max() <= 1e-6
        assert np.abs(last - results[0][2]).max() < 1e-9


def test_prefix_keys_and_values_never_change(weights):
    """Appending 20 more tokens leaves the keys and values of the first 48 as
    they were (bit for bit)."""
    prompt = tiny_decoder_prompt(1, P, SPEC)
    m = OracleTinyDecoder(weights, SPEC)
    cache = m.new_cache()
    m.forward(prompt, cache)
    K0, V0 = cache.K[:, :, :, :P].copy(), cache.V[:, :, :, :P].copy()
    m.forward(tiny_decoder_prompt(2, 20, SPEC), cache)
    assert np.array_equal(cache.K[:, :, :, :P], K0) and np.array_equal(cache.V[:, :, :, :P], V0)


def test_position_restarting_at_zero_is_caught(weights):
    """A planted mistake: decode steps take position row 0. The equality check
    fails (the page's pitfall "Position restarts at 0")."""
    prompt = tiny_decoder_prompt(1, P, SPEC)
    bad = OracleTinyDecoder(weights, SPEC, position_bug=True)
    _, lc, _ = generate_with_cache(bad, prompt, 8)
    _, ln = generate_no_cache(OracleTinyDecoder(weights, SPEC), prompt, 8)
    assert np.abs(lc[1:] - ln[1:]).max() > 1e-3
    assert np.abs(lc[0] - ln[0]).max() < 1e-9      # the prefill itself is right
