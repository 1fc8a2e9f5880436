"""Drive one call script through the HIP path (libkvc via its binding) and the
CPU oracle side by side, comparing every result.

Bars: cache contents, fill counts and nbytes bit-exact; attention outputs
max-abs <= 1e-5 for an fp32 cache and ||dO||_F / ||O_ref||_F <= 2e-3 per call
for fp16/bf16 caches (over the rows compared).
"""
from __future__ import annotations

import sys
import time
from dataclasses import dataclass, field

import numpy as np

from oracle import OracleCache, storage_bits

FP32_MAX_ABS = 1e-5
HALF_REL_FROB = 2e-3


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


@dataclass
class Report:
    calls: int = 0
    attends: int = 0
    worst_abs: float = 0.0
    worst_rel: float = 0.0
    worst_tag: str = ""
    failures: list = field(default_factory=list)
    row_errors: list = None      # (tag, layer, worst per-row relative error) per 16-bit call, when asked for

    def ok(self) -> bool:
        return not self.failures


def to_device(x: np.ndarray, dtype: str, device):
    import torch
    from kv_cached_gqa_amd.kvc import torch_dtype
    # convert on the host, so the device gets exactly the bits input_values() describes
    t = torch.from_numpy(np.ascontiguousarray(x)).to(torch_dtype(dtype)).contiguous()
    return t.to(device=device)


def input_values(x: np.ndarray, dtype: str) -> np.ndarray:
    """The float32 values an input of `dtype` carries (the harness converts
    fp32 draws to 16-bit inputs with torch; both sides then see those values)."""
    if dtype == "fp32":
        return x
    import torch
    from kv_cached_gqa_amd.kvc import torch_dtype
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch_dtype(dtype)).float().numpy()


def compare_out(got: np.ndarray, want: np.ndarray, dtype: str, rows=None):
    """Returns (max_abs, rel_frob) over all rows or the sampled (b, h, i)."""
    if rows is not None:
        idx = tuple(np.array(rows).T)
        got = got[idx]
        want = want[idx]
    diff = got.astype(np.float64) - want
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    denom = float(np.linalg.norm(want))
    rel = float(np.linalg.norm(diff) / denom) if denom > 0 else max_abs
    return max_abs, rel


def worst_row_error(got: np.ndarray, want: np.ndarray, rows=None) -> float:
    """The largest per-row relative error ||o_gpu - o_ref|| / ||o_ref|| over the
    call's query rows (b, h, i), each row a d_h vector: the diagnostic reported
    beside the per-call Frobenius figure for 16-bit caches."""
    if rows is not None:
        idx = tuple(np.array(rows).T)
        got, want = got[idx], want[idx]
    g = got.reshape(-1, got.shape[-1]).astype(np.float64)
    w = want.reshape(-1, want.shape[-1])
    num = np.linalg.norm(g - w, axis=1)
    den = np.linalg.norm(w, axis=1)
    return float(np.max(num / np.where(den > 0, den, 1.0))) if num.size else 0.0


def sample_rows(rng, B, Hq, T, n, groups=None, G=1):
    """About n query rows (b, h, i), always including (0, 0, T-1) and (B-1,
    Hq-1, 0). With groups = k, the rows are drawn inside k random (row, KV
    head) units, query heads h of group g = h // G, so the oracle reads the
    keys of only a few units per call."""
    if groups is None:
        rows = {(int(rng.integers(B)), int(rng.integers(Hq)), int(rng.integers(T))) for _ in range(n)}
    else:
        units = [(int(rng.integers(B)), int(rng.integers(Hq // G))) for _ in range(groups)]
        rows = set()
        for _ in range(n):
            b, g = units[int(rng.integers(len(units)))]
            rows.add((b, g * G + int(rng.integers(G)), int(rng.integers(T))))
    rows |= {(0, 0, T - 1), (B - 1, Hq - 1, 0)}
    return sorted(rows)


def run_script(shape, calls, *, device="cuda", q_dtype="fp32", kv_dtype="fp32", sample=None,
               compare_cache=True, check_every_call=True, verbose=True, cache=None, oracle=None,
               out_log=None, full_rows_at=None, row_errors=False, sample_groups=None):
    """Run `calls` on both sides. sample=n compares n random rows per attend
    (all rows when None). Returns (report, cache, oracle)."""
    from kv_cached_gqa_amd.kvc import KVCache
    import torch

    if cache is None:
        cache = KVCache(shape.n_layers, shape.n_kv_heads, shape.d_head, shape.max_len, batch=shape.batch,
                        n_q_heads=shape.n_q_heads, dtype=shape.dtype, device=device)
    if oracle is None:
        oracle = OracleCache(shape.n_layers, shape.batch, shape.n_q_heads, shape.n_kv_heads, shape.d_head,
                             shape.max_len, shape.dtype)
    rep = Report()
    if row_errors:
        rep.row_errors = []
    rng = np.random.default_rng(12345)
    n_pass = 0
    t0 = time.time()
    for call in calls:
        rep.calls += 1
        if call.op in ("append", "pass"):
            kd, vd = to_device(call.k, kv_dtype, device), to_device(call.v, kv_dtype, device)
            cache.append(call.layer, kd, vd)
            oracle.append(call.layer, input_values(call.k, kv_dtype), input_values(call.v, kv_dtype))
            del kd, vd
        if call.op == "pass":
            qd = to_device(call.q, q_dtype, device)
            got = cache.attend(call.layer, qd).cpu().numpy()
            rows = None
            if sample is not None and not (full_rows_at is not None and full_rows_at(n_pass, call)):
                rows = sample_rows(rng, shape.batch, shape.n_q_heads, call.T, sample, sample_groups,
                                   shape.n_q_heads // shape.n_kv_heads)
            n_pass += 1
            want = oracle.attend(call.layer, input_values(call.q, q_dtype), rows=rows)
            mabs, rel = compare_out(got, want, shape.dtype, rows)
            rep.attends += 1
            # written so that a NaN anywhere (either side, or the error itself) fails
            bad = not (mabs <= FP32_MAX_ABS) if shape.dtype == "fp32" else not (rel <= HALF_REL_FROB)
            sel = tuple(np.array(rows).T) if rows is not None else slice(None)
            if not np.isfinite(got[sel]).all() or not np.isfinite(want[sel]).all():
                bad = True
            if rep.row_errors is not None and shape.dtype != "fp32":
                rep.row_errors.append((call.tag, call.layer, worst_row_error(got, want, rows)))
            if mabs > rep.worst_abs:
                rep.worst_abs = mabs
            if rel > rep.worst_rel:
                rep.worst_rel, rep.worst_tag = rel, f"{call.tag} layer {call.layer}"
            if bad:
                rep.failures.append((call.tag, call.layer, mabs, rel))
            if out_log is not None:
                out_log.append((call.tag, call.layer, call.T, mabs, rel))
        if call.op == "truncate":
            cache.truncate(call.n)
            oracle.truncate(call.n)
        if check_every_call:
            for layer in range(shape.n_layers):
                if not np.array_equal(cache.seq_len(layer), oracle.seq_len(layer)):
                    rep.failures.append((call.tag, layer, "seq_len", None))
            if not np.array_equal(cache.seq_len(), oracle.seq_len()):
                rep.failures.append((call.tag, -1, "committed seq_len", None))
        if verbose and rep.calls % 200 == 0:
            log(f"  ... {rep.calls} calls, {time.time() - t0:.1f}s, worst abs {rep.worst_abs:.2e} "
                f"rel {rep.worst_rel:.2e}")
    torch.cuda.synchronize()
    if compare_cache:
        if not cache_bits_equal(cache, oracle):
            rep.failures.append(("cache", -1, "bits differ", None))
    if cache.nbytes() != oracle.nbytes():
        rep.failures.append(("nbytes", -1, cache.nbytes(), oracle.nbytes()))
    return rep, cache, oracle


def gpu_bits(t) -> np.ndarray:
    import torch
    if t.dtype == torch.float32:
        return t.cpu().view(torch.int32).numpy().view(np.uint32)
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def cache_bits_equal(cache, oracle, layer_slice=slice(None)) -> bool:
    for which, st in (("K", cache.k_storage), ("V", cache.v_storage)):
        g = gpu_bits(st[layer_slice])
        o = storage_bits((oracle.K if which == "K" else oracle.V)[layer_slice], oracle.dtype)
        if not np.array_equal(g, o):
            return False
    return True
