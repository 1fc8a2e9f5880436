"""Per-work-group timestamps of the batched-decode attention call.

    python -m kv_cached_gqa_amd.probe [--workdir DIR] [--bursts N] [--out FILE]

builds a copy of this package in DIR (a new temporary directory by default)
with KVC_DECODE_TIMESTAMPS=1: there the matrix-core decode kernel records, per
work-group, when it starts, when its first segment is located, when its first
tile is issued and when it ends (the GPU's 100 MHz clock), with its XCC and
hardware ids and its slice's keys, and the merge pass records, per block,
when it starts, when its contributors are known, when their records are merged
and when it ends. A child process runs the batched-decode workload (B=32,
H_q=32, H_kv=8, d_h=128, bf16, lengths U{1024..4095} seed 0, 4 rotating cache
instances) on that copy: a warm-up of at least 0.3 s, then N bursts of 20
attention calls, reading the records of each burst's last call. The summary
(markdown) covers the start-up phases, the spread of the work-groups' ends,
the XCDs' streaming rates and the merge pass, and how much of the spread the
XCD and the CU account for. The library itself is never built with the
timestamps.
"""
from __future__ import annotations

import argparse
import json
import os
import shutil
import subprocess
import sys
import tempfile

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
TICKS_PER_US = 100.0
BYTES_PER_KEY = 512          # K and V of one key at d_h = 128, bf16

_CHILD = r'''
import json, os, sys, time
work = sys.argv[1]; n_bursts = int(sys.argv[2])
sys.path.insert(0, work)
import ctypes
import numpy as np, torch
import kv_cached_gqa_amd.kvc as K
assert K.LIB_PATH.startswith(work), K.LIB_PATH
from kv_cached_gqa_amd.workloads import batched_lengths
lib = K._lib
lib.kvc_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int]
NW, NM = 8192, 16384
B, HQ, HKV, D, ML = 32, 32, 8, 128, 4096
lengths = batched_lengths(np.random.default_rng(0), B, 1024, ML - 1)
dev = torch.device("cuda:0"); gen = torch.Generator(device=dev); gen.manual_seed(5)
caches = []
for c in range(4):
    cache = K.KVCache(1, HKV, D, ML, batch=B, n_q_heads=HQ, dtype="bf16", device=dev)
    k = torch.randn((B, HKV, ML - 1, D), generator=gen, device=dev, dtype=torch.bfloat16)
    cache.append(0, k, k); del k; cache.truncate(lengths); caches.append(cache)
q = torch.randn((B, HQ, 1, D), generator=gen, device=dev, dtype=torch.bfloat16)
kv = torch.randn((B, HKV, 1, D), generator=gen, device=dev, dtype=torch.bfloat16)
out = torch.empty((B, HQ, 1, D), device=dev, dtype=torch.float32)
for c in caches: c.append(0, kv, kv)
t = time.perf_counter(); i = 0
while time.perf_counter() - t < 0.3:
    caches[i % 4].attend(0, q, out=out); i += 1
bursts = []
for rep in range(n_bursts):
    assert lib.kvc_probe_clear() == 0
    for i in range(20): caches[i % 4].attend(0, q, out=out)
    torch.cuda.synchronize()
    wg = np.zeros(NW * 6, np.uint64); mg = np.zeros(NM * 4, np.uint64)
    assert lib.kvc_probe_read(wg.ctypes.data, NW, mg.ctypes.data, NM) == 0
    wg = wg.reshape(NW, 6); mg = mg.reshape(NM, 4)
    bursts.append({"wg": wg[wg[:, 3] > 0].astype(np.int64).tolist(), "merge": mg[mg[:, 3] > 0].astype(np.int64).tolist()})
    print(f"burst {rep} recorded", file=sys.stderr, flush=True)
for c in caches: c.close()
print(json.dumps(bursts))
'''


def _cu_ids(ids: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """(XCD, CU) of each record from the XCC id (high word) and the hardware
    id register (low word: CU bits 8-11, shader array bit 12, engine 13-15)."""
    xcc = (ids >> 32) & 0xF
    hw = ids & 0xFFFFFFFF
    cu = xcc * 1000 + ((hw >> 13) & 7) * 100 + ((hw >> 12) & 1) * 20 + ((hw >> 8) & 0xF)
    return xcc, cu


def _var_explained(r: np.ndarray, groups: np.ndarray) -> float:
    tot = ((r - r.mean()) ** 2).sum()
    if tot == 0:
        return 0.0
    within = sum(((r[groups == g] - r[groups == g].mean()) ** 2).sum() for g in np.unique(groups))
    return 1.0 - within / tot


def summarize(bursts: list[dict]) -> str:
    """Markdown summary of the recorded bursts (each: 'wg' rows of [start,
    located, issued, end, ids, keys], 'merge' rows of [start, known, merged,
    end], GPU clock ticks)."""
    rows = ["| Burst | Work-groups | Start spread (us) | First segment located, median (us after start) | "
            "First tile issued, median (us after start) | Median end (us) | Last end (us) | Merge: first block "
            "after the last end (us) | Merge block, median (us) | Merge end (us) |",
            "|---|---|---|---|---|---|---|---|---|---|"]
    xcd_rate = [[] for _ in range(8)]
    xcd_dev = [[] for _ in range(8)]
    ends, xccs, cus = [], None, None
    for i, b in enumerate(bursts):
        a = np.array(b["wg"], dtype=np.int64).reshape(-1, 6)
        m = np.array(b["merge"], dtype=np.int64).reshape(-1, 4)
        t0 = a[:, 0].min()
        st = (a[:, 0] - t0) / TICKS_PER_US
        en = (a[:, 3] - t0) / TICKS_PER_US
        loc = (a[:, 1] - a[:, 0]) / TICKS_PER_US
        iss = (a[:, 2] - a[:, 0]) / TICKS_PER_US
        xcc, cu = _cu_ids(a[:, 4])
        if len(m):
            ms = (m[:, 0] - t0) / TICKS_PER_US
            mt = (m[:, 3] - m[:, 0]) / TICKS_PER_US
            merge = f"{ms.min() - en.max():.2f} | {np.median(mt):.2f} | {(m[:, 3].max() - t0) / TICKS_PER_US:.1f}"
        else:
            merge = "— | — | —"
        rows.append(f"| {i} | {len(a)} | {st.max():.2f} | {np.median(loc):.2f} | {np.median(iss):.2f} | "
                    f"{np.median(en):.1f} | {en.max():.1f} | {merge} |")
        for x in range(8):
            sel = xcc == x
            if sel.any():
                xcd_rate[x].append(a[sel, 5].sum() * BYTES_PER_KEY / (en[sel].max() - st[sel].min()) / 1e6)
                xcd_dev[x].append(np.median(en[sel]) - np.median(en))
        if xccs is None or len(a) == len(xccs):
            ends.append(en)
            xccs, cus = xcc, cu
    out = ["Per burst (the records of each burst's last call; times from the call's first work-group start):", "",
           *rows, "",
           "Per XCD over the bursts (the rate counts the keys of each slice's padded range, virtual keys included):",
           "", "| XCD | Streaming rate, min-max (TB/s) | Median end minus the call's median, min-max (us) |",
           "|---|---|---|"]
    for x in range(8):
        if xcd_rate[x]:
            out.append(f"| {x} | {min(xcd_rate[x]):.3f}-{max(xcd_rate[x]):.3f} | "
                       f"{min(xcd_dev[x]):+.1f} to {max(xcd_dev[x]):+.1f} |")
    if len(ends) >= 2:
        e = np.array(ends)
        per_burst_xcd = np.mean([_var_explained(e[i], xccs) for i in range(len(e))])
        res = e.copy()
        for i in range(len(e)):
            for x in np.unique(xccs):
                sel = xccs == x
                res[i, sel] -= e[i, sel].mean()
        r = res.mean(0)
        pairs = [np.corrcoef(res[i], res[j])[0, 1] for i in range(len(e)) for j in range(i + 1, len(e))
                 if res[i].std() > 0 and res[j].std() > 0]
        corr = f"correlates {np.mean(pairs):.2f} from burst to burst" if pairs else "is zero"
        out += ["", f"Spread of the work-groups' ends: the XCD accounts for {100 * per_burst_xcd:.0f}% of the "
                    f"variance within a call; after each call's XCD means are removed, what remains "
                    f"(std {r.std():.2f} us over the bursts' mean) {corr}, and the CU accounts for "
                    f"{100 * _var_explained(r, cus):.0f}% of it."]
    return "\n".join(out)


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--workdir", default=None, help="where the instrumented copy is built (default: a new temp dir)")
    ap.add_argument("--bursts", type=int, default=8)
    ap.add_argument("--out", default=None, help="also write the summary here")
    a = ap.parse_args()
    work = os.path.abspath(a.workdir or tempfile.mkdtemp(prefix="kvc_probe_"))
    dst = os.path.join(work, "kv_cached_gqa_amd")
    if os.path.exists(dst):
        shutil.rmtree(dst)
    shutil.copytree(PKG, dst, ignore=shutil.ignore_patterns("_build", "libkvc.so*", "__pycache__"))
    if not os.path.exists(os.path.join(work, "include")):
        shutil.copytree(os.path.join(ROOT, "include"), os.path.join(work, "include"))
    env = dict(os.environ, KVC_BUILD_DEFINES="KVC_DECODE_TIMESTAMPS=1")
    print(f"building the instrumented copy in {work}", file=sys.stderr, flush=True)
    subprocess.run([sys.executable, "-m", "kv_cached_gqa_amd.build"], cwd=work, env=env, check=True)
    r = subprocess.run([sys.executable, "-c", _CHILD, work, str(a.bursts)], stdout=subprocess.PIPE, check=True,
                       text=True)
    text = summarize(json.loads(r.stdout.strip().splitlines()[-1]))
    print(text)
    if a.out:
        with open(a.out, "w") as fh:
            fh.write(text + "\n")


if __name__ == "__main__":
    main()
