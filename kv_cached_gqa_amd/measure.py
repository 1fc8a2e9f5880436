"""Measurement helpers: HBM traffic from rocprofv3 counters, calibrated, and
per-kernel durations from a rocprofv3 kernel trace.

The TCC counters FETCH_SIZE and WRITE_SIZE (KiB per dispatch) do not read the
bytes a kernel moves one to one on this GPU. Each is therefore scaled by what
it reads for a plain elementwise copy of known size (N bytes read, N written)
in the same run: factor = N / counter(copy). The calibrated traffic of a
kernel is counter(kernel) * factor.

    python -m kv_cached_gqa_amd.measure summarize --fetch DIR --write DIR \\
        --copy-bytes N --out profiles/<name>.md --cmd-fetch "..." --cmd-write "..."

reads the *_counter_collection.csv files of two rocprofv3 --pmc runs (one
counter each) and writes a short markdown summary whose last lines hold the
calibrated bytes per attention call and a digest of the decode sources, which
bench.py reads back (and ignores once the sources have changed).

    python -m kv_cached_gqa_amd.measure trace --trace FILE [--tags a,b]

prints, from a rocprofv3 --kernel-trace CSV, the calls of the library grouped
by the kernels and grids they hold (an append, a decode kernel and the merge
pass that follow one another on the same queue count as one call), with each
kernel's average duration and the call's span from its first kernel's start to
its last kernel's end; then the durations of every dispatch per (kernel, grid).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import re
import statistics
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
# Sources whose change invalidates a stored decode traffic figure.
DECODE_SOURCES = tuple(sorted(os.path.relpath(f, PKG) for f in glob.glob(os.path.join(PKG, "csrc", "kvc_decode*")))) + (
    "csrc/kvc_kernels.h", "csrc/kvc_device.h", "csrc/kvc_mfma.h", "csrc/kvc_api.cpp")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_attend_c3_bf16_traffic.md")
COPY_KERNEL_TAG = "MulFunctor"          # the calibration copy: torch.mul(src, 1, out=dst)


def source_digest(files=DECODE_SOURCES) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(PKG, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def read_counters(run_dir: str) -> dict[str, dict[str, list[float]]]:
    """{kernel name: {counter: [value per dispatch]}} from one rocprofv3 --pmc run."""
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {run_dir}")
    per: dict[str, dict[str, dict[str, float]]] = defaultdict(lambda: defaultdict(dict))
    for f in files:
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                did = r.get("Dispatch_Id") or r.get("Correlation_Id") or str(len(per))
                per[r["Kernel_Name"]][r["Counter_Name"]][did] = (
                    per[r["Kernel_Name"]][r["Counter_Name"]].get(did, 0.0) + float(r["Counter_Value"]))
    return {k: {c: list(d.values()) for c, d in v.items()} for k, v in per.items()}


def _mean_for(counters, tag: str, counter: str) -> tuple[float, int]:
    vals = [x for name, cs in counters.items() if tag in name for x in cs.get(counter, [])]
    if not vals:
        raise KeyError(f"no dispatch of a kernel matching {tag!r} with {counter}")
    return sum(vals) / len(vals), len(vals)


def summarize(fetch_dir: str, write_dir: str, copy_bytes: int, out: str, cmd_fetch: str, cmd_write: str,
              kernels=("decode_mfma", "decode_combine"),
              title: str = "HBM traffic of one decode attention call, batched decode (B=32, H_q=32, H_kv=8, "
                           "d_h=128, bf16, lengths U{1024..4095} seed 0, T=1)",
              workload: str = "c3_attend", unit: str = "attend") -> int:
    fc, wc = read_counters(fetch_dir), read_counters(write_dir)
    cf, ncf = _mean_for(fc, COPY_KERNEL_TAG, "FETCH_SIZE")
    cw, ncw = _mean_for(wc, COPY_KERNEL_TAG, "WRITE_SIZE")
    f_fac, w_fac = copy_bytes / cf, copy_bytes / cw
    rows, total = [], 0.0
    for k in kernels:
        f, nf = _mean_for(fc, k, "FETCH_SIZE")
        w, nw = _mean_for(wc, k, "WRITE_SIZE")
        rb, wb = f * f_fac, w * w_fac
        total += rb + wb
        rows.append(f"| {k} | {nf} | {f:,.1f} | {rb / 1e6:,.2f} | {w:,.1f} | {wb / 1e6:,.2f} |")
    text = [
        f"# {title}",
        "",
        f"Two rocprofv3 counter runs of `bench.py --pmc-workload {workload}` (a calibration copy, then 40 calls "
        "of the workload), one counter each:",
        "",
        f"    {cmd_fetch}",
        f"    {cmd_write}",
        "",
        f"Calibration copy (torch.mul(src, 1, out=dst), {copy_bytes:,} bytes read and written): "
        f"FETCH_SIZE {cf:,.1f} KiB per dispatch over {ncf} dispatches -> factor {f_fac:.2f} B per counter unit; "
        f"WRITE_SIZE {cw:,.1f} KiB over {ncw} -> factor {w_fac:.2f}.",
        "",
        "| Kernel | Dispatches | FETCH_SIZE (KiB) | Read (MB, calibrated) | WRITE_SIZE (KiB) | Written (MB, calibrated) |",
        "|---|---|---|---|---|---|",
        *rows,
        "",
        f"traffic_bytes_per_{unit}: {int(round(total))}",
        f"decode_sources_sha256: {source_digest()}",
        "",
    ]
    os.makedirs(os.path.dirname(os.path.abspath(out)), exist_ok=True)
    with open(out, "w") as fh:
        fh.write("\n".join(text))
    return int(round(total))


def stored_traffic(path: str = TRAFFIC_FILE) -> int | None:
    """Calibrated bytes per attention call from the stored summary, or None when
    there is none or the decode sources changed since it was taken."""
    try:
        with open(path) as fh:
            lines = fh.read().splitlines()
    except OSError:
        return None
    vals = {}
    for ln in lines:
        if ":" in ln and not ln.startswith(("|", "#", " ")):
            k, _, v = ln.partition(":")
            vals[k.strip()] = v.strip()
    if vals.get("decode_sources_sha256") != source_digest():
        return None
    try:
        return int(vals["traffic_bytes_per_attend"])
    except (KeyError, ValueError):
        return None


# kernels of this library, and which of them start a call (a merge pass only
# closes one)
LIB_KERNELS = ("append_kernel", "rope_kernel", "table_set_kernel", "gather_kernel", "decode_attn",
               "decode_rows", "decode_mfma", "prefill_attn", "decode_combine")
_NAME_RE = re.compile(r"::([A-Za-z_]\w*(?:<[^()]*>)?)\(")


def short_name(name: str) -> str:
    """'void ns::(anonymous namespace)::decode_mfma<128, 2, false>(Args)' -> 'decode_mfma<128, 2, false>'."""
    found = _NAME_RE.findall(name)
    return found[-1] if found else name.split("(")[0][:60]


def read_trace(path: str) -> list[dict]:
    """Dispatches of a rocprofv3 kernel trace in start order: name, grid in
    work-groups (x, y, z), work-group size, start and end (ns), queue."""
    out = []
    with open(path, newline="") as fh:
        for r in csv.DictReader(fh):
            wx, wy = int(r["Workgroup_Size_X"]), int(r["Workgroup_Size_Y"])
            out.append({
                "name": short_name(r["Kernel_Name"]),
                "grid": (int(r["Grid_Size_X"]) // max(wx, 1), int(r["Grid_Size_Y"]) // max(wy, 1),
                         int(r["Grid_Size_Z"]) // max(int(r["Workgroup_Size_Z"]), 1)),
                "wg": wx * wy * int(r["Workgroup_Size_Z"]),
                "start": int(r["Start_Timestamp"]), "end": int(r["End_Timestamp"]),
                "queue": r.get("Queue_Id", ""),
            })
    out.sort(key=lambda d: d["start"])
    return out


def _grid(g: tuple) -> str:
    """(768, 1, 1) -> '768x1', (8, 2, 32) -> '8x2x32'."""
    return "x".join(str(v) for v in (g if g[2] > 1 else g[:2]))


def _stats_ns(v: list[float]) -> str:
    return (f"{len(v)} | {statistics.fmean(v):,.0f} | {statistics.median(v):,.0f} | {min(v):,.0f} | "
            f"{max(v):,.0f}")


def trace_tables(path: str, tags=LIB_KERNELS) -> str:
    """Markdown: each call pattern of the library (see the module docstring)
    with the duration of each of its kernels and its span, then every
    dispatch of the tagged kernels per (kernel, grid)."""
    ds = read_trace(path)
    lib = [d for d in ds if any(d["name"].startswith(t) for t in LIB_KERNELS)]
    decode = ("decode_attn", "decode_rows", "decode_mfma")
    calls: dict[tuple, list[list[dict]]] = defaultdict(list)
    i = 0
    while i < len(lib):
        call = [lib[i]]
        j = i + 1
        if lib[i]["name"].startswith("append_kernel") and j < len(lib) and \
                lib[j]["name"].startswith(decode) and lib[j]["queue"] == lib[i]["queue"]:
            call.append(lib[j])
            j += 1
        if call[-1]["name"].startswith(decode) and j < len(lib) and \
                lib[j]["name"].startswith("decode_combine") and lib[j]["queue"] == call[-1]["queue"]:
            call.append(lib[j])
            j += 1
        calls[tuple((d["name"], d["grid"]) for d in call)].append(call)
        i = j
    lines = ["| Call: kernels (grid in work-groups) | Calls | Kernel averages (ns) | Span average (ns) | "
             "Span median (ns) | Span min (ns) | Span max (ns) |",
             "|---|---|---|---|---|---|---|"]
    for key, cs in sorted(calls.items(), key=lambda kv: -len(kv[1])):
        name = " + ".join(f"{n} ({_grid(g)})" for n, g in key)
        avgs = " + ".join(f"{statistics.fmean(c[k]['end'] - c[k]['start'] for c in cs):,.0f}" for k in range(len(key)))
        spans = [c[-1]["end"] - c[0]["start"] for c in cs]
        lines.append(f"| {name} | {len(cs)} | {avgs} | {statistics.fmean(spans):,.0f} | "
                     f"{statistics.median(spans):,.0f} | {min(spans):,.0f} | {max(spans):,.0f} |")
    per: dict[tuple, list[float]] = defaultdict(list)
    for d in ds:
        if any(d["name"].startswith(t) for t in tags):
            per[(d["name"], d["grid"], d["wg"])].append(d["end"] - d["start"])
    lines += ["", "| Kernel | Grid (work-groups) x work-group | Dispatches | Average (ns) | Median (ns) | Min (ns) | Max (ns) |",
              "|---|---|---|---|---|---|---|"]
    for (n, g, wg), v in sorted(per.items(), key=lambda kv: -len(kv[1])):
        lines.append(f"| {n} | {_grid(g)} x {wg} | {_stats_ns(v)} |")
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("summarize")
    s.add_argument("--fetch", required=True)
    s.add_argument("--write", required=True)
    s.add_argument("--copy-bytes", type=int, required=True)
    s.add_argument("--out", default=TRAFFIC_FILE)
    s.add_argument("--cmd-fetch", default="")
    s.add_argument("--cmd-write", default="")
    s.add_argument("--kernels", default="decode_mfma,decode_combine", help="kernel name tags, comma separated")
    s.add_argument("--title", default=None)
    s.add_argument("--workload", default="c3_attend")
    s.add_argument("--unit", default="attend", help="what one counted call is (attend, step)")
    t = sub.add_parser("trace")
    t.add_argument("--trace", required=True, help="a rocprofv3 *_kernel_trace.csv")
    t.add_argument("--tags", default=",".join(LIB_KERNELS), help="kernel name prefixes to tabulate")
    a = ap.parse_args()
    if a.cmd == "trace":
        print(trace_tables(a.trace, tuple(a.tags.split(","))))
        return
    kw = {"title": a.title} if a.title else {}
    total = summarize(a.fetch, a.write, a.copy_bytes, a.out, a.cmd_fetch, a.cmd_write,
                      kernels=tuple(a.kernels.split(",")), workload=a.workload, unit=a.unit, **kw)
    print(f"wrote {a.out}: {total:,} bytes per attention call")


if __name__ == "__main__":
    main()
