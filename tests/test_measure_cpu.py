"""The traffic calibration (kv_cached_gqa_amd/measure.py) on the CPU, from
synthetic rocprofv3 counter files: each counter is scaled by what it reads
for a copy of known size, dispatches are averaged per kernel, and a stored
figure is used only while the decode sources are the ones it was taken on."""
import csv
import os

import numpy as np

from kv_cached_gqa_amd import measure


def _write_run(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "p_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (kernel, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": kernel, "Counter_Name": counter, "Counter_Value": value})


def test_calibrated_traffic_and_digest_gate(tmp_path):
    copy = 1 << 20
    copy_k = "void at::native::elementwise_kernel<MulFunctor<float>>"
    # the copy reads 1 MiB but FETCH_SIZE shows half of it (512 KiB); WRITE_SIZE is exact (1024 KiB)
    _write_run(tmp_path / "f", "FETCH_SIZE", [(copy_k, 512.0), (copy_k, 512.0),
                                             ("decode_mfma<128>", 1000.0), ("decode_mfma<128>", 1200.0),
                                             ("decode_combine<128>", 10.0)])
    _write_run(tmp_path / "w", "WRITE_SIZE", [(copy_k, 1024.0), ("decode_mfma<128>", 50.0),
                                             ("decode_combine<128>", 4.0), ("decode_combine<128>", 6.0)])
    out = tmp_path / "traffic.md"
    total = measure.summarize(str(tmp_path / "f"), str(tmp_path / "w"), copy, str(out), "cmd f", "cmd w")
    f_fac, w_fac = copy / 512.0, copy / 1024.0            # 2048 and 1024 bytes per counted KiB
    want = (1100.0 * f_fac + 50.0 * w_fac) + (10.0 * f_fac + 5.0 * w_fac)
    assert total == round(want)
    text = out.read_text()
    assert "cmd f" in text and "cmd w" in text
    assert measure.stored_traffic(str(out)) == total           # sources unchanged: the figure is used
    stale = text.replace(measure.source_digest(), "0" * 64)
    out.write_text(stale)
    assert measure.stored_traffic(str(out)) is None             # another digest: ignored
    assert measure.stored_traffic(str(tmp_path / "missing.md")) is None


def test_trace_tables_group_calls(tmp_path):
    """A decode kernel and the merge pass right after it are one call; an
    append right before a decode kernel joins that call; grids are reported in
    work-groups."""
    f = tmp_path / "kt_kernel_trace.csv"
    cols = ["Kind", "Queue_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp", "Workgroup_Size_X",
            "Workgroup_Size_Y", "Workgroup_Size_Z", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"]
    dec = "void kvc::(anonymous namespace)::decode_mfma<128, 2, false>(kvc::DecodeArgs)"
    comb = "void kvc::(anonymous namespace)::decode_combine<128>(kvc::DecodeArgs)"
    app = "void kvc::(anonymous namespace)::append_kernel<2, 2>(kvc::AppendArgs)"
    rows = [(dec, 0, 60, 64, 49152, 1, 1), (comb, 61, 65, 256, 2048, 2, 32),      # attention: span 65
            (dec, 100, 170, 64, 49152, 1, 1), (comb, 171, 175, 256, 2048, 2, 32),  # attention: span 75
            (app, 200, 204, 256, 4096, 2, 1), (dec, 205, 265, 64, 49152, 1, 1), (comb, 266, 270, 256, 2048, 2, 32)]
    with open(f, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=cols)
        w.writeheader()
        for name, st, en, wg, gx, gy, gz in rows:
            w.writerow({"Kind": "KERNEL_DISPATCH", "Queue_Id": 1, "Kernel_Name": name, "Start_Timestamp": st,
                        "End_Timestamp": en, "Workgroup_Size_X": wg, "Workgroup_Size_Y": 1, "Workgroup_Size_Z": 1,
                        "Grid_Size_X": gx, "Grid_Size_Y": gy, "Grid_Size_Z": gz})
    text = measure.trace_tables(str(f))
    lines = text.splitlines()
    attn = [ln for ln in lines if ln.startswith("| decode_mfma<128, 2, false> (768x1) + decode_combine<128> (8x2x32)")]
    assert len(attn) == 1 and "| 2 | 65 + 4 | 70 | 70 | 65 | 75 |" in attn[0]
    step = [ln for ln in lines if ln.startswith("| append_kernel<2, 2> (16x2) + decode_mfma")]
    assert len(step) == 1 and "| 1 | 4 + 60 + 4 | 70 |" in step[0]
    assert any(ln.startswith("| decode_mfma<128, 2, false> | 768x1 x 64 | 3 |") for ln in lines)
    assert any(ln.startswith("| decode_combine<128> | 8x2x32 x 256 | 3 |") for ln in lines)


def test_probe_summary_on_synthetic_records():
    """The timestamp probe's summary: phases from the records, per-XCD rates,
    and the share of the end-time spread the XCD accounts for (here the whole
    of it: every work-group of XCD x ends x microseconds after the others')."""
    from kv_cached_gqa_amd import probe
    rng = np.random.default_rng(0)
    bursts = []
    for _ in range(3):
        wg, merge = [], []
        for k in range(64):
            x = k % 8
            start = 1000 + int(rng.integers(0, 20))
            end = 1000 + 5000 + 100 * x
            ids = (x << 32) | ((k // 8) << 8)
            wg.append([start, start + 50, start + 110, end, ids, 900])
        for j in range(16):
            merge.append([6800 + j, 6900 + j, 7000 + j, 7020 + j])
        bursts.append({"wg": wg, "merge": merge})
    text = probe.summarize(bursts)
    lines = text.splitlines()
    first = [ln for ln in lines if ln.startswith("| 0 | 64 |")]
    assert len(first) == 1
    cells = [c.strip() for c in first[0].strip("|").split("|")]
    assert cells[3] == "0.50" and cells[4] == "1.10"          # located, issued (us after start)
    assert float(cells[7]) > 0                                 # the merge starts after the last work-group
    assert any(ln.startswith("| 7 |") for ln in lines)
    assert "the XCD accounts for 100% of the variance" in text
