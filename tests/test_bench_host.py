"""Host logic of bench.py (no GPU): the kernel-trace summary counts only the
timed steps' launches, so profiled per-launch times compare with the bench's
own timed launches."""
import csv
import os

import bench


def _write_trace(path, steps, warmup, attn_us):
    os.makedirs(os.path.join(path, "host", "1"))
    rows, t = [], 0
    for step in range(warmup + steps):
        for name, dur in [("void pab::quant_mxfp4_kernel<bf16>(pab::QuantArgs)", 40_000),
                          ("void pab::quant_mxfp4_kernel<bf16>(pab::QuantArgs)", 42_000),
                          ("void pab::attn_fwd_kernel<128, true, 0, true, false>(pab::AttnArgs)",
                           attn_us[step] * 1000)]:
            rows.append({"Kernel_Name": name, "Start_Timestamp": t, "End_Timestamp": t + dur})
            t += dur + 100
    rows.append({"Kernel_Name": "copy", "Start_Timestamp": t, "End_Timestamp": t + 700})
    with open(os.path.join(path, "host", "1", "run_kernel_trace.csv"), "w") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        w.writerows(rows)


def test_trace_summary_leaves_out_warmup(tmp_path):
    # warm-up launches are slow (3000 us); the timed ones take 2600..2604 us
    attn = [3000, 3000, 2600, 2601, 2602, 2603, 2604]
    _write_trace(str(tmp_path), steps=5, warmup=2, attn_us=attn)
    table = bench.trace_summary(str(tmp_path), steps=5, warmup=2)
    lines = {l.split("|")[1].strip(): [c.strip() for c in l.split("|")[2:-1]]
             for l in table.splitlines()[2:]}
    att = lines["`pab::attn_fwd_kernel<128, true, 0, true, false>`"]
    assert att[0].startswith("5 (1 per step)")
    assert float(att[1]) == 2602.0 and float(att[2]) == 2602.0            # median, mean
    assert float(att[3]) == 2600.0 and float(att[4]) == 2604.0            # min, max
    q = lines["`pab::quant_mxfp4_kernel<bf16>`"]
    assert q[0].startswith("10 (2 per step)") and float(q[1]) == 41.0
    assert lines["`copy`"][0].startswith("1 (not per step")
