"""Turn two rocprofv3 counter passes over `bench.py --profile-only --calibrate-copy` into
the per-launch HBM traffic record that bench.py reports as `roofline.traffic`.

    python bench_counters.py FETCH_DIR WRITE_DIR "<profile command>" PROFILE_LOG
    python bench_counters.py --stats DIR OUT.md TITLE "<profile command>" DESCRIPTION
    python bench_counters.py --mfma DIR OUT.md "<profile command>"

FETCH_DIR / WRITE_DIR hold run_counter_collection.csv from
    rocprofv3 --pmc FETCH_SIZE -d FETCH_DIR -o run --output-format csv -- python3 bench.py --profile-only --steps 2 --warmup 0 --calibrate-copy
and the same with WRITE_SIZE.  Both counters are per dispatch, in KiB.  The scales come
from the known-size kernels at the end of the run: w12_stream_read over 1 GiB - 256 B
(read with the nontemporal 16-byte buffer loads the GEMM issues for W12 tiles) for
FETCH_SIZE, and the 1 GiB fill before it (writes 1 GiB) for WRITE_SIZE; the 1 GiB
device-to-device copy after it is reported as a cross-check of the read scale.  A
`w12_gemm` launch is one GEMM kernel (K-split launches complete inside it).  The FP8
launches of the same shapes (`w12_gemm_f8`, after the profiled W12 / BF16 steps) get their
own rows.  Writes profiles/w12_gemm_traffic.json and profiles/w12_gemm_mlp_block_traffic.md.

With --stats it summarises a `rocprofv3 --kernel-trace --stats` run instead: the stats
table and the average duration of every (kernel, grid) launch shape, as markdown; with
--mfma, a counter pass of the MFMA counters (flops counted, busy fraction) per launch shape.
"""
from __future__ import annotations

import csv
import json
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

PROFILED_STEPS = 2   # --steps of the profile command
ENCODE_KERNELS = ("k_fill_zero", "k_hist", "k_codebook", "k_count_tiles", "k_scan", "k_pack",
                  "k_bf16_tile")


def read(d: str, counter: str):
    rows = []
    with open(os.path.join(d, "run_counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], int(r["Grid_Size"]),
                         float(r["Counter_Value"])))
    rows.sort()
    return rows


def is_gemm(name: str) -> bool:
    return "w12::k_gemm" in name


def is_f8(name: str) -> bool:
    """An FP8 instantiation: weight source 4, the third template argument of k_gemm_cs."""
    if "w12::k_gemm_cs<" not in name:
        return False
    args = name.split("k_gemm_cs<", 1)[1].split(">", 1)[0].split(",")
    return len(args) == 4 and args[2].strip() == "4"


def launches(rows, f8: bool = False):
    """The GEMM-family dispatches, one per w12_gemm / w12_gemm_bf16 launch (f8: one per
    w12_gemm_f8 launch)."""
    out = []
    for _, name, grid, val in rows:
        if not is_gemm(name) or is_f8(name) != f8:
            continue
        short = name.split("(")[0].replace("void ", "")
        out.append({"kernels": [short], "grid": grid, "value": val})
    return out


def main():
    fetch_dir, write_dir, command, log_path = sys.argv[1:5]
    w12_bytes = {}
    with open(log_path) as f:
        for line in f:
            if line.startswith("bench: W12 bytes"):
                t = line.split()
                w12_bytes = {t[3]: int(t[4]), t[5]: int(t[6])}
    shapes = {"gate_up": (bench.N_GU, bench.K_GU), "down": (bench.N_DN, bench.K_DN)}
    fr, wr = read(fetch_dir, "FETCH_SIZE"), read(write_dir, "WRITE_SIZE")
    # calibration kernels after the last GEMM: the streaming read of 1 GiB - 256 B (the
    # GEMM's load type) scales FETCH_SIZE, the 1 GiB fill scales WRITE_SIZE, the 1 GiB
    # copy cross-checks the read scale
    tail_f = [r for r in fr if r[0] > max(x[0] for x in fr if is_gemm(x[1]))]
    tail_w = [r for r in wr if r[0] > max(x[0] for x in wr if is_gemm(x[1]))]
    stream_f = [r for r in tail_f if "k_stream_read" in r[1]][-1]
    copy_f = max((r for r in tail_f if "w12::" not in r[1]), key=lambda r: r[3])
    fill_w = max((r for r in tail_w if "w12::" not in r[1]), key=lambda r: r[3])
    fetch_scale = (bench.COPY_BYTES - 256) / (stream_f[3] * 1024.0)
    write_scale = bench.COPY_BYTES / (fill_w[3] * 1024.0)
    copy_scale = bench.COPY_BYTES / (copy_f[3] * 1024.0)
    # the profiled steps are the last PROFILED_STEPS (W12 step, BF16 step) pairs of 20
    # launches; the time-based warm-up before them varies in length between the passes
    lf, lw = launches(fr), launches(wr)
    assert len(lf) % 20 == 0 and len(lw) % 20 == 0 and min(len(lf), len(lw)) >= 20 * PROFILED_STEPS
    lf, lw = lf[-20 * PROFILED_STEPS:], lw[-20 * PROFILED_STEPS:]
    assert [a["grid"] for a in lf] == [b["grid"] for b in lw]
    keys = [f"M{m}_{name}" for m in bench.MS for name in ("gate_up", "down")]
    rec = {"source_sha256": bench.kernel_source_hash(), "profile": command,
           "fetch_scale": fetch_scale, "write_scale": write_scale,
           "calibration": {"stream_read_fetch_kib": stream_f[3], "stream_read_bytes": bench.COPY_BYTES - 256,
                           "copy_kernel": copy_f[1][:80], "copy_fetch_kib": copy_f[3],
                           "copy_fetch_scale": copy_scale,
                           "fill_kernel": fill_w[1][:80], "fill_write_kib": fill_w[3],
                           "bytes": bench.COPY_BYTES},
           "launches": {}, "bf16_launches": {}, "f8_launches": {}}
    steps = len(lf) // 20
    for i, key in enumerate(keys):
        for kind, off in (("launches", 0), ("bf16_launches", 10)):
            idx = [20 * s + off + i for s in range(steps)]
            f_kib = sum(lf[j]["value"] for j in idx) / steps
            w_kib = sum(lw[j]["value"] for j in idx) / steps
            m = int(key.split("_")[0][1:])
            n, k = shapes[key.split("_", 1)[1]]
            wb = w12_bytes[key.split("_", 1)[1]] if kind == "launches" else 2 * n * k
            rec[kind][key] = {"kernels": lf[idx[0]]["kernels"], "grid": lf[idx[0]]["grid"],
                              "fetch_kib": round(f_kib, 3), "write_kib": round(w_kib, 3),
                              "hbm_bytes": int(round(f_kib * 1024 * fetch_scale
                                                     + w_kib * 1024 * write_scale)),
                              "alg_bytes": wb + 2 * m * k + 2 * m * n}
    # the FP8 GEMMs of the same shapes, 10 launches per profiled step after the W12 / BF16 steps
    ff, fw = launches(fr, f8=True), launches(wr, f8=True)
    assert len(ff) == len(fw) == 10 * PROFILED_STEPS, (len(ff), len(fw))
    for i, key in enumerate(keys):
        idx = [10 * s + i for s in range(PROFILED_STEPS)]
        f_kib = sum(ff[j]["value"] for j in idx) / PROFILED_STEPS
        w_kib = sum(fw[j]["value"] for j in idx) / PROFILED_STEPS
        m = int(key.split("_")[0][1:])
        n, k = shapes[key.split("_", 1)[1]]
        rec["f8_launches"][key] = {"kernels": ff[idx[0]]["kernels"], "grid": ff[idx[0]]["grid"],
                                   "fetch_kib": round(f_kib, 3), "write_kib": round(w_kib, 3),
                                   "hbm_bytes": int(round(f_kib * 1024 * fetch_scale
                                                          + w_kib * 1024 * write_scale)),
                                   "alg_bytes": bench.f8_bytes(n, k, m)}
    with open(os.path.join(ROOT, "profiles", "w12_gemm_traffic.json"), "w") as f:
        json.dump(rec, f, indent=1)
    lines = ["# HBM traffic per launch: MLP block GEMMs (rocprofv3 counters)", "",
             "Commands (from the repository root, on one MI355X):", "",
             f"    {command.replace('PMC', 'FETCH_SIZE').replace('DIR', fetch_dir)}",
             f"    {command.replace('PMC', 'WRITE_SIZE').replace('DIR', write_dir)}",
             f"    python bench_counters.py {fetch_dir} {write_dir} \"<command>\" <profile log>",
             "",
             f"Scales: FETCH_SIZE x {fetch_scale:.4f} (`w12::k_stream_read` over 1 GiB - 256 B with the "
             f"GEMM's nontemporal 16-byte buffer loads reads {stream_f[3]:.0f} KiB; a 1 GiB device copy, "
             f"`{copy_f[1][:40]}`, reads {copy_f[3]:.0f} KiB, scale {copy_scale:.4f}), "
             f"WRITE_SIZE x {write_scale:.4f} (a 1 GiB fill, `{fill_w[1][:40]}`, writes "
             f"{fill_w[3]:.0f} KiB).  GEMM sources sha256 `{rec['source_sha256'][:16]}...`.", "",
             "| launch | kernels | W12: HBM bytes | algorithmic | ratio | BF16 kernel: HBM bytes | algorithmic | ratio |",
             "|---|---|---|---|---|---|---|---|"]
    for key in keys:
        a, b = rec["launches"][key], rec["bf16_launches"][key]
        lines.append(f"| {key} | `{' + '.join(a['kernels'])}` | {a['hbm_bytes']:,} | {a['alg_bytes']:,} | "
                     f"{a['hbm_bytes'] / a['alg_bytes']:.3f} | {b['hbm_bytes']:,} | {b['alg_bytes']:,} | "
                     f"{b['hbm_bytes'] / b['alg_bytes']:.3f} |")
    lines += ["", "The same shapes in FP8 checkpoint form (`w12_gemm_f8`: E4M3 codes + FP32 block "
              "scales; algorithmic bytes = codes + scales + x + y):", "",
              "| launch | kernels | FP8: HBM bytes | algorithmic | ratio |", "|---|---|---|---|---|"]
    for key in keys:
        c = rec["f8_launches"][key]
        lines.append(f"| {key} | `{' + '.join(c['kernels'])}` | {c['hbm_bytes']:,} | {c['alg_bytes']:,} | "
                     f"{c['hbm_bytes'] / c['alg_bytes']:.3f} |")
    with open(os.path.join(ROOT, "profiles", "w12_gemm_mlp_block_traffic.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps({k: v["hbm_bytes"] for k, v in rec["launches"].items()}))


def stats_main():
    """--stats DIR OUT TITLE COMMAND DESCRIPTION: kernel-duration summary of a
    `rocprofv3 --kernel-trace --stats -d DIR -o run --output-format csv` run as markdown."""
    d, out, title, command, desc = sys.argv[2:7]
    with open(os.path.join(d, "run_kernel_stats.csv")) as f:
        stats = list(csv.DictReader(f))
    lines = [f"# {title}", "", "Command (from the repository root, on one MI355X):", "",
             f"    {command}", "", desc, "", "rocprofv3 `--stats` summary:", "",
             "| kernel | calls | avg us | min us | max us | share |", "|---|---|---|---|---|---|"]
    for r in stats:
        name = r["Name"].split("(")[0].replace("void ", "")
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.1f} % |")
    shapes = {}
    with open(os.path.join(d, "run_kernel_trace.csv")) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"].split("(")[0].replace("void ", "")
            if "w12::" not in name:
                continue
            wg = int(r["Workgroup_Size_X"])
            key = (name, int(r["Grid_Size_X"]) // wg, int(r["Grid_Size_Y"]), wg)
            shapes.setdefault(key, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    lines += ["", "Per launch shape (same run, from the kernel trace; workgroups x splits):", "",
              "| kernel | grid | calls | avg us | median us | min us |", "|---|---|---|---|---|---|"]
    for (name, gx, gy, wg), ts in sorted(shapes.items(), key=lambda kv: -sum(kv[1])):
        med = sorted(ts)[len(ts) // 2]
        lines.append(f"| `{name}` | {gx} x {gy} wg of {wg} | {len(ts)} | "
                     f"{sum(ts) / len(ts) / 1e3:.2f} | {med / 1e3:.2f} | {min(ts) / 1e3:.2f} |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def mfma_main():
    """--mfma DIR OUT COMMAND: MFMA use per launch shape from one counter pass
    (SQ_INSTS_VALU_MFMA_MOPS_BF16, SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE) over the W12
    and BF16 GEMM kernels, as markdown."""
    d, out, command = sys.argv[2:5]
    per = {}
    with open(os.path.join(d, "run_counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            e = per.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"].split("(")[0].replace("void ", ""),
                                                      "grid": int(r["Grid_Size"]), "wg": int(r["Workgroup_Size"]),
                                                      "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
            e[r["Counter_Name"]] = float(r["Counter_Value"])
    shapes = {}
    for e in per.values():
        if "k_gemm" not in e["name"]:
            continue
        shapes.setdefault((e["name"], e["grid"] // e["wg"], e["wg"]), []).append(e)
    lines = ["# MFMA use per launch: MLP block GEMMs (rocprofv3 counters)", "",
             "Command (from the repository root, on one MI355X):", "", f"    {command}", "",
             "`SQ_INSTS_VALU_MFMA_MOPS_BF16` counts BF16 MFMA work in units of 512 flops (it "
             "equals 2 x 16 x padded rows x K for the 16-column launches: the MFMA tiles include "
             "the padding columns and waves).  `GRBM_GUI_ACTIVE` is summed over the 8 XCDs, so "
             "the busy fraction is `SQ_VALU_MFMA_BUSY_CYCLES` / (`GRBM_GUI_ACTIVE` / 8 x 1024 "
             "SIMDs).  TFLOP/s = the counted flops / the dispatch duration under counter "
             "collection, against the 2.5 PFLOP/s dense BF16 peak.  Every launch is bound by HBM "
             "(the roofline), not by the matrix cores.", "",
             "| kernel | workgroups | dispatches | MFMA GFLOP | TFLOP/s | % of 2.5 PFLOP/s | MFMA busy % |",
             "|---|---|---|---|---|---|---|"]
    for (name, nwg, wg), es in sorted(shapes.items(), key=lambda kv: (kv[0][0], kv[0][1])):
        fl = sum(e.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) for e in es) / len(es) * 512
        ns = sum(e["ns"] for e in es) / len(es)
        busy = sum(e.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / max(e.get("GRBM_GUI_ACTIVE", 1.0) / 8 * 1024, 1.0)
                   for e in es) / len(es)
        tf = fl / ns / 1e3
        lines.append(f"| `{name}` | {nwg} x {wg} | {len(es)} | {fl / 1e9:.2f} | {tf:.1f} | "
                     f"{100 * tf / 2500:.1f} | {100 * busy:.1f} |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "--stats":
        stats_main()
    elif len(sys.argv) > 1 and sys.argv[1] == "--mfma":
        mfma_main()
    else:
        main()
