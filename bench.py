"""Benchmark of the W12 decode/verification GEMM on one MI355X.

Workload (default): the MLP block of a dense ~22B decoder -- fused gate+up
W [34816, 5120] and down W [5120, 17408], BF16 ~N(0, 0.02^2) packed to W12, x rows
BF16 ~N(0, 1) -- at M = 1, 4, 8, 16 and 32 rows.  One step = the ten W12 GEMMs
(gate+up and down at every M).  `value` is the step's algorithmic bytes (W12 format
bytes + x + y of every GEMM) divided by the step time, in GB/s, with all inputs
resident in HBM.  The same step on plain BF16 weights with the same kernel family
gives the speedup.  Weight copies are rotated so that no GEMM finds its weights in the
256 MB Infinity Cache.

Protocol:
  * before any timing, every GEMM of the step runs once on the W12 kernel and both BF16
    kernels, and the CPU oracle, timed on a bounded sample (the `cpu_baseline` leg: the
    first rows of both matrices at every M), checks those outputs on the same rows;
    a mismatch stops the run;
  * every timed loop is preceded by at least WARM_S seconds of the same or mixed work
    (the GPU clock ramps up from idle), and the warm-up steps the caller asks for;
  * the headline times exactly --steps W12 steps between two synchronisations (HIP
    events on the launching stream, one per step for the CI);
  * the speedups come from three interleaved rounds (W12, row-major BF16, tiled BF16 steps
    in rotated order), medians per kind;
  * per launch: three rounds of 100 launches per (M, matrix, kernel), median round; their
    sum over the step is reported beside the step time;
  * the streaming-read ceiling for the same byte counts (w12_stream_read, the GEMM's own
    nontemporal loads, best of several grid sizes, rotated over 2 GiB).

More workloads are timed in the same run and reported beside the main line: the same
matrices at M = 64 and 128 (batched regime); the same shapes in FP8 checkpoint form (E4M3
codes with FP32 128 x 128 block scales, the GEMMs of FP8 targets) at M = 1..128, their
sampled outputs checked by the oracle first; the LM-head greedy verification ([151936,
5120], M = 16, and 24 requests in one pass) and a whole weight-streaming decode step (64
layers of q, k, v, o, gate, up, down + LM head, M = 24, RMS-chained).

`roofline.traffic` is the HBM traffic of the dominant launch measured by rocprofv3
counters (FETCH_SIZE and WRITE_SIZE passes over `--profile-only --calibrate-copy`,
scaled by what the counters read for the streaming-read kernel over 1 GiB and a 1 GiB
fill); it is read from profiles/w12_gemm_traffic.json and reported only while the kernel
sources still hash to the value recorded there (null otherwise).

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--no-extras]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W12 GEMM achieved HBM GB/s (% of peak) and speedup vs BF16, M=1..32"
PEAK_GBPS = 8000.0          # MI355X HBM3E peak
MS = (1, 4, 8, 16, 32)
BATCHED_MS = (64, 128)      # batched regime (several requests' rows at once), reported beside
N_GU, K_GU = 34816, 5120
N_DN, K_DN = 5120, 17408
WARM_S = 1.0                # seconds of work before the headline loop (clock ramp from idle)
SAMPLE_ROWS = 256           # rows of each matrix the oracle checks (cpu_baseline leg)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def w12_bytes(t) -> int:
    return t.nbytes()


def gemm_bytes(t, m: int) -> int:
    return w12_bytes(t) + 2 * m * t.k + 2 * m * t.n


def bf16_bytes(n: int, k: int, m: int) -> int:
    return 2 * n * k + 2 * m * k + 2 * m * n


def cpu_baseline(host_w, xs_host, gpu_out, seconds_target: float = 12.0):
    """The CPU oracle on a bounded sample of the workload: its W12 GEMM (bit-exact decode of
    the first SAMPLE_ROWS rows of both matrices, then the FP64 product) at every M, timed
    for about seconds_target; the same results check the GPU outputs on those rows (W12
    and both BF16 kernels), which the run captured before any timing.  Returns the baseline
    record and the parity record."""
    import numpy as np
    from oracle import w12_oracle as o
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    rows = SAMPLE_ROWS
    blobs = {name: o.encode(w[:rows]) for name, w in host_w.items()}
    parity = {}
    done_bytes, t_total, reps = 0, 0.0, 0
    while (t_total < seconds_target and reps < 50) or reps == 0:
        for m in MS:
            for name, blob in blobs.items():
                x = xs_host[(m, name)]
                t0 = time.perf_counter()
                z, s = o.gemm_w12(x, blob)
                t_total += time.perf_counter() - t0
                done_bytes += o.blob_bytes(blob) + 2 * m * blob.k + 2 * m * rows
                if reps == 0:
                    parity[f"M{m}_{name}"] = {kind: bool(o.gemm_accept(y[:, :rows], z, s).all())
                                              for kind, y in gpu_out[(m, name)].items()}
        reps += 1
    base = {"value": done_bytes / t_total / 1e9, "unit": "GB/s", "cores": int(blas_threads),
            "kind": "oracle",
            "sample": f"oracle W12 GEMM (decode + FP64 product) on the first {rows} rows of the "
                      f"gate+up [{rows}x{K_GU}] and down [{rows}x{K_DN}] matrices, M in {list(MS)}, "
                      f"{reps} passes, {t_total:.1f} s; BLAS threads {blas_threads}"}
    return base, parity


def f8_parity(x_host, q_rows, s_rows, y_rows):
    """Oracle check of sampled FP8 GEMM outputs (cpu_baseline leg): the first 128-row
    scale block of a matrix (q_rows, s_rows) against the GPU's outputs on those rows."""
    from oracle import w12_oracle as o
    z, sa = o.gemm_f8_reference(x_host, q_rows, s_rows)
    return bool(o.gemm_accept(y_rows, z, sa).all())


def f8_bytes(n: int, k: int, m: int) -> int:
    """Algorithmic bytes of one FP8 GEMM: the codes, the block scales, x and y."""
    return n * k + 4 * ((n + 127) // 128) * (k // 128) + 2 * m * k + 2 * m * n


def fp8_gemms(torch, w12, wi, np, dev, n_copies, per, batched, check):
    """FP8 GEMM routing: the MLP matrices in FP8 checkpoint form (the Gaussian draw of the
    device generator quantized to E4M3 with 128 x 128 block scales) at every M of the step
    and of the batched regime, beside W12 and the tiled BF16 kernel on the same shapes.
    With `check`, sampled outputs of an untimed pass are checked against the oracle first."""
    res, parity = {}, {}
    for name, n, k, seed, tx in (("gate_up", N_GU, K_GU, 2026_0800, wi.T_X),
                                 ("down", N_DN, K_DN, 2026_0801, wi.T_X2)):
        q0, s0 = wi.device_f8_weight(torch, seed, n, k, dev)
        q_rows, s_rows = q0[:128].cpu().numpy(), s0[:1].cpu().numpy()
        copies = [w12.f8_tile(q0)]
        del q0
        while len(copies) < n_copies(n * k):
            copies.append(copies[0].clone())
        for m in MS + BATCHED_MS:
            x_host = wi.activations(3, tx, m, k)
            x = torch.from_numpy(x_host.view(np.int16)).to(dev)
            y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            key = f"M{m}_{name}"
            if check:
                w12.gemm_f8(x, copies[0], s0, n, k, out=y)
                y_rows = y[:, :128].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
                parity[key] = f8_parity(x_host, q_rows, s_rows, y_rows)
            us, _ = launch_rounds(torch, lambda i: w12.gemm_f8(x, copies[i % len(copies)], s0, n, k,
                                                               out=y))
            ref = per.get(key) or batched.get(key)
            res[key] = {"us_f8": round(us, 2), "gbps_f8": round(f8_bytes(n, k, m) / us / 1e3, 1),
                        "pct_peak_f8": round(100 * f8_bytes(n, k, m) / us / 1e3 / PEAK_GBPS, 1),
                        "us_w12": ref["us_w12"], "speedup_vs_w12": round(ref["us_w12"] / us, 3),
                        "speedup_vs_bf16_tiled": round(ref["us_bf16_tiled"] / us, 3)}
        del copies
    res["format"] = "E4M3 codes, FP32 scale per 128x128 block, BF16 x, FP32 accumulation"
    res["rotated_copies"] = {"gate_up": n_copies(N_GU * K_GU), "down": n_copies(N_DN * K_DN)}
    if check:
        res["parity_sampled_vs_oracle"] = parity
        if not all(parity.values()):
            raise RuntimeError(f"FP8 GEMM outputs outside the oracle's acceptance rule: {parity}")
    return res


FP8_LAYER_MS = (24, 64, 128)


def fp8_layers(torch, w12, wi, np, dev, rotate_bytes):
    """One decoder layer's GEMMs at the decode-step shapes (q/k/v in one launch, o, gate/up
    in one launch, down; plain products, no RMS), FP8 checkpoint weights against W12
    weights, at M = 24, 64 and 128: microseconds per layer over rotated layer copies."""
    shapes = {name: (n, k) for name, n, k in wi.LAYER_MATS}
    names = [name for name, _, _ in wi.LAYER_MATS]
    f8_bytes_layer = sum(n * k for n, k in shapes.values())
    copies = max(2, -(-int(rotate_bytes) // f8_bytes_layer))
    f8l, w12l = [], []
    for c in range(copies):
        F, W = {}, {}
        for mi, name in enumerate(names):
            n, k = shapes[name]
            q, sc = wi.device_f8_weight(torch, 2026_0900 + 8 * c + mi, n, k, dev)
            F[name] = (w12.f8_tile(q), sc, n)
            del q
            W[name] = w12.encode(wi.device_layer_weight(torch, c, mi, n, k))
        f8l.append(F)
        w12l.append(W)
    torch.cuda.synchronize()
    w12_bytes_layer = sum(t.nbytes() for t in w12l[0].values())
    hid, mlp = shapes["q"][1], shapes["down"][1]
    res = {}
    for m in FP8_LAYER_MS:
        x = torch.from_numpy(wi.activations(5, wi.T_X, m, hid).view(np.int16)).to(dev)
        xd = torch.from_numpy(wi.activations(5, wi.T_X2, m, mlp).view(np.int16)).to(dev)
        ys = {name: torch.empty((m, shapes[name][0]), dtype=torch.bfloat16, device=dev) for name in names}
        io = 2 * m * (3 * hid + mlp) + 2 * m * sum(n for n, _ in shapes.values())

        def calls_f8(F):
            return [w12.prepare_gemm_f8_group(x, [F["q"], F["k"], F["v"]], hid, [ys["q"], ys["k"], ys["v"]]),
                    w12.prepare_gemm_f8(x, F["o"][0], F["o"][1], F["o"][2], hid, ys["o"]),
                    w12.prepare_gemm_f8_group(x, [F["gate"], F["up"]], hid, [ys["gate"], ys["up"]]),
                    w12.prepare_gemm_f8(xd, F["down"][0], F["down"][1], F["down"][2], mlp, ys["down"])]

        def calls_w12(W):
            return [w12.prepare_gemm_group(x, [W["q"], W["k"], W["v"]], [ys["q"], ys["k"], ys["v"]]),
                    w12.prepare_gemm(x, W["o"], ys["o"]),
                    w12.prepare_gemm_group(x, [W["gate"], W["up"]], [ys["gate"], ys["up"]]),
                    w12.prepare_gemm(xd, W["down"], ys["down"])]
        pf = [calls_f8(F) for F in f8l]
        pw = [calls_w12(W) for W in w12l]

        def run(prep):
            def fn(i):
                for c in prep[i % len(prep)]:
                    c()
            return fn
        us_f8, _ = launch_rounds(torch, run(pf))
        us_w12, _ = launch_rounds(torch, run(pw))
        res[f"M{m}"] = {"us_f8": round(us_f8, 2), "gbps_f8": round((f8_bytes_layer + io) / us_f8 / 1e3, 1),
                        "us_w12": round(us_w12, 2),
                        "gbps_w12": round((w12_bytes_layer + io) / us_w12 / 1e3, 1),
                        "speedup_vs_w12": round(us_w12 / us_f8, 3)}
    res["workload"] = ("one decoder layer: q/k/v [5120+1024+1024, 5120] in one launch, o [5120, "
                       "5120], gate/up [2x17408, 5120] in one launch, down [5120, 17408]; FP8 "
                       "checkpoint weights vs W12, no RMS")
    res["rotated_layers"] = copies
    del f8l, w12l
    return res


COPY_BYTES = 1 << 30
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "w12_gemm_traffic.json")


# Sources the GEMM launches of the counter record are built and planned from (the GEMM
# kernel family, its instantiations, the host layer that plans and launches them, the
# internal header, and the streaming-read kernel that calibrates the counters).
TRAFFIC_SOURCES = ("w12_gemm_kernel.h", "w12_gemm_run.hip", "w12_gemm_lut.hip", "w12_gemm_bf16.hip",
                   "w12_gemm_bf16t.hip", "w12_internal.h", "w12_api.cpp", "w12_stream.hip")


def kernel_source_hash() -> str:
    """sha256 over the sources of the GEMM launches: counters taken on other sources do
    not describe the kernels that run now."""
    h = hashlib.sha256()
    files = [os.path.join(ROOT, "lossless_bit_weight_w12_amd", "csrc", f) for f in TRAFFIC_SOURCES]
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(dom_key: str):
    """HBM bytes per launch of the dominant GEMM from the recorded counter passes, or
    None when no record matches the current sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None, "no counter record"
    if rec.get("source_sha256") != kernel_source_hash():
        return None, "kernel sources changed since the counters were taken"
    k = rec.get("launches", {}).get(dom_key)
    if k is None:
        return None, f"no counter record for {dom_key}"
    return int(k["hbm_bytes"]), (f"FETCH_SIZE x {rec['fetch_scale']:.4f} + WRITE_SIZE x "
                                 f"{rec['write_scale']:.4f} per launch ({rec['profile']})")


def bootstrap_ci(np, samples, n_boot: int = 10000, seed: int = 0):
    """95 % bootstrap interval of the median of the per-step times."""
    a = np.asarray(samples, dtype=np.float64)
    if a.size < 2:
        return None
    idx = np.random.default_rng(seed).integers(0, a.size, size=(n_boot, a.size))
    med = np.median(a[idx], axis=1)
    return [round(float(np.percentile(med, 2.5)), 4), round(float(np.percentile(med, 97.5)), 4)]


def gpu_state():
    """Clock, temperature and power of GPU 0 from amd-smi (None where the tool or a
    field is unavailable).  Not under a profiler: its preloaded library would start the
    tool's interpreter with the GPU already initialised."""
    import subprocess
    if "rocprof" in os.environ.get("LD_PRELOAD", ""):
        return None
    try:
        out = subprocess.run(["amd-smi", "metric", "-g", "0", "-c", "-t", "-p", "--json"],
                             capture_output=True, text=True, timeout=30)
        d = json.loads(out.stdout)
    except Exception:
        return None
    if isinstance(d, dict) and "gpu_data" in d:
        d = d["gpu_data"]
    d = d[0] if isinstance(d, list) and d else d

    def find(obj, *keys):
        for k in keys:
            if not isinstance(obj, dict) or k not in obj:
                return None
            obj = obj[k]
        return obj.get("value", obj) if isinstance(obj, dict) else obj
    gfx = [find(d, "clock", f"gfx_{i}", "clk") for i in range(8)]
    gfx = [v for v in gfx if isinstance(v, (int, float))]
    return {"gfx_clk_mhz_max_of_xcds": max(gfx) if gfx else None,
            "mem_clk_mhz": find(d, "clock", "mem_0", "clk"),
            "hotspot_c": find(d, "temperature", "hotspot"),
            "mem_c": find(d, "temperature", "mem"),
            "power_w": find(d, "power", "socket_power")}


def warm(torch, fns, seconds: float):
    """Run fns(i) in turn for at least `seconds` of wall time with the GPU never idle: two
    batches stay queued (the host waits for the batch before the last one), so the GPU
    clock ramps up under continuous load and the host clock follows the GPU."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    i = 0
    pending = []
    while time.perf_counter() - t0 < seconds:
        for f in fns:
            f(i)
        i += 1
        e = torch.cuda.Event()
        e.record()
        pending.append(e)
        if len(pending) > 2:
            pending.pop(0).synchronize()
    torch.cuda.synchronize()


def time_calls(torch, fn, reps: int, warm_s: float = 0.05) -> float:
    """Mean milliseconds per call of fn() over reps calls between one event pair, after
    warm_s seconds of the same calls."""
    warm(torch, [lambda i: fn()], warm_s)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def timed(torch, step_fn, steps: int):
    """Exactly `steps` steps between two synchronisations: mean ms per step over the
    event pair around all of them, and the per-step durations from events recorded
    between the steps (no synchronisation inside the timed region)."""
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for i in range(steps):
        step_fn(i)
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    return ev[0].elapsed_time(ev[steps]) / steps, per


def launch_rounds(torch, fn, reps: int = 100, rounds: int = 3, warm_s: float = 0.03):
    """Per-launch microseconds of fn(i) (i rotating weight copies): rounds of `reps`
    launches between event pairs after warm_s seconds of the same launches; returns the
    median round and the mean over all rounds."""
    warm(torch, [fn], warm_s)
    res = []
    for _ in range(rounds):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        res.append(e0.elapsed_time(e1) / reps * 1e3)
    return statistics.median(res), sum(res) / len(res)


def read_ceiling(torch, w12, sizes, dev, reps: int = 20):
    """Streaming-read ceiling for each byte count: w12_stream_read (the GEMM's nontemporal
    16-byte buffer loads) over windows rotating through 2 GiB, so the 256 MB Infinity
    Cache cannot serve a repeat; the best of several grid sizes, median of three rounds."""
    span = 2 << 30
    buf = torch.empty(span, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    grids = (256, 512, 768, 1024, 1536, 2048, 4096)
    sink = torch.empty(4 * max(grids), dtype=torch.int32, device=dev)
    out = {}
    for name, nbytes in sizes.items():
        nb = nbytes - nbytes % 256
        nwin = max(1, span // nb)          # windows [i nb, (i + 1) nb) inside the 2 GiB
        per = {}
        for wg in grids:
            us, _ = launch_rounds(torch, lambda i: w12.stream_read(buf, (i % nwin) * nb, nb, wg, sink),
                                  reps=reps)
            per[wg] = round(nb / us / 1e3, 1)
        best = max(per, key=per.get)
        out[name] = {"bytes": nb, "gbps": per[best], "pct_of_peak": round(100 * per[best] / PEAK_GBPS, 1),
                     "workgroups": best, "gbps_by_workgroups": per}
    del buf
    return out


def build_decode_stack(torch, w12, wi, np, dev, head=None):
    """The 64-layer stack (+ LM head) of the decode step, drawn on the device and
    encoded by the library, prepared for M = 24 with the seeded draft."""
    from lossless_bit_weight_w12_amd.decode_step import DecodeStack, MATS
    c5 = wi.CONFIG_SHAPES[5]
    vocab, hid, m5 = c5["vocab"], c5["hidden"], c5["m"][0]
    if head is None:
        head = w12.encode(wi.device_lm_head(torch, vocab, hid))
    t0 = time.time()
    shapes = {name: (n, k) for name, n, k in wi.LAYER_MATS}
    layers = []
    for li in range(c5["layers"]):
        L = {}
        for mi, name in enumerate(MATS):
            n, k = shapes[name]
            L[name] = w12.encode(wi.device_layer_weight(torch, li, mi, n, k))
        layers.append(L)
        if li % 16 == 15:
            log(f"bench: {li + 1} layers encoded ({time.time() - t0:.1f} s)")
    torch.cuda.synchronize()
    stack = DecodeStack(layers, head, m5)
    h0 = torch.from_numpy(wi.decode_step_x(m5, hid).view(np.int16)).to(dev)
    d5 = torch.from_numpy(wi.decode_step_draft(vocab, m5)).to(dev)
    stack.prepare(d5)
    return stack, h0


def extra_workloads(torch, w12, wi, np, dev, args):
    """LM-head verification (M = 16) and the 64-layer decode step (M = 24).  Weights
    are drawn on the device (randn * 0.02 -> BF16, seeded) and encoded by the library."""
    c5 = wi.CONFIG_SHAPES[5]
    vocab, hid, m5 = c5["vocab"], c5["hidden"], c5["m"][0]
    t0 = time.time()
    head_bf16 = wi.device_lm_head(torch, vocab, hid)
    head = w12.encode(head_bf16)
    screen = w12.screen_encode(head_bf16)   # the 8-bit screen copy of two-level verification
    torch.cuda.synchronize()
    del head_bf16
    log(f"bench: LM head encoded (W12 and screen copy) in {time.time() - t0:.1f} s; timing verification ...")

    # ---- LM-head greedy verification, M = 16; the BF16-out GEMM of the same shape is timed
    # in alternating rounds with it, so both see the same clock
    x16 = torch.from_numpy(wi.verify_batch_x(0).view(np.int16)).to(dev)
    am, _ = w12.lmhead_verify(x16, head, torch.zeros(0, dtype=torch.int32, device=dev))
    p, r = wi.verify_mismatch(0, vocab)
    draft = am.clone()
    if p < 16:
        draft[p] = (draft[p] + 1 + r) % vocab
    am_out = torch.empty(16, dtype=torch.int32, device=dev)
    acc_out = torch.empty(1, dtype=torch.int32, device=dev)
    vcall = w12.prepare_verify(x16, head, draft, am_out, acc_out)
    am2_out = torch.empty(16, dtype=torch.int32, device=dev)
    acc2_out = torch.empty(1, dtype=torch.int32, device=dev)
    v2call = w12.prepare_verify2(x16, head, screen, draft, am2_out, acc2_out)
    y16 = torch.empty((16, vocab), dtype=torch.bfloat16, device=dev)
    gcall = w12.prepare_gemm(x16, head, y16)
    warm(torch, [lambda i: vcall(), lambda i: v2call(), lambda i: gcall()], WARM_S)
    rv, rv2, rg = [], [], []
    for _ in range(5):
        rv.append(time_calls(torch, vcall, 20, warm_s=0.0))
        rv2.append(time_calls(torch, v2call, 20, warm_s=0.0))
        rg.append(time_calls(torch, gcall, 20, warm_s=0.0))
    ms_verify, ms_v2, ms_gemm16 = statistics.median(rv), statistics.median(rv2), statistics.median(rg)
    accepted = int(acc_out.item())
    # the verification's algorithmic bytes: the W12 head, x, the per-block records of
    # pass 1 (16 B per row and 16-row block, written and read) and the argmax
    v_bytes = head.nbytes() + 2 * 16 * hid + 2 * 16 * 16 * (vocab // 16) + 4 * 16
    g_bytes = head.nbytes() + 2 * 16 * hid + 2 * 16 * vocab
    verify = {
        "workload": f"LM head [{vocab}x{hid}] W12, M=16, greedy verify of a 16-token draft",
        "us_per_verify": round(ms_verify * 1e3, 1),
        "gbps_verify": round(v_bytes / (ms_verify * 1e-3) / 1e9, 1),
        "pct_peak_verify": round(100 * v_bytes / (ms_verify * 1e-3) / 1e9 / PEAK_GBPS, 1),
        "us_gemm_bf16_out_same_shape": round(ms_gemm16 * 1e3, 1),
        "gbps_gemm_same_shape": round(g_bytes / (ms_gemm16 * 1e-3) / 1e9, 1),
        "verify_overhead_us": round((ms_verify - ms_gemm16) * 1e3, 1),
        "accepted": accepted, "planted_mismatch_at": p,
        "accepted_matches_plant": accepted == p}
    log(f"bench: verify {verify['us_per_verify']} us ({verify['gbps_verify']} GB/s), "
        f"GEMM of the same shape {verify['us_gemm_bf16_out_same_shape']} us")

    # ---- two-level verification (the screen copy first, W12 rows only for the logits the
    # screen cannot rule out), timed in the same alternating rounds, and at 1 and 8 rows
    nc2 = w12.verify2_candidates(head, 16).cpu().numpy()
    two = {"workload": verify["workload"] + ", two levels (8-bit screen copy, then W12)",
           "us_per_verify": round(ms_v2 * 1e3, 1),
           "speedup_vs_single_level": round(ms_verify / ms_v2, 3),
           "screen_copy_bytes": screen.nbytes(),
           "screen_bytes_vs_w12": round(screen.nbytes() / head.nbytes(), 4),
           "candidates_per_row_mean": round(float(nc2[:, 0].mean()), 1),
           "candidates_per_row_max": int(nc2[:, 0].max()),
           "rows_needing_exact_sums": int((nc2[:, 1] > 1).sum()),
           "argmax_equals_single_level": bool(torch.equal(am2_out, am_out)),
           "accepted": int(acc2_out.item()), "accepted_matches_plant": int(acc2_out.item()) == p}
    by_m = {}
    for mm in (1, 8):
        xm_ = torch.from_numpy(wi.verify_batch_x(0)[:mm].copy().view(np.int16)).to(dev)
        am_a = torch.empty(mm, dtype=torch.int32, device=dev)
        am_b = torch.empty(mm, dtype=torch.int32, device=dev)
        acc_a = torch.empty(1, dtype=torch.int32, device=dev)
        acc_b = torch.empty(1, dtype=torch.int32, device=dev)
        d_m = draft[:mm].contiguous()
        c1 = w12.prepare_verify(xm_, head, d_m, am_a, acc_a)
        c2 = w12.prepare_verify2(xm_, head, screen, d_m, am_b, acc_b)
        warm(torch, [lambda i: c1(), lambda i: c2()], 0.2)
        r1, r2 = [], []
        for _ in range(3):
            r1.append(time_calls(torch, c1, 20, warm_s=0.0))
            r2.append(time_calls(torch, c2, 20, warm_s=0.0))
        m1_, m2_ = statistics.median(r1), statistics.median(r2)
        by_m[f"M{mm}"] = {"us_single_level": round(m1_ * 1e3, 1), "us_two_level": round(m2_ * 1e3, 1),
                          "speedup": round(m1_ / m2_, 3),
                          "argmax_equal": bool(torch.equal(am_a, am_b)) and int(acc_a.item()) == int(acc_b.item())}
    two["by_m"] = by_m
    verify["two_level"] = two
    log(f"bench: two-level verify {two}")

    # ---- batched verification: 24 requests x 5 rows in one pass over the head
    xb = torch.from_numpy(wi.batched_verify_x().view(np.int16)).to(dev)
    mb = xb.shape[0]
    off, nd, pb, rb = wi.batched_verify_table(vocab)
    amb, _ = w12.lmhead_verify(xb, head, torch.zeros(0, dtype=torch.int32, device=dev))
    draft_b = amb.cpu().numpy().astype(np.int32)
    for r in range(len(nd)):
        if pb[r] < nd[r]:
            i = off[r] + pb[r]
            draft_b[i] = (draft_b[i] + 1 + rb[r]) % vocab
    t_i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    amb_out = torch.empty(mb, dtype=torch.int32, device=dev)
    accb_out = torch.empty(len(nd), dtype=torch.int32, device=dev)
    bcall = w12.prepare_verify_batched(xb, head, t_i32(off), t_i32(nd), t_i32(draft_b), amb_out,
                                       accb_out)
    ms_vb = time_calls(torch, bcall, 30, warm_s=0.1)
    accb = accb_out.cpu().numpy()
    amb2_out = torch.empty(mb, dtype=torch.int32, device=dev)
    accb2_out = torch.empty(len(nd), dtype=torch.int32, device=dev)
    bcall2 = w12.prepare_verify2_batched(xb, head, screen, t_i32(off), t_i32(nd), t_i32(draft_b),
                                         amb2_out, accb2_out)
    ms_vb2 = time_calls(torch, bcall2, 30, warm_s=0.1)
    vb_bytes = head.nbytes() + 2 * mb * hid + 2 * 16 * mb * (vocab // 16) + 4 * mb + 4 * len(nd)
    verify_batched = {
        "workload": f"LM head [{vocab}x{hid}] W12, {len(nd)} requests x {mb // len(nd)} rows "
                    f"(M={mb}), per-request greedy verify of {int(nd[0])}-token drafts",
        "us_per_verify": round(ms_vb * 1e3, 1),
        "gbps_verify": round(vb_bytes / (ms_vb * 1e-3) / 1e9, 1),
        "us_per_request": round(ms_vb * 1e3 / len(nd), 2),
        "accepted_match_plants": bool((accb == np.minimum(pb, nd)).all()),
        "argmax_equals_single_request_call": bool(torch.equal(amb_out, amb)),
        "us_two_level": round(ms_vb2 * 1e3, 1),
        "two_level_equals_single_level": bool(torch.equal(amb2_out, amb_out)) and
                                         bool(torch.equal(accb2_out, accb_out))}
    verify["batched"] = verify_batched
    log(f"bench: batched verify {verify_batched}; building the 64-layer stack ...")

    # ---- decode step, 64 layers + head, M = 24
    t0 = time.time()
    stack, h0 = build_decode_stack(torch, w12, wi, np, dev, head)
    layers = stack.layers

    def one_step():
        stack.h.copy_(h0)
        stack.run()
    ms_step = time_calls(torch, one_step, args.decode_steps, warm_s=WARM_S)
    am_eager, h_eager = stack.argmax.clone(), stack.h.clone()
    # the same step captured once as a HIP graph and replayed (no memset nodes: the
    # library's calls are kernels only); every replay must give the eager answer
    ms_graph, graph_ok = None, None
    if not args.no_graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            stack.prepare(stack.draft)            # marshal the calls on the capture stream
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=side):
                stack.h.copy_(h0)
                stack.run()
        torch.cuda.current_stream().wait_stream(side)
        graph_ok = True
        for _ in range(3):
            graph.replay()
            torch.cuda.synchronize()
            graph_ok = graph_ok and bool(torch.equal(stack.argmax, am_eager)) and \
                bool(torch.equal(stack.h.view(torch.int16), h_eager.view(torch.int16)))
            torch.zeros(1, device=dev).add_(1)    # eager work between the replays
        ms_graph = time_calls(torch, graph.replay, args.decode_steps, warm_s=0.1)
        stack.prepare(stack.draft)                # back to the current stream
    wb, io = stack.weight_bytes(), stack.io_bytes()
    n_params = sum(t.n * t.k for L in layers for t in L.values()) + head.n * head.k
    step = {
        "workload": f"decode step: {c5['layers']} layers x (q,k,v,o,gate,up,down) + LM head "
                    f"verify, M={m5}, RMS-chained, {n_params} params",
        "ms_per_step": round(ms_step, 3),
        "tokens_per_s_equiv": round(1e3 / ms_step, 1),
        "rows_per_s": round(m5 * 1e3 / ms_step, 1),
        "w12_weight_gb": round(wb / 1e9, 3), "io_gb": round(io / 1e9, 4),
        "gbps": round((wb + io) / (ms_step * 1e-3) / 1e9, 1),
        "pct_peak": round(100 * (wb + io) / (ms_step * 1e-3) / 1e9 / PEAK_GBPS, 1),
        "bits_per_weight": round(8 * wb / n_params, 5),
        "timed_steps": args.decode_steps, "setup_s": round(time.time() - t0, 1),
        "ms_per_step_hip_graph": None if ms_graph is None else round(ms_graph, 3),
        "hip_graph_replays_match_eager": graph_ok}
    log(f"bench: decode step {step['ms_per_step']} ms ({step['gbps']} GB/s)")
    return verify, step, head.nbytes()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--rotate-bytes", type=float, default=float(1 << 30),
                    help="bytes of weight copies each timed loop rotates over (defeats the "
                         "256 MB Infinity Cache)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the CPU oracle leg (and with it the sampled parity check)")
    ap.add_argument("--profile-only", action="store_true",
                    help="run a few W12 steps and exit (for rocprofv3)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="with --profile-only: also stream 1 GiB with w12_stream_read and fill "
                         "1 GiB, the known-size kernels that scale the traffic counters")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the LM-head verification and decode-step workloads")
    ap.add_argument("--decode-steps", type=int, default=20)
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph replay of the decode step")
    ap.add_argument("--profile-decode", action="store_true",
                    help="build the 64-layer decode stack, run --steps steps and exit (for rocprofv3)")
    ap.add_argument("--profile-batched", action="store_true",
                    help="run --steps batched GEMMs (W12 at M = 64, 128; FP8 at M = 1, 16, 32, 64, 128) and batched verifications and exit")
    ap.add_argument("--profile-verify", action="store_true",
                    help="run --steps LM-head verifications (M = 16) and exit (for rocprofv3)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (the library "
              f"runs each GEMM and verification on one MI355X; it has no multi-GPU sharding)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    gpu_before = gpu_state()
    import torch
    import w12_inputs as wi
    import lossless_bit_weight_w12_amd as w12

    dev = torch.device("cuda:0")
    if args.profile_verify:
        c5 = wi.CONFIG_SHAPES[5]
        head_bf16 = wi.device_lm_head(torch, c5["vocab"], c5["hidden"])
        head = w12.encode(head_bf16)
        screen = w12.screen_encode(head_bf16)
        del head_bf16
        x16 = torch.from_numpy(wi.verify_batch_x(0).view(np.int16)).to(dev)
        draft = torch.zeros(16, dtype=torch.int32, device=dev)
        for _ in range(args.steps):   # single level, then two levels, alternating
            w12.lmhead_verify(x16, head, draft)
            w12.lmhead_verify2(x16, head, screen, draft)
        torch.cuda.synchronize()
        log("bench: profile-verify run done")
        return
    if args.profile_batched:
        # batched regime: the MLP matrices at 64 and 128 rows (W12, then FP8), then the
        # 24-request verification on the LM head
        for name, t, k in (("gate_up", (N_GU, K_GU), wi.T_W), ("down", (N_DN, K_DN), wi.T_W2)):
            tt = w12.encode(torch.from_numpy(wi.weight(3, k, t).view(np.int16)).to(dev))
            for m in BATCHED_MS:
                xb = torch.from_numpy(wi.activations(3, wi.T_X, m, t[1]).view(np.int16)).to(dev)
                yb_ = torch.empty((m, t[0]), dtype=torch.bfloat16, device=dev)
                for _ in range(args.steps):
                    w12.gemm(xb, tt, out=yb_)
            del tt
        # the same shapes in FP8 checkpoint form (M 1, 16, 32, 64, 128)
        for name, (n, k), seed in (("gate_up", (N_GU, K_GU), 2026_0800), ("down", (N_DN, K_DN), 2026_0801)):
            q0, s0 = wi.device_f8_weight(torch, seed, n, k, dev)
            qt = w12.f8_tile(q0)
            del q0
            for m in (1, 16, 32) + BATCHED_MS:
                xb = torch.from_numpy(wi.activations(3, wi.T_X, m, k).view(np.int16)).to(dev)
                yb_ = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
                for _ in range(args.steps):
                    w12.gemm_f8(xb, qt, s0, n, k, out=yb_)
            del qt
        c5 = wi.CONFIG_SHAPES[5]
        head = w12.encode(wi.device_lm_head(torch, c5["vocab"], c5["hidden"]))
        xb = torch.from_numpy(wi.batched_verify_x().view(np.int16)).to(dev)
        off, nd, _, _ = wi.batched_verify_table(c5["vocab"])
        t_i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
        draft = torch.zeros(xb.shape[0], dtype=torch.int32, device=dev)
        for _ in range(args.steps):
            w12.lmhead_verify_batched(xb, head, t_i32(off), t_i32(nd), draft)
        torch.cuda.synchronize()
        log("bench: profile-batched run done")
        return
    if args.profile_decode:
        stack, h0 = build_decode_stack(torch, w12, wi, np, dev)
        for _ in range(args.steps):
            stack.h.copy_(h0)
            stack.run()
        torch.cuda.synchronize()
        log("bench: profile-decode run done")
        return
    log("bench: generating the MLP-block weights (seeded, host) ...")
    t0 = time.time()
    host_w = {"gate_up": wi.weight(3, wi.T_W, (N_GU, K_GU)), "down": wi.weight(3, wi.T_W2, (N_DN, K_DN))}
    w_gu = torch.from_numpy(host_w["gate_up"].view(np.int16)).to(dev)
    w_dn = torch.from_numpy(host_w["down"].view(np.int16)).to(dev)
    log(f"bench: weights on device in {time.time() - t0:.1f} s; encoding to W12 ...")
    t_gu = [w12.encode(w_gu)]
    t_dn = [w12.encode(w_dn)]
    b_gu, b_dn = [w_gu], [w_dn]

    def n_copies(nbytes):
        return max(2, -(-int(args.rotate_bytes) // int(nbytes)))

    def clone(t):
        return w12.W12Tensor(**{**t.__dict__, "tiles": t.tiles.clone(),
                                "esc_off": t.esc_off.clone(), "esc": t.esc.clone()})
    while len(t_gu) < n_copies(t_gu[0].nbytes()):
        t_gu.append(clone(t_gu[0]))
    while len(t_dn) < n_copies(t_dn[0].nbytes()):
        t_dn.append(clone(t_dn[0]))
    while len(b_gu) < n_copies(2 * N_GU * K_GU):
        b_gu.append(w_gu.clone())
    while len(b_dn) < n_copies(2 * N_DN * K_DN):
        b_dn.append(w_dn.clone())
    # second baseline: the same BF16 weights in 4 KB tiles (full-line streaming loads)
    bt_gu = [w12.bf16_tile(b) for b in b_gu]
    bt_dn = [w12.bf16_tile(b) for b in b_dn]
    xs_host = {}
    for m in MS:
        xs_host[(m, "gate_up")] = wi.activations(3, wi.T_X, m, K_GU)
        xs_host[(m, "down")] = wi.activations(3, wi.T_X2, m, K_DN)
    xs = {m: (torch.from_numpy(xs_host[(m, "gate_up")].view(np.int16)).to(dev),
              torch.from_numpy(xs_host[(m, "down")].view(np.int16)).to(dev)) for m in MS}
    ys = {m: (torch.empty((m, N_GU), dtype=torch.bfloat16, device=dev),
              torch.empty((m, N_DN), dtype=torch.bfloat16, device=dev)) for m in MS}
    yb = {m: (torch.empty((m, N_GU), dtype=torch.bfloat16, device=dev),
              torch.empty((m, N_DN), dtype=torch.bfloat16, device=dev)) for m in MS}
    yt = {m: (torch.empty((m, N_GU), dtype=torch.bfloat16, device=dev),
              torch.empty((m, N_DN), dtype=torch.bfloat16, device=dev)) for m in MS}
    torch.cuda.synchronize()
    # encode throughput (one-off work, reported beside the step): the whole of
    # w12_encode_count (which synchronises to return the codebook) + w12_encode
    enc_reps = 5
    torch.cuda.synchronize()
    t_enc = time.perf_counter()
    for _ in range(enc_reps):
        w12.encode(w_gu)
    torch.cuda.synchronize()
    enc_s = (time.perf_counter() - t_enc) / enc_reps
    encode_info = {"matrix": f"gate+up [{N_GU}x{K_GU}] BF16 -> W12", "ms": round(enc_s * 1e3, 3),
                   "gbps_bf16_read": round(2 * N_GU * K_GU / enc_s / 1e9, 1),
                   "gweights_per_s": round(N_GU * K_GU / enc_s / 1e9, 2)}
    log(f"bench: encode {encode_info}")
    log(f"bench: bits/weight gate+up {t_gu[0].bits_per_weight():.5f}, down {t_dn[0].bits_per_weight():.5f}")
    log(f"bench: W12 bytes gate_up {t_gu[0].nbytes()} down {t_dn[0].nbytes()}")

    def w12_step(c):
        for m in MS:
            w12.gemm(xs[m][0], t_gu[c % len(t_gu)], out=ys[m][0])
            w12.gemm(xs[m][1], t_dn[c % len(t_dn)], out=ys[m][1])

    def bf16_step(c):
        for m in MS:
            w12.gemm_bf16(xs[m][0], b_gu[c % len(b_gu)], out=yb[m][0])
            w12.gemm_bf16(xs[m][1], b_dn[c % len(b_dn)], out=yb[m][1])

    def bf16t_step(c):
        for m in MS:
            w12.gemm_bf16_tiled(xs[m][0], bt_gu[c % len(bt_gu)], N_GU, K_GU, out=yt[m][0])
            w12.gemm_bf16_tiled(xs[m][1], bt_dn[c % len(bt_dn)], N_DN, K_DN, out=yt[m][1])

    if args.profile_only:
        warm(torch, [w12_step, bf16_step], 0.2)   # the GPU clock ramps up under load
        for i in range(args.warmup):
            w12_step(i)
        for i in range(args.steps):
            w12_step(i)
            bf16_step(i)
        # the same GEMMs in FP8 checkpoint form (the FP8 rows of the counter record)
        f8w = {}
        for name, n, k, seed in (("gate_up", N_GU, K_GU, 2026_0800), ("down", N_DN, K_DN, 2026_0801)):
            q0, s0 = wi.device_f8_weight(torch, seed, n, k, dev)
            f8w[name] = (w12.f8_tile(q0), s0, n, k)
            del q0
        yf = {m: (torch.empty((m, N_GU), dtype=torch.bfloat16, device=dev),
                  torch.empty((m, N_DN), dtype=torch.bfloat16, device=dev)) for m in MS}
        for i in range(args.steps):
            for m in MS:
                for j, name in ((0, "gate_up"), (1, "down")):
                    qt, sc, n, k = f8w[name]
                    w12.gemm_f8(xs[m][j], qt, sc, n, k, out=yf[m][j])
        if args.calibrate_copy:
            # known-size kernels for the counters: 1 GiB streamed with the GEMM's
            # nontemporal loads, a 1 GiB fill, and a 1 GiB device copy
            src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
            dst = torch.empty_like(src)
            sink = torch.empty(4 * 4096, dtype=torch.int32, device=dev)
            src.fill_(1)
            torch.cuda.synchronize()
            w12.stream_read(src, 0, COPY_BYTES - 256, 4096, sink)
            dst.copy_(src)
        torch.cuda.synchronize()
        log("bench: profile-only run done")
        return

    step_bytes = sum(gemm_bytes(t_gu[0], m) + gemm_bytes(t_dn[0], m) for m in MS)
    step_bytes_bf16 = sum(bf16_bytes(N_GU, K_GU, m) + bf16_bytes(N_DN, K_DN, m) for m in MS)

    # ---- one untimed pass of every kernel; the CPU oracle (cpu_baseline leg) checks sampled
    # rows of these outputs before anything is timed
    w12_step(0)
    bf16_step(0)
    bf16t_step(0)
    torch.cuda.synchronize()
    cpu_base, parity = None, None
    if not args.no_cpu_baseline:
        bits = lambda t: t[:, :SAMPLE_ROWS].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        gpu_out = {(m, name): {"w12": bits(ys[m][i]), "bf16": bits(yb[m][i]), "bf16_tiled": bits(yt[m][i])}
                   for m in MS for i, name in ((0, "gate_up"), (1, "down"))}
        log("bench: CPU oracle on a bounded sample (timed), checking the GPU outputs on it ...")
        cpu_base, parity = cpu_baseline(host_w, xs_host, gpu_out)
        bad = {k: v for k, v in parity.items() if not all(v.values())}
        if bad:
            raise RuntimeError(f"GPU outputs outside the oracle's acceptance rule: {bad}")
        log(f"bench: sampled parity ok for {len(parity)} (M, matrix) launches x 3 kernels")
    # W12 and BF16 launches that split K the same way add the same products in the same
    # order, so their outputs agree bit for bit; where the BF16 kernel splits K
    # differently the last bit can differ
    same = {f"M{m}_{name}": bool(torch.equal(ys[m][i].view(torch.int16), yb[m][i].view(torch.int16)))
            for m in MS for i, name in ((0, "gate_up"), (1, "down"))}

    # ---- headline: warm-up by time, the caller's warm-up steps, exactly --steps timed steps
    log("bench: timing W12 steps ...")
    warm(torch, [w12_step, bf16_step, bf16t_step], WARM_S)
    for i in range(args.warmup):
        w12_step(i)
    ms_w12, per_w12 = timed(torch, w12_step, args.steps)
    gpu_head = gpu_state()

    # ---- speedups: three interleaved rounds, kinds in rotated order, medians per kind
    log("bench: interleaved W12 / BF16 / tiled-BF16 rounds ...")
    fns = {"w12": w12_step, "bf16": bf16_step, "bf16t": bf16t_step}
    rounds = {k: [] for k in fns}
    for order in (("w12", "bf16", "bf16t"), ("bf16", "bf16t", "w12"), ("bf16t", "w12", "bf16")):
        warm(torch, list(fns.values()), 0.1)
        for kind in order:
            rounds[kind].append(timed(torch, fns[kind], args.steps)[0])
    med = {k: statistics.median(v) for k, v in rounds.items()}
    gpu_rounds = gpu_state()

    # ---- per-(M, matrix) launch durations on rotating copies
    per, mean_us = {}, {}
    for m in MS:
        for name, tl, bl, btl, xi in (("gate_up", t_gu, b_gu, bt_gu, 0),
                                      ("down", t_dn, b_dn, bt_dn, 1)):
            nn, kk = tl[0].n, tl[0].k
            launch = {
                "w12": lambda i: w12.gemm(xs[m][xi], tl[i % len(tl)], out=ys[m][xi]),
                "bf16": lambda i: w12.gemm_bf16(xs[m][xi], bl[i % len(bl)], out=yb[m][xi]),
                "bf16t": lambda i: w12.gemm_bf16_tiled(xs[m][xi], btl[i % len(btl)], nn, kk,
                                                       out=yt[m][xi])}
            res = {}
            for kind, fn in launch.items():
                res[kind], mean_us[(f"M{m}_{name}", kind)] = launch_rounds(torch, fn)
            nbytes = gemm_bytes(tl[0], m)
            per[f"M{m}_{name}"] = {
                "us_w12": round(res["w12"], 2), "us_bf16": round(res["bf16"], 2),
                "gbps_w12": round(nbytes / res["w12"] / 1e3, 1),
                "pct_peak_w12": round(100 * nbytes / res["w12"] / 1e3 / PEAK_GBPS, 1),
                "gbps_bf16": round(bf16_bytes(tl[0].n, tl[0].k, m) / res["bf16"] / 1e3, 1),
                "speedup_vs_bf16": round(res["bf16"] / res["w12"], 3),
                "us_bf16_tiled": round(res["bf16t"], 2),
                "gbps_bf16_tiled": round(bf16_bytes(tl[0].n, tl[0].k, m) / res["bf16t"] / 1e3, 1),
                "speedup_vs_bf16_tiled": round(res["bf16t"] / res["w12"], 3)}
    launch_sum_ms = sum(v["us_w12"] for v in per.values()) / 1e3

    # ---- streaming-read ceiling for the W12 byte counts (and the LM head's)
    log("bench: streaming-read ceiling ...")
    c5 = wi.CONFIG_SHAPES[5]
    head_bytes = w12.tiles_bytes(c5["vocab"], c5["hidden"]) + 4 * (c5["vocab"] // 16 + 1) + 64
    ceil_sizes = {"down_w12": t_dn[0].nbytes(), "gate_up_w12": t_gu[0].nbytes(), "lm_head_w12": head_bytes}
    ceiling = read_ceiling(torch, w12, ceil_sizes, dev)
    for key, v in per.items():
        cg = ceiling["down_w12" if key.endswith("down") else "gate_up_w12"]["gbps"]
        v["pct_of_read_ceiling_w12"] = round(100 * v["gbps_w12"] / cg, 1)
    log(f"bench: read ceiling {ceiling}")

    # batched regime: the same matrices at 64 and 128 rows (several requests' draft
    # rows verified together), W12 against the tiled BF16 kernel
    batched = {}
    for m in BATCHED_MS:
        for name, tl, btl, k in (("gate_up", t_gu, bt_gu, K_GU), ("down", t_dn, bt_dn, K_DN)):
            xb = torch.from_numpy(wi.activations(3, wi.T_X if name == "gate_up" else wi.T_X2,
                                                 m, k).view(np.int16)).to(dev)
            yb_ = torch.empty((m, tl[0].n), dtype=torch.bfloat16, device=dev)
            nn = tl[0].n
            us_w, _ = launch_rounds(torch, lambda i: w12.gemm(xb, tl[i % len(tl)], out=yb_))
            us_b, _ = launch_rounds(torch, lambda i: w12.gemm_bf16_tiled(xb, btl[i % len(btl)], nn, k,
                                                                          out=yb_))
            batched[f"M{m}_{name}"] = {
                "us_w12": round(us_w, 2), "gbps_w12": round(gemm_bytes(tl[0], m) / us_w / 1e3, 1),
                "us_bf16_tiled": round(us_b, 2), "speedup_vs_bf16_tiled": round(us_b / us_w, 3)}
    log(f"bench: batched GEMMs {batched}")
    log("bench: FP8 GEMMs ...")
    fp8 = fp8_gemms(torch, w12, wi, np, dev, n_copies, per, batched, not args.no_cpu_baseline)
    log(f"bench: FP8 GEMMs {fp8}")
    fp8["layer"] = fp8_layers(torch, w12, wi, np, dev, args.rotate_bytes)
    log(f"bench: FP8 / W12 layers {fp8['layer']}")

    # dominant kernel = the (M, matrix) GEMM with the largest share of the step; its
    # achieved bandwidth from the mean launch time over its timed rounds
    dom_key = max(per, key=lambda kk: per[kk]["us_w12"])
    m_dom = int(dom_key.split("_")[0][1:])
    t_dom = t_gu[0] if dom_key.endswith("gate_up") else t_dn[0]
    alg = gemm_bytes(t_dom, m_dom)
    avg_us = mean_us[(dom_key, "w12")]
    traffic, traffic_note = measured_traffic(dom_key)
    roofline = {"bound": "hbm", "achieved": round(alg / avg_us / 1e3, 1), "peak": PEAK_GBPS,
                "unit": "GB/s", "frac": round(alg / avg_us / 1e3 / PEAK_GBPS, 4),
                "traffic": traffic, "traffic_note": traffic_note,
                "kernel": f"w12_gemm {dom_key}", "alg_bytes_per_launch": alg,
                "avg_launch_us": round(avg_us, 2),
                "pct_of_read_ceiling": round(100 * alg / avg_us / 1e3 /
                                             ceiling["down_w12" if dom_key.endswith("down") else "gate_up_w12"]["gbps"], 1)}

    value = step_bytes / (ms_w12 * 1e-3) / 1e9
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_w12, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded BF16 ~N(0,0.02^2) weights, x ~N(0,1))",
        "config": {"workload": "mlp_block gate+up[34816x5120] + down[5120x17408], M in 1,4,8,16,32",
                   "m": list(MS), "rotated_copies": {"w12_gate_up": len(t_gu), "w12_down": len(t_dn),
                                                     "bf16_gate_up": len(b_gu), "bf16_down": len(b_dn)},
                   "bits_per_weight": round(t_gu[0].bits_per_weight(), 5)},
        "pct_of_peak": round(100 * value / PEAK_GBPS, 2),
        "step_ms_median": round(float(np.median(per_w12)), 4),
        "step_ms_ci95": bootstrap_ci(np, per_w12),
        "w12_launch_sum_ms": round(launch_sum_ms, 4),
        "step_vs_launch_sum": round(ms_w12 / launch_sum_ms, 4),
        "gpu_state": {"before": gpu_before, "after_headline": gpu_head, "after_rounds": gpu_rounds},
        "interleaved_ms_per_step": {k: [round(v, 4) for v in vs] for k, vs in rounds.items()},
        "speedup_vs_bf16": round(med["bf16"] / med["w12"], 4),
        "bf16_ms_per_step": round(med["bf16"], 4),
        "bf16_gbps": round(step_bytes_bf16 / (med["bf16"] * 1e-3) / 1e9, 1),
        "speedup_vs_bf16_tiled": round(med["bf16t"] / med["w12"], 4),
        "bf16_tiled_ms_per_step": round(med["bf16t"], 4),
        "bf16_tiled_gbps": round(step_bytes_bf16 / (med["bf16t"] * 1e-3) / 1e9, 1),
        "w12_equals_bf16_bitwise": same,
        "parity_sampled_vs_oracle": parity,
        "per_gemm": per,
        "read_ceiling": ceiling,
        "batched_gemm": batched,
        "fp8_gemm": fp8,
        "encode": encode_info,
        "roofline": roofline,
        "cpu_baseline": cpu_base,
        "host": {"cpu": platform.processor() or platform.machine(),
                 "affinity_cores": len(os.sched_getaffinity(0))},
    }
    if not args.no_extras:
        del t_gu, t_dn, b_gu, b_dn, bt_gu, bt_dn, w_gu, w_dn
        torch.cuda.empty_cache()
        out["lm_head_verify"], out["decode_step"], head_b = extra_workloads(torch, w12, wi, np, dev, args)
        out["lm_head_verify"]["pct_of_read_ceiling"] = round(
            100 * out["lm_head_verify"]["gbps_verify"] / ceiling["lm_head_w12"]["gbps"], 1)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
