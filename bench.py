"""Benchmark of the fused decode + dequantise + GEMV over a Huffman-coded matrix.

Workload: the Llama-3.1-8B MLP up/gate shape, 14336 x 4096, 4-bit codes
q = clamp(rint(N(7.5, 1.8)), 0, 15) coded in pairs (one length-limited
canonical Huffman table per matrix, 64x256 tiles of 32 lanes), fp16 d/m per
256-weight super-block, fp16 x, batch 1 (synthetic inputs, synth.py).

One step = one lw_gemv call (stage, lane decode, dequantise, dot, reduce);
for the three-matrix 70B MLP workload, one lw_gemv per matrix, with the
chained pass (gate, up, lw_swiglu, down on the activations) timed beside it.
Each step reads a different copy of the bundle so that the 256 MB Infinity
Cache cannot serve the weights: the timed bytes come from HBM.  The timed
steps are captured once into a HIP graph and replayed, with HIP events around
the replay on the stream the kernels run on, so the host's per-call launch
cost is not part of the figure (the eager per-step time is reported beside
it as us_per_step_eager).

    python bench.py [--gpus 1] [--steps 200] [--warmup 20]

Prints one JSON line.  Extra flags: --workload NAME (default
q4_up_14336x4096; the others are q4_256x1024, q4_down_4096x14336,
bf16_up_14336x4096 and q6_mlp_70b),
--batch, --no-cpu (skip the oracle CPU baseline), --copy-calib (also run a
plain device copy of known size, for counter calibration).
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
MALL_BYTES = 256 << 20
ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")


# the files a decoding kernel is built from besides its own source: the
# shared decoder, the launch arguments, and the bundle layout it reads
SHARED_SOURCES = ("lane_decode.hpp", "kernels.h", "lw_internal.h", "bundle.cpp", "runtime.hip")


def kernel_source(kind_name: str, batch: int) -> str:
    """Source file of the kernel that dominates a workload's step: the
    matrix-core kernel from batch 8, else the decode kernel of the bundle's
    kind."""
    if batch >= 8:
        return "mfma.hip"
    return "bf16.hip" if kind_name == "bf16" else "fused_q.hip"


def _code_text(text: str) -> str:
    """Source text without comments, whitespace runs collapsed: an edit to a
    comment leaves the digest of the code unchanged."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return re.sub(r"\s+", " ", text).strip()


def sources_digest(kernel_file: str) -> str:
    """Digest of the dominant kernel's sources (their code, comments left
    out): a recorded traffic figure is only reported while the kernel it was
    measured on is unchanged."""
    h = hashlib.sha256()
    for name in sorted(SHARED_SOURCES + (kernel_file,)):
        h.update(name.encode())
        with open(os.path.join(ROOT, "decode_gemv_amd", "csrc", name), encoding="utf-8") as fh:
            h.update(_code_text(fh.read()).encode())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str, batch: int, digest: str):
    """HBM bytes per launch of the dominant kernel from the counter runs
    recorded in profiles/hbm_traffic.txt (FETCH_SIZE and WRITE_SIZE, each
    scaled by its copy-kernel calibration factor), or None when no record
    matches this workload, batch and source digest."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as fh:
        for line in fh:
            f = line.split()
            if not f or f[0].startswith("#"):
                continue
            if f[0] == workload and int(f[1]) == batch and f[3] == digest:
                return int(f[2])
    return None


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="q4_up_14336x4096")
    p.add_argument("--batch", type=int, default=1)
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--no-extras", action="store_true")
    p.add_argument("--copy-calib", action="store_true")
    p.add_argument("--copies", type=int, default=0,
                   help="bundle copies cycled through (default: enough that one pass over their coded "
                        "bytes exceeds twice the MALL; 1 measures with the bundle cache-resident)")
    p.add_argument("--code", choices=("huffman", "compact"), default="huffman",
                   help="code lengths of the timed bundles: the optimal 11-bit-limited Huffman code "
                        "(the format's default) or the opt-in compact code")
    p.add_argument("--trace-stats", metavar="CSV",
                   help="summarise a rocprofv3 kernel trace (kernel_trace.csv) per kernel -- calls, "
                        "mean, median, p10, p90, min, max in us -- and exit")
    return p.parse_args()


def copies_for(nbytes: int) -> int:
    """Copies needed so that one pass over their `nbytes` each (the bytes a
    step reads) exceeds twice the MALL."""
    return int(max(2, min(96, -(-2 * MALL_BYTES // max(nbytes, 1)))))


def trace_stats(path: str) -> list:
    """Per-kernel duration statistics of a rocprofv3 --kernel-trace CSV
    (columns Kernel_Name, Start_Timestamp, End_Timestamp in ns)."""
    import csv
    by = {}
    with open(path) as fh:
        for row in csv.DictReader(fh):
            d = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3
            by.setdefault(row["Kernel_Name"], []).append(d)
    out = []
    for name, v in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        a = np.array(v)
        out.append({"kernel": name, "calls": a.size, "mean_us": round(float(a.mean()), 3),
                    "median_us": round(float(np.median(a)), 3), "p10_us": round(float(np.percentile(a, 10)), 3),
                    "p90_us": round(float(np.percentile(a, 90)), 3), "min_us": round(float(a.min()), 3),
                    "max_us": round(float(a.max()), 3)})
    return out


def host_cpu():
    """The host's CPU model and the cores this process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    return model, cores, os.cpu_count() or cores


def time_loop(torch, fn, n_copies, steps, warmup):
    """Eager launches: HIP events around `steps` calls (includes host launch cost)."""
    for i in range(warmup):
        fn(i % n_copies)
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for i in range(steps):
        fn(i % n_copies)
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps       # ms per step


def time_graph(torch, fn, n_copies, steps, warmup):
    """The same `steps` calls captured once into a HIP graph and replayed:
    HIP events on the replay stream time the GPU work without the host's
    per-call launch cost.  Returns ms per step, or None if capture fails."""
    for i in range(warmup):
        fn(i % n_copies)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    try:
        with torch.cuda.graph(g):
            for i in range(steps):
                fn(i % n_copies)
    except Exception as e:                    # capture unsupported here: eager timing only
        print(f"graph capture failed ({e}); reporting eager timing", file=sys.stderr)
        return None
    g.replay()                                # untimed replay
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(s)
    g.replay()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def cpu_baseline(mat, codes, d, m, xb, batch, coded):
    """The oracle as it stands -- limit-method decode of every tile, then the
    fp64 GEMV -- on the whole matrix: once on one thread, then split by row
    bands over every core this process may use (the C routines release the
    GIL, and row bands are independent, so the threaded result is the same y)."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle as O
    ob = O.build_bundle_q(O.KIND[mat.kind], codes, d, m)
    nbc, nrb = mat.cols // 256, mat.rows // 64

    def band_range(r0, r1):
        syms, _ = O.decode_limit(ob["table"], ob["tile_off"][r0 * nbc:r1 * nbc + 1], ob["words"], ob["spl"])
        q = O.unsymbolise_q(ob["kind"], (r1 - r0) * 64, mat.cols, syms)
        return O.gemv_q(q, d[r0 * 64:r1 * 64], m[r0 * 64:r1 * 64], xb, batch)

    t = time.time()
    y1 = band_range(0, nrb)
    t1 = time.time() - t
    model, cores, nproc = host_cpu()
    parts = 4 * cores
    cuts = [nrb * i // parts for i in range(parts + 1)]
    times = []
    with ThreadPoolExecutor(cores) as ex:
        for _ in range(3):
            t = time.time()
            ys = list(ex.map(lambda i: band_range(cuts[i], cuts[i + 1]), range(parts)))
            times.append(time.time() - t)
    tc = min(times)
    assert np.array_equal(np.concatenate(ys, axis=1), y1), "threaded oracle differs from one thread"
    return {"value": round(coded / tc / 1e9, 4), "unit": "GB/s (coded bytes)", "cores": cores, "kind": "oracle",
            "sample": f"whole {mat.rows}x{mat.cols} matrix, limit-method decode + fp64 GEMV, row bands over "
                      f"{cores} threads, best of 3: {tc * 1e6:.0f} us/matrix; one thread: {t1 * 1e6:.0f} us/matrix",
            "one_thread_value": round(coded / t1 / 1e9, 4), "cpu_model": model, "nproc": nproc}


def pipeline_legs(torch, dg, mat, db, a):
    """"Unweight"'s pipelines on the bf16 matrix: lw_autotune times the fused
    kernels (batch <= 16), full decode + library GEMM, the exponent-only and
    the palette transcode each + the reconstructive GEMM, and the
    reconstructive GEMM over a palette form transcoded once (direct palette),
    the reconstructive pipelines in every variant, at each batch, and keeps
    the fastest per batch bucket (one resident copy of the bundle, as an
    autotuner on the target would see it).  The direct palette's form is
    attached to that copy for the leg and not used by the timed steps."""
    batches = [1, 4, 16, 64, 256, 1024]
    rng = np.random.default_rng(5)
    import synth
    xb = synth.f32_to_bf16_bits(rng.standard_normal((max(batches), mat.cols), dtype=np.float32))
    x = torch.from_numpy(xb.view(np.int16)).cuda()
    y = torch.empty((max(batches), mat.rows), dtype=torch.float32, device="cuda")
    scratch = max(dg.lw_pipeline_scratch_bytes(db, p) for p in range(dg.LW_PIPE_COUNT))
    wbuf = torch.empty(scratch, dtype=torch.uint8, device="cuda")
    pbuf = torch.empty(dg.lw_pipeline_scratch_bytes(db, dg.LW_PIPE_DIRECT_PALETTE), dtype=torch.uint8,
                       device="cuda")
    dg.lw_bundle_attach_palette(db, pbuf)
    us = dg.lw_autotune(db, batches, x, y, wbuf, reps=10)
    names = {dg.LW_PIPE_FUSED: "fused", dg.LW_PIPE_FULL_DECODE: "full_decode", dg.LW_PIPE_EXPONENT: "exponent",
             dg.LW_PIPE_PALETTE: "palette", dg.LW_PIPE_DIRECT_PALETTE: "direct_palette"}
    out = {}
    for i, b in enumerate(batches):
        row = {names[p]: (round(float(us[i, p]), 2) if us[i, p] > 0 else None) for p in names}
        row["chosen"] = names[dg.lw_pipeline_get(db, b)]
        out[f"batch_{b}"] = row
    del wbuf
    return out


def read_probe(torch, dg, nbytes, a):
    """HBM bandwidth of a plain read-only kernel (lw_read_probe), cold: at the
    workload's coded size (a different buffer each step, as for the decoding
    kernels) and over 2 GiB."""
    out = {}
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    for name, size in (("coded_size", (nbytes + 15) // 16 * 16), ("2GiB", 2 << 30)):
        n = copies_for(size)
        bufs = [torch.zeros(size, dtype=torch.uint8, device="cuda") for _ in range(n)]
        f = lambda i: dg.lw_read_probe(bufs[i], sink)
        steps = a.steps if size < (256 << 20) else max(5, a.steps // 20)
        ms = time_graph(torch, f, n, steps, min(a.warmup, steps)) or time_loop(torch, f, n, steps, a.warmup)
        out[name] = {"bytes": size, "us": round(ms * 1e3, 3), "GBs": round(size / (ms * 1e-3) / 1e9, 1),
                     "frac_of_peak": round(size / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del bufs
    return out


def skip_legs(torch, dg, synth, mat, codes, d, m, x, batch, a):
    """Tile-skipping fixed-width GEMV (lw_skip_gemv): the same 4-bit codes and
    scales in the tile-transposed layout with every tile listed and with a
    seeded 40 % launch list, and the representative configuration of the
    skipping kernel's page (1024 x 4096, 2-bit codes, 6 of 16 tiles).  Bytes
    are the traffic ledger: listed tiles' words and scales + x + listed y rows."""
    out = {}

    def leg(words, dm, bits, rows, cols, tiles, xx, name):
        n_act = len(set(int(t) for t in tiles))
        wpr = cols * bits // 32
        ledger = n_act * (wpr * 64 * 4 + (cols // 256) * 64 * 4) + 2 * batch * cols + 4 * batch * 64 * n_act
        per_copy = words.nbytes + dm.nbytes
        n = max(2, -(-2 * MALL_BYTES // per_copy))
        wd = [torch.from_numpy(words.view(np.int32)).cuda() for _ in range(n)]
        dd = [torch.from_numpy(dm.view(np.int32)).cuda() for _ in range(n)]
        td = torch.from_numpy(np.ascontiguousarray(tiles, np.int32)).cuda()
        yy = torch.empty((batch, rows), dtype=torch.float32, device="cuda")
        f = lambda i: dg.lw_skip_gemv(wd[i], dd[i], bits, rows, cols, td, xx, yy, batch)
        ms = time_graph(torch, f, n, a.steps, a.warmup) or time_loop(torch, f, n, a.steps, a.warmup)
        out[name] = {"us": round(ms * 1e3, 3), "active_tiles": n_act, "tiles": rows // 64,
                     "ledger_bytes": ledger, "GBs": round(ledger / (ms * 1e-3) / 1e9, 2)}
        del wd, dd

    words, dm = dg.lw_skip_pack(codes, 4, d, m)
    nt = mat.rows // 64
    leg(words, dm, 4, mat.rows, mat.cols, np.arange(nt, dtype=np.int32), x, "all_tiles")
    leg(words, dm, 4, mat.rows, mat.cols, synth.active_tiles(nt, int(round(0.4 * nt)), 41), x, "active_40pct")
    pc, pd, pm, px = synth.gen_fixed(1024, 4096, 2, 40)
    pw, pdm = dg.lw_skip_pack(pc, 2, pd, pm)
    pxd = torch.from_numpy(np.ascontiguousarray(px[:batch]).view(np.int16)).cuda()
    leg(pw, pdm, 2, 1024, 4096, synth.active_tiles(16, 6, 41), pxd, "page_1024x4096_b2_6of16")
    return out


def rans_leg(torch, dg, kind, codes, a, huffman_us=None, halves=1):
    """Decode-only over the rANS twin of the same codes (lw_rans_decode), the
    decoder ablation: time, coded bytes (words + offsets + table) and the
    ratio to the Huffman decode-only kernel on the same matrix; one stream a
    tile row, or two (halves=2: two independent chains a lane)."""
    rows, cols = codes.shape
    r = dg.lw_rans_build(kind, codes, halves)
    coded = r["words"].nbytes + r["tile_off"].nbytes + 2 * r["freq"].nbytes
    n = copies_for(r["words"].nbytes)
    wd = [torch.from_numpy(r["words"].view(np.int32)).cuda() for _ in range(n)]
    to = torch.from_numpy(r["tile_off"].view(np.int32)).cuda()
    lut = torch.from_numpy(r["lut"].view(np.int32)).cuda()
    out = torch.empty(rows * cols // (2 if kind == dg.LW_Q4_PAIR else 1), dtype=torch.uint8, device="cuda")
    f = lambda i: dg.lw_rans_decode(kind, rows, cols, lut, to, wd[i], r["max_tile_words"], out, halves=halves)
    nd = max(a.steps // 4, 10)
    ms = time_graph(torch, f, n, nd, a.warmup) or time_loop(torch, f, n, nd, a.warmup)
    sym = rows * cols // (2 if kind == dg.LW_Q4_PAIR else 1)
    res = {"us_per_matrix": round(ms * 1e3, 3), "coded_bytes": coded,
           "bits_per_weight": round(8 * coded / (rows * cols), 4),
           "coded_GBs": round(coded / (ms * 1e-3) / 1e9, 2), "symbols_per_s": sym / (ms * 1e-3),
           "max_tile_words": r["max_tile_words"]}
    if huffman_us:
        res["over_huffman_decode_time"] = round(ms * 1e3 / huffman_us, 3)
    del wd
    return res


def timed_bundle_leg(torch, dg, build, mats, inputs, kinds, batch, a):
    """The fused kernel on bundles built by `build` (one copy set rotated
    like the main steps): us per matrix, coded bytes and bits per weight."""
    bl = [build(kinds[mm.kind], inp[0], inp[1], inp[2]) for mm, inp in zip(mats, inputs)]
    inf = [dg.lw_bundle_get_info(b) for b in bl]
    coded = sum(int(i["coded_bytes"]) for i in inf)
    n = copies_for(coded)
    dbs = [[dg.lw_bundle_upload(b, torch.empty(int(i["image_bytes"]), dtype=torch.uint8, device="cuda"))
            for b, i in zip(bl, inf)] for _ in range(n)]
    xs = [torch.from_numpy(np.ascontiguousarray(inp[3][:batch]).view(np.int16)).cuda() for inp in inputs]
    ys = [torch.empty((batch, mm.rows), dtype=torch.float32, device="cuda") for mm in mats]

    def step(i):
        for j in range(len(mats)):
            dg.lw_gemv(dbs[i][j], xs[j], ys[j], batch)

    ms = time_graph(torch, step, n, a.steps, a.warmup) or time_loop(torch, step, n, a.steps, a.warmup)
    weights = sum(mm.rows * mm.cols for mm in mats)
    res = {"us_per_matrix": round(ms * 1e3 / len(mats), 3), "coded_bytes": coded,
           "bits_per_weight": round(8 * coded / weights, 4),
           "coded_GBs": round(coded / (ms * 1e-3) / 1e9, 2)}
    del dbs
    return res


def main():
    a = parse()
    if a.trace_stats:
        for row in trace_stats(a.trace_stats):
            print(json.dumps(row))
        return
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path (asked for {a.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import decode_gemv_amd as dg
    import synth

    mats = synth.WORKLOADS[a.workload]
    kinds = {"q4": dg.LW_Q4_PAIR, "q6": dg.LW_Q6_SINGLE, "bf16": dg.LW_BF16_EXP}
    t0 = time.time()
    inputs, bundles = [], []
    for mat in mats:                      # one matrix, or the three of a 70B MLP pass
        if mat.kind == "bf16":
            w, xb = synth.gen_bf16(mat)
            bundles.append((dg.lw_bundle_build_bf16 if a.code == "huffman" else dg.lw_bundle_build_bf16_compact)(w))
            inputs.append((None, None, None, xb))
            del w
        else:
            codes, d, m, xb = synth.gen_q(mat)
            build = dg.lw_bundle_build_q if a.code == "huffman" else dg.lw_bundle_build_q_compact
            bundles.append(build(kinds[mat.kind], codes, d, m))
            inputs.append((codes, d, m, xb))
    infos = [dg.lw_bundle_get_info(b) for b in bundles]
    build_s = time.time() - t0
    mat = mats[0]
    kind = kinds[mat.kind]
    codes, d, m, xb = inputs[0]

    total_coded = sum(int(i["coded_bytes"]) for i in infos)
    n_copies = a.copies if a.copies > 0 else copies_for(total_coded)
    dbs = []                              # dbs[copy][matrix]
    for _ in range(n_copies):
        row = []
        for b, info in zip(bundles, infos):
            buf = torch.empty(int(info["image_bytes"]), dtype=torch.uint8, device="cuda")
            row.append(dg.lw_bundle_upload(b, buf))
        dbs.append(row)
    torch.cuda.synchronize()
    batch = a.batch
    xs = [torch.from_numpy(np.ascontiguousarray(inp[3][:batch]).view(np.int16)).cuda() for inp in inputs]
    ys = [torch.empty((batch, mm.rows), dtype=torch.float32, device="cuda") for mm in mats]

    def step(i):
        for j in range(len(mats)):
            dg.lw_gemv(dbs[i][j], xs[j], ys[j], batch)

    digest = sources_digest(kernel_source(mat.kind, batch))
    ms_eager = time_loop(torch, step, n_copies, a.steps, a.warmup)
    ms_graph = time_graph(torch, step, n_copies, a.steps, a.warmup)
    ms = ms_graph if ms_graph is not None else ms_eager
    us = ms * 1e3
    coded = sum(int(i["coded_bytes"]) for i in infos)
    twin_bytes = sum(int(i["twin_bytes"]) for i in infos)
    weights = sum(mm.rows * mm.cols for mm in mats)
    algo_bytes = coded + sum(2 * batch * mm.cols + 4 * batch * mm.rows for mm in mats)
    achieved = algo_bytes / (us * 1e-6) / 1e9
    shape = " + ".join(f"{mm.rows}x{mm.cols}" for mm in mats)
    symbols = sum(mm.rows * mm.cols // (2 if mm.kind == "q4" else 1) for mm in mats)
    result = {
        "metric": "fused decode+GEMV us/matrix; coded-byte HBM GB/s and % of MI355X HBM peak",
        "value": round(coded / (us * 1e-6) / 1e9, 2),
        "unit": "GB/s (coded bytes)",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp16 x, fp32 accumulate" if kind != dg.LW_BF16_EXP else "bf16 x, fp32 accumulate",
        "data": "synthetic",
        "config": {"workload": f"{' + '.join(mm.name for mm in mats)}: {shape} {mat.kind} coded, batch {batch}",
                   "matrices": len(mats), "batch": batch, "bundle_copies": n_copies,
                   "code": "optimal 11-bit-limited Huffman" if a.code == "huffman" else "compact (opt-in)",
                   "rotated_coded_bytes": n_copies * coded},
        "timing": "hip graph replay of the timed steps" if ms_graph is not None else "eager launches",
        "us_per_step_eager": round(ms_eager * 1e3, 3),
        "us_per_matrix": round(us / len(mats), 3),
        "us_per_step": round(us, 3),
        "pct_hbm_peak_coded": round(100 * coded / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
        "coded_bytes": coded,
        "bits_per_weight": round(8 * coded / weights, 4),
        "equiv_uncompressed_GBs": round(twin_bytes / (us * 1e-6) / 1e9, 2),
        "B_eff_GBs": round(2 * weights / (us * 1e-6) / 1e9, 2),
        "symbols_per_s": symbols / (us * 1e-6),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic(a.workload, batch, digest),
                     "algorithmic_bytes_per_launch": algo_bytes // len(mats)},
    }

    if not a.no_extras and kind == dg.LW_Q4_PAIR and len(mats) == 1:
        # fixed-width twin on the same codes and scales (latency bar)
        twin, dmw = dg.lw_twin_build(codes, 4, d, m)
        tw0 = torch.from_numpy(twin).cuda()
        dm0 = torch.from_numpy(dmw.view(np.int32)).cuda()
        tn = copies_for(twin.nbytes)
        tws = [tw0.clone() for _ in range(tn)]
        yt = torch.empty_like(ys[0])
        twin_step = lambda i: dg.lw_twin_gemv(tws[i], dm0, 4, mat.rows, mat.cols, xs[0], yt, batch)
        tms = time_graph(torch, twin_step, tn, a.steps, a.warmup) or time_loop(torch, twin_step, tn, a.steps, a.warmup)
        tbytes = twin.nbytes + dmw.nbytes
        result["twin"] = {"us_per_matrix": round(tms * 1e3, 3), "bytes": tbytes,
                          "GBs": round(tbytes / (tms * 1e-3) / 1e9, 2),
                          "fused_over_twin_time": round(us / (tms * 1e3), 3)}
        del tws
        # decode only (restores the packed codes to HBM)
        out = torch.empty(mat.rows * mat.cols // 2, dtype=torch.uint8, device="cuda")
        dec_step = lambda i: dg.lw_decode_only(dbs[i][0], out)
        nd = max(a.steps // 4, 10)
        dms = time_graph(torch, dec_step, n_copies, nd, a.warmup) or time_loop(torch, dec_step, n_copies, nd, a.warmup)
        result["decode_only"] = {"us_per_matrix": round(dms * 1e3, 3),
                                 "symbols_per_s": (mat.rows * mat.cols // 2) / (dms * 1e-3)}
        result["rans_decode_only"] = rans_leg(torch, dg, kind, codes, a, dms * 1e3)
        result["rans2_decode_only"] = rans_leg(torch, dg, kind, codes, a, dms * 1e3, halves=2)
    if not a.no_extras and kind == dg.LW_Q6_SINGLE:
        # decoder ablation on the first 6-bit matrix: Huffman and rANS decode-only
        out = torch.empty(mat.rows * mat.cols, dtype=torch.uint8, device="cuda")
        dec_step = lambda i: dg.lw_decode_only(dbs[i][0], out)
        nd = max(a.steps // 4, 10)
        dms = time_graph(torch, dec_step, n_copies, nd, a.warmup) or time_loop(torch, dec_step, n_copies, nd, a.warmup)
        result["decode_only"] = {"matrix": mat.name, "us_per_matrix": round(dms * 1e3, 3),
                                 "symbols_per_s": (mat.rows * mat.cols) / (dms * 1e-3)}
        del out
        result["rans_decode_only"] = rans_leg(torch, dg, kind, codes, a, dms * 1e3)
        result["rans2_decode_only"] = rans_leg(torch, dg, kind, codes, a, dms * 1e3, halves=2)
    if not a.no_extras and kind == dg.LW_Q4_PAIR and len(mats) == 1 and batch <= 4:
        result["skip_twin"] = skip_legs(torch, dg, synth, mat, codes, d, m, xs[0], batch, a)
    if not a.no_extras and kind != dg.LW_BF16_EXP:
        # the other code of the same matrices, beside the timed one
        other = "compact" if a.code == "huffman" else "huffman"
        build = dg.lw_bundle_build_q_compact if other == "compact" else dg.lw_bundle_build_q
        leg = timed_bundle_leg(torch, dg, build, mats, inputs, kinds, batch, a)
        leg["over_timed_code_time"] = round(leg["us_per_matrix"] / (us / len(mats)), 3)
        result[f"{other}_code"] = leg
    if not a.no_extras and a.workload == "q4_down_4096x14336":
        # the batches the down projection's workload names: 1, 4 and 16 (matrix cores)
        by = {}
        for b in (1, 4, 16):
            leg = timed_bundle_leg(torch, dg, dg.lw_bundle_build_q if a.code == "huffman"
                                   else dg.lw_bundle_build_q_compact, mats, inputs, kinds, b, a)
            by[f"batch_{b}"] = {"us_per_matrix": leg["us_per_matrix"], "coded_GBs": leg["coded_GBs"]}
        result["batches"] = by
    if not a.no_extras and len(mats) == 3 and mats[2].cols == mats[0].rows:
        # the whole MLP pass, chained: gate and up on x, SwiGLU to fp16 h,
        # down on h (each graph step depends on the one before it)
        h = torch.empty((batch, mats[0].rows), dtype=torch.int16, device="cuda")
        yo = torch.empty((batch, mats[2].rows), dtype=torch.float32, device="cuda")

        def pass_step(i):
            dg.lw_gemv(dbs[i][0], xs[0], ys[0], batch)
            dg.lw_gemv(dbs[i][1], xs[0], ys[1], batch)
            dg.lw_swiglu(ys[0], ys[1], h)
            dg.lw_gemv(dbs[i][2], h, yo, batch)

        pms = time_graph(torch, pass_step, n_copies, a.steps, a.warmup) or \
            time_loop(torch, pass_step, n_copies, a.steps, a.warmup)
        result["mlp_pass"] = {"us_per_pass": round(pms * 1e3, 3),
                              "coded_GBs": round(coded / (pms * 1e-3) / 1e9, 2),
                              "over_three_independent_gemvs": round(pms / ms, 4)}
    if not a.no_extras and kind == dg.LW_BF16_EXP and len(mats) == 1:
        result["pipelines"] = pipeline_legs(torch, dg, mat, dbs[0][0], a)
    if not a.no_extras:
        result["attainable_read"] = read_probe(torch, dg, coded, a)
    if a.copy_calib:
        src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calib_bytes"] = src.numel()

    if not a.no_cpu and kind != dg.LW_BF16_EXP and len(mats) == 1:
        result["cpu_baseline"] = cpu_baseline(mat, codes, d, m, xb, batch, coded)
    result["kernel_sources_digest"] = digest
    result["build_s"] = round(build_s, 2)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
