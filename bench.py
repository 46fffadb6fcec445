"""Benchmark of the quantized-GEMV hot path on one MI355X.

Headline step: one batch-1 decode token through the linear layers of a
32-layer 7B-style transformer (4096 hidden, 11008 FFN) with weight-only int8
weights (per-row absmax scales) and bf16 activations: per layer q, k, v, o
(4096 x 4096), gate, up (11008 x 4096) and down (4096 x 11008).  Every layer
has its own weight copy (6.5 GB in total), so nothing is served from the
256 MB Infinity Cache.  Projections that read the same activation share one
grouped launch, so a layer is 4 launches -- (q,k,v), o, (gate,up), down --
and the step's 128 launches are captured once in a HIP graph and replayed.
`value` = weight bytes streamed per second.

Also measured (in the same JSON line): each workload of the suite on its
own (tiny W8A8, the three decode shapes, ternary, sign + residual, W8A8
prefill GEMM with outlier split), the roofline of the dominant kernel and the
CPU oracle's throughput on a bounded sample of the same workload.

HBM traffic (roofline "traffic") comes from two rocprofv3 --pmc passes over
`--profile-workload` (FETCH_SIZE, then WRITE_SIZE), turned into
profiles/hbm_traffic_counters.json by `--summarize-counters`; the figures are
used only while the kernel sources still hash to the values recorded there.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--layers L]
                       [--no-cpu-baseline] [--only-headline]
       python bench.py --profile-workload
       python bench.py --summarize-counters FETCH_DIR WRITE_DIR
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
INT8_MFMA_PEAK_TOPS = 5000.0     # MI355X dense int8 MFMA, TOP/s
FP4_MFMA_PEAK_TFLOPS = 10100.0   # MI355X dense FP4 (MXFP4) MFMA, TFLOP/s
COUNTERS_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_counters.json")
CSRC = os.path.join(ROOT, "quantized_gemv_amd", "csrc")
# sources whose hash keys the recorded counters of each kernel
KERNEL_SOURCES = {
    "qgemv": ("qgemv.hip", "qg_device.h", "qg_launch.h"),
    "qgemm": ("qgemm.hip", "qg_gemm.h", "qg_device.h", "qg_launch.h"),
    "sepq": ("sepq.hip", "qg_device.h", "qg_launch.h"),
}
KERNEL_NAME_KEYS = {"qgemv": "qg::qgemv_kernel", "qgemm": "qgemm_w8a8_kernel", "sepq": "sep_qgemv_kernel"}
COPY_BYTES = 256 << 20           # calibration copy: bytes read and bytes written
COPY_REPS = 2                    # calibration copies: the first copy dispatches of the profiled run


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-headline", action="store_true")
    ap.add_argument("--profile-workload", action="store_true",
                    help="run the calibration copy, 2 decode steps and 2 prefill calls, then exit "
                         "(the workload of the rocprofv3 --pmc passes)")
    ap.add_argument("--hashes-out", metavar="PATH",
                    help="with --profile-workload: write the kernel source hashes the run used to PATH")
    ap.add_argument("--summarize-counters", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "HASHES"),
                    help="turn the two rocprofv3 --pmc output folders (and the hashes written by the "
                         "profiled runs) into " + os.path.relpath(COUNTERS_FILE, ROOT))
    return ap.parse_args()


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def src_hash(kernel):
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(kernel):
    """HBM bytes per launch from the recorded counters, or None when they are
    missing or were taken on other kernel sources."""
    try:
        with open(COUNTERS_FILE) as f:
            cnt = json.load(f)
        rec = cnt["kernels"][kernel]
        if rec.get("src_sha256_16") == src_hash(kernel):
            return rec.get("hbm_bytes_per_launch")
    except (OSError, ValueError, KeyError, TypeError):
        pass
    return None


class Timed:
    """Capture a list of launch closures into one HIP graph; replay and time it."""

    def __init__(self, torch, launches):
        self.torch = torch
        self.n = len(launches)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for f in launches:  # eager warm-up outside the capture
                f()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            for f in launches:
                f()
        torch.cuda.synchronize()

    def run(self, reps):
        """Returns seconds per replay measured with events on the launching
        stream (graph replays run on the current stream)."""
        torch = self.torch
        st = torch.cuda.current_stream()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(reps):
            self.graph.replay()
        e1.record(st)
        e1.synchronize()
        return e0.elapsed_time(e1) / 1e3 / reps


def build_headline(torch, qg, synth, dev, L):
    """Weights of L decode layers (own copy per layer) and the step's launches."""
    shapes = synth.DECODE_7B_SHAPES
    log("quantizing the three 7B projection shapes on the GPU")
    base = {}
    xs = {}
    for name, (n, k) in shapes.items():
        wl = synth.decode_w8a16(n=n, k=k, seed=synth.DECODE_7B_SEEDS[name])
        wq, s_w = qg.quantize_absmax(torch.from_numpy(wl.tensors["w"]).to(dev), per_row=True)
        base[name] = (wq, s_w)
        xs[k] = torch.from_numpy(wl.tensors["x_bf16"]).to(dev).view(torch.bfloat16)
    layer_plan = ["attn_4096x4096"] * 4 + ["ffn_up_11008x4096"] * 2 + ["ffn_down_4096x11008"]
    log("replicating weights for %d layers" % L)
    weights = []  # (name, QWeight, CWeight)
    for _ in range(L):
        for name in layer_plan:
            n, k = shapes[name]
            wq, s_w = base[name]
            W = qg.QWeight(qg.QG_WFMT_INT8, n, k, wq.clone(), s_w.clone())
            weights.append((name, W, W.c_struct()))
    torch.cuda.synchronize()
    ys = {n: torch.empty(n, dtype=torch.bfloat16, device=dev) for n in (4096, 11008)}
    # One decode layer = 4 dependent launches: the projections that read the
    # same activation go in one grouped launch (q, k, v) and (gate, up).
    y_proj = [torch.empty(shapes[name][0], dtype=torch.bfloat16, device=dev) for name in layer_plan]
    groups_per_layer = [[0, 1, 2], [3], [4, 5], [6]]
    launches = []
    keep = []
    for li in range(L):
        for grp in groups_per_layer:
            ws_ = [weights[li * len(layer_plan) + i][1] for i in grp]
            gl = qg.GroupLaunch(ws_, xs[ws_[0].k], [y_proj[i] for i in grp], act_int8=False)
            keep.append(gl)
            launches.append(gl.launch)
    step_bytes = sum(W.n * W.k + 4 * W.n for _, W, _ in weights)  # int8 codes + fp32 per-row scales
    act_bytes = sum(2 * (W.k + W.n) for _, W, _ in weights)       # bf16 x read + y written
    return dict(weights=weights, xs=xs, ys=ys, y_proj=y_proj, launches=launches, keep=keep,
                step_bytes=step_bytes, act_bytes=act_bytes)


def build_prefill(torch, qg, synth, dev, cur_stream):
    """Operands of the 2048 x 4096 x 4096 prefill with 20 outlier channels;
    returns closures for the full call, its split alone and its GEMM alone
    (on the split's outputs; run the split once before timing it)."""
    import ctypes
    wl = synth.prefill_outlier()
    m, k, n, n_out = 2048, 4096, 4096, 20
    idx = wl.tensors["idx"].tolist()
    wdev = torch.from_numpy(wl.tensors["w"]).to(dev)
    wq, s_w = qg.quantize_absmax(wdev, per_row=True)
    w_out = qg.gather_columns_bf16(wdev, idx)
    del wdev
    xp = torch.from_numpy(wl.tensors["x_bf16"]).to(dev).view(torch.bfloat16)
    yp = torch.empty((m, n), dtype=torch.float32, device=dev)
    ws = torch.empty(qg.lib().qg_qgemm_workspace_bytes(m, k, n_out), dtype=torch.uint8, device=dev)
    xq = torch.empty((m, k), dtype=torch.int8, device=dev)
    sx = torch.empty(m, dtype=torch.float32, device=dev)
    ld = qg.out_ld(n_out)  # row stride of the outlier operands (w_out comes back as [n][ld])
    xo = torch.empty((m, ld), dtype=torch.bfloat16, device=dev)
    cidx = (ctypes.c_int32 * n_out)(*idx)
    L = qg.lib()
    hold = (wq, s_w, w_out, xp, yp, ws, xq, sx, xo, cidx)

    def full():
        st = L.qg_qgemm_w8a8_outlier(ctypes.c_void_p(xp.data_ptr()), m, k, cidx, n_out,
                                     ctypes.c_void_p(wq.data_ptr()), ctypes.c_void_p(s_w.data_ptr()),
                                     ctypes.c_void_p(w_out.data_ptr()), ld, n, ctypes.c_void_p(yp.data_ptr()),
                                     None, ctypes.c_void_p(ws.data_ptr()), ws.numel(), ctypes.c_void_p(cur_stream()))
        if st != 0:
            raise RuntimeError("qg_qgemm_w8a8_outlier failed: %s" % qg.status_str(st))

    def split_only():
        st = L.qg_quantize_absmax_split(ctypes.c_void_p(xp.data_ptr()), m, k, cidx, n_out,
                                        ctypes.c_void_p(xq.data_ptr()), ctypes.c_void_p(sx.data_ptr()),
                                        ctypes.c_void_p(xo.data_ptr()), ld, ctypes.c_void_p(cur_stream()))
        if st != 0:
            raise RuntimeError("qg_quantize_absmax_split failed: %s" % qg.status_str(st))

    def gemm_only():
        st = L.qg_qgemm_w8a8(ctypes.c_void_p(xq.data_ptr()), ctypes.c_void_p(sx.data_ptr()),
                             ctypes.c_void_p(xo.data_ptr()), ld, m, k, n_out, ctypes.c_void_p(wq.data_ptr()),
                             ctypes.c_void_p(s_w.data_ptr()), ctypes.c_void_p(w_out.data_ptr()), ld, n,
                             ctypes.c_void_p(yp.data_ptr()), None, ctypes.c_void_p(cur_stream()))
        if st != 0:
            raise RuntimeError("qg_qgemm_w8a8 failed: %s" % qg.status_str(st))
    full.hold = hold
    dims = dict(m=m, k=k, n=n, n_out=n_out, xq=xq, wq=wq, gemm_only=gemm_only, idx=idx)
    # algorithmic HBM bytes of the GEMM kernel: int8 X and W, their scales, the
    # bf16 outlier operands (rows of ld), fp32 Y written
    gemm_bytes = m * k + n * k + 4 * (m + n) + 2 * ld * (m + n) + 4 * m * n
    return full, split_only, dims, gemm_bytes


def profile_workload(args):
    """Fixed workload for the rocprofv3 --pmc passes: a device copy of known
    size (the calibration), two decode steps, two prefill calls and two
    thresholded separated products."""
    import torch
    import quantized_gemv_amd as qg
    import synth
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    qg.lib()
    dev = torch.device("cuda:0")

    def cur_stream():
        return torch.cuda.current_stream().cuda_stream
    src = torch.ones(COPY_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(COPY_REPS):  # before any other copy of the process
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    h = build_headline(torch, qg, synth, dev, args.layers)
    for _ in range(2):
        for f in h["launches"]:
            f()
    torch.cuda.synchronize()
    del h
    torch.cuda.empty_cache()
    full, _, _, _ = build_prefill(torch, qg, synth, dev, cur_stream)
    for _ in range(2):
        full()
    torch.cuda.synchronize()
    del full
    torch.cuda.empty_cache()
    wl = synth.sign_residual_decode()
    sw = qg.split_sep_threshold(torch.from_numpy(wl.tensors["w"]).to(dev), 80, 50)
    xs = torch.from_numpy(wl.tensors["x_bf16"]).to(dev).view(torch.bfloat16)
    for _ in range(2):
        qg.qgemv_sep(sw, xs)
    torch.cuda.synchronize()
    if args.hashes_out:
        with open(args.hashes_out, "w") as f:
            json.dump({k: src_hash(k) for k in KERNEL_SOURCES}, f)
    log("profile workload done")


def _counter_rows(folder, counter):
    """[(dispatch id, kernel name, value)] of one counter from a rocprofv3
    --pmc csv folder, in dispatch order."""
    import csv
    import glob
    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no *counter_collection.csv under %s" % folder)
    rows = []
    for fn in files:
        with open(fn) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    rows.sort()
    return rows


def summarize_counters(fetch_dir, write_dir, hashes_path):
    """Scale the qgemv / qgemm FETCH_SIZE and WRITE_SIZE (KiB per dispatch) by
    what the same counters read for the calibration copy, and record them
    under the source hashes of the kernels the profiled run executed."""
    with open(hashes_path) as f:
        hashes = json.load(f)
    fetch = _counter_rows(fetch_dir, "FETCH_SIZE")
    write = _counter_rows(write_dir, "WRITE_SIZE")

    def calibration(rows):
        cps = [r for r in rows if "copyBuffer" in r[1]][:COPY_REPS]
        if len(cps) < COPY_REPS:
            raise SystemExit("calibration copies not found")
        return cps[0][1], sum(v for _, _, v in cps) / len(cps)

    def kernel_mean(rows, key):
        vals = [(name, v) for _, name, v in rows if key in name]
        if not vals:
            raise SystemExit("no dispatch of a kernel matching %r" % key)
        return sum(v for _, v in vals) / len(vals), len(vals), sorted({name for name, _ in vals})
    ck, cf = calibration(fetch)
    _, cw = calibration(write)
    f_fetch = COPY_BYTES / (cf * 1024.0)
    f_write = COPY_BYTES / (cw * 1024.0)
    out = {"calibration": {"kernel": ck, "dispatches": COPY_REPS, "bytes_read": COPY_BYTES,
                           "bytes_written": COPY_BYTES, "fetch_kib": round(cf, 1), "write_kib": round(cw, 1),
                           "fetch_scale": round(f_fetch, 4), "write_scale": round(f_write, 4)},
           "kernels": {}}
    for kern, key in KERNEL_NAME_KEYS.items():
        fk, nf, names = kernel_mean(fetch, key)
        wk, _, _ = kernel_mean(write, key)
        hbm = fk * 1024.0 * f_fetch + wk * 1024.0 * f_write
        out["kernels"][kern] = {"src_sha256_16": hashes[kern], "dispatches": nf, "kernel_names": names,
                                "fetch_kib_per_dispatch": round(fk, 1), "write_kib_per_dispatch": round(wk, 1),
                                "hbm_bytes_per_launch": round(hbm)}
    with open(COUNTERS_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def main():
    args = parse()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (requested --gpus %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    if args.profile_workload:
        profile_workload(args)
        return

    import numpy as np
    import torch

    import quantized_gemv_amd as qg
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    qg.lib()
    dev = torch.device("cuda:0")

    def cur_stream():
        return torch.cuda.current_stream().cuda_stream

    # ---------------------------------------------------------------- headline stack
    L = args.layers
    h = build_headline(torch, qg, synth, dev, L)
    launches, step_bytes, act_bytes = h["launches"], h["step_bytes"], h["act_bytes"]
    launches_per_step = len(launches)

    log("capturing the decode step (%d launches, %.2f GB of weights)" % (launches_per_step, step_bytes / 1e9))
    step = Timed(torch, launches)
    for _ in range(args.warmup):
        step.graph.replay()
    torch.cuda.synchronize()
    # timed region: K replays, bracketed by device synchronisation, with HIP
    # events recorded on the stream the graph is replayed on
    st = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(st)
    for _ in range(args.steps):
        step.graph.replay()
    e1.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_s = e0.elapsed_time(e1) / 1e3 / args.steps
    ms_per_step = wall / args.steps * 1e3
    value = step_bytes / (wall / args.steps) / 1e9
    # dominant kernel: the W8A16 qgemv (the step contains nothing else)
    per_launch_s = ev_s / launches_per_step
    per_launch_bytes = (step_bytes + act_bytes) / launches_per_step
    achieved = per_launch_bytes / per_launch_s / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": recorded_traffic("qgemv"),
                "kernel": "qgemv_kernel<INT8 weights, bf16 x, bf16 y> (grouped and single launches)",
                "algorithmic_bytes_per_launch": round(per_launch_bytes), "avg_launch_us": round(per_launch_s * 1e6, 3)}
    log("decode step: %.3f ms, %.1f GB/s weights (%.1f%% of HBM peak)" % (ms_per_step, value, 100 * value / HBM_PEAK_GBS))

    result = {
        "metric": "qgemv weight GB/s & % of HBM peak at batch 1; prefill int8 TOPS & % MFMA peak",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "7B-style decode, weight-only int8 (W8A16), batch 1: %d layers x "
                               "[4 x 4096x4096, 2 x 11008x4096, 1 x 4096x11008] per token; "
                               "launches per layer: (q,k,v) grouped, o, (gate,up) grouped, down" % L,
                   "weight_bytes_per_step": step_bytes, "launches_per_step": launches_per_step,
                   "hbm_peak_frac": round(value / HBM_PEAK_GBS, 4)},
        "roofline": roofline,
    }

    if not args.only_headline:
        result["configs"] = bench_configs(torch, qg, synth, np, dev, cur_stream, h["weights"], h["xs"], h["ys"])
        result["prefill"] = result["configs"].pop("prefill_w8a8_outlier")
    result["context"] = {
        "note": "figures quoted from the pages for context; not targets",
        "fp16_7b_bytes_per_token_GB": 14, "fp16_7b_ms_per_token_at_2TBps": 7.0,
        "separated_quant_claimed_decode_speedup": 1.78,
        "qadd_prefill_speedup_dgx_spark": 1.49,
        "this_step_weight_GB": round(step_bytes / 1e9, 3),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(np, synth)
    print(json.dumps(result), flush=True)


def sep_threshold_bytes(torch, sw, skip):
    """Bytes one product reads by definition: the class plane, the residual
    codes actually stored (not the zero tail) and the per-row scales."""
    c = sw.cls.to(torch.int32)
    nres = int(sum(((c >> (2 * i)) & 3).eq(3).sum().item() for i in range(4)))
    if skip:
        return sw.cls.numel() + 4 * sw.n, nres
    return sw.cls.numel() + nres + 8 * sw.n, nres


def bench_sep_threshold(torch, qg, synth, dev, rotate_count):
    wl = synth.sign_residual_decode()
    n, k = wl.tensors["w"].shape
    sw = qg.split_sep_threshold(torch.from_numpy(wl.tensors["w"]).to(dev), 80, 50)
    xs = torch.from_numpy(wl.tensors["x_bf16"]).to(dev).view(torch.bfloat16)
    ys = torch.empty(n, dtype=torch.float32, device=dev)
    out = {}
    for skip in (False, True):
        per, nres = sep_threshold_bytes(torch, sw, skip)
        copies = [qg.SepWeight(sw.cls.clone(), sw.rv if skip else sw.rv.clone(), sw.alpha.clone(), sw.s_r.clone(), k)
                  for _ in range(rotate_count(per))]

        def mk(c):
            return lambda: qg.qgemv_sep(c, xs, skip_residual=skip, y=ys)
        t = Timed(torch, [mk(c) for c in copies])
        t.run(1)
        sec = t.run(5) / t.n
        name = "sep_threshold_skip_residual_28672x8192" if skip else "sep_threshold_28672x8192"
        out[name] = {"us": round(sec * 1e6, 3), "weight_GBps": round(per / sec / 1e9, 1),
                     "hbm_frac": round(per / sec / 1e9 / HBM_PEAK_GBS, 4),
                     "bytes_per_weight": round(per / (n * k), 4), "residual_share": round(nres / (n * k), 4),
                     "weights_per_ns": round(n * k / sec / 1e9, 1), "rotating_copies": len(copies),
                     "algorithmic_bytes": per}
        if not skip:
            out[name]["traffic"] = recorded_traffic("sepq")
        log("%s: %.2f us, %.0f GB/s" % (name, sec * 1e6, per / sec / 1e9))
        del copies, t
        torch.cuda.empty_cache()
    return out


def bench_small_batch(torch, qg, dev, weights, batches=(4, 16)):
    """The headline's decode step (32 layers, the same weights and the same
    four launches per layer) for a batch of M tokens."""
    per_layer = 7
    layers = len(weights) // per_layer
    groups_per_layer = [[0, 1, 2], [3], [4, 5], [6]]
    step_bytes = sum(W.n * W.k + 4 * W.n for _, W, _ in weights)
    out = {}
    for m in batches:
        xs = {k: torch.randn(m, k, device=dev).to(torch.bfloat16) for k in (4096, 11008)}
        ys = [torch.empty((m, W.n), dtype=torch.bfloat16, device=dev) for _, W, _ in weights[:per_layer]]
        launches = []
        for li in range(layers):
            for grp in groups_per_layer:
                ws_ = [weights[li * per_layer + i][1] for i in grp]
                yy = [ys[i] for i in grp]
                launches.append((lambda ws_, yy: (lambda: qg.qgemv_batch_grouped(ws_, xs[ws_[0].k], ys=yy)))(ws_, yy))
        t = Timed(torch, launches)
        t.run(1)
        sec = t.run(5)
        out["small_batch_decode_step_m%d" % m] = {
            "tokens": m, "ms_per_step": round(sec * 1e3, 4), "tokens_per_s": round(m / sec, 1),
            "weight_GBps": round(step_bytes / sec / 1e9, 1), "hbm_frac": round(step_bytes / sec / 1e9 / HBM_PEAK_GBS, 4),
            "launches_per_step": len(launches),
            "note": "32 layers x (q,k,v grouped, o, (gate,up) grouped, down), bf16 MFMA on int8 codes widened in registers"}
        log("small batch m=%d: %.3f ms per step, %.0f tokens/s" % (m, sec * 1e3, m / sec))
        del t, launches
    return out


def bench_mxfp4_prefill(torch, qg, synth, dev, int8_gemm_sec):
    wl = synth.prefill_outlier()
    xb = torch.from_numpy(wl.tensors["x_bf16"]).to(dev).view(torch.bfloat16)
    m, k = xb.shape
    wc, wsc = qg.quantize_mxfp4(torch.from_numpy(wl.tensors["w"]).to(dev))
    n = wc.shape[0]
    xc, xsc = qg.quantize_mxfp4(xb)
    y = torch.empty((m, n), dtype=torch.float32, device=dev)
    ws = torch.empty(int(qg.lib().qg_prefill_mxfp4_workspace_bytes(m, k)), dtype=torch.uint8, device=dev)
    tg = Timed(torch, [lambda: qg.gemm_mxfp4(xc, xsc, wc, wsc, y=y)] * 20)
    tg.run(2)
    sec_gemm = tg.run(10) / 20
    tq = Timed(torch, [lambda: qg.quantize_mxfp4(xb)] * 20)
    tq.run(2)
    sec_q = tq.run(10) / 20
    tp = Timed(torch, [lambda: qg.prefill_mxfp4(xb, wc, wsc, y=y, ws=ws)] * 20)
    tp.run(2)
    sec_call = tp.run(10) / 20
    flops = 2.0 * m * n * k
    tf = flops / sec_gemm / 1e12
    log("mxfp4 prefill: gemm %.1f us (%.0f TFLOP/s), call %.1f us" % (sec_gemm * 1e6, tf, sec_call * 1e6))
    return {"metric": "FP4 TFLOP/s of the MXFP4 GEMM (2*M*N*K / GEMM time)", "shape": "M=2048 K=4096 N=4096",
            "gemm_us": round(sec_gemm * 1e6, 2), "quantize_x_us": round(sec_q * 1e6, 2),
            "call_us": round(sec_call * 1e6, 2), "fp4_TFLOPs": round(tf, 1),
            "mfma_frac": round(tf / FP4_MFMA_PEAK_TFLOPS, 4),
            "speedup_vs_int8_gemm": round(int8_gemm_sec / sec_gemm, 3),
            "note": "format separation: the prefill in the matrix cores' native MXFP4, decode weight-only int8"}


def bench_configs(torch, qg, synth, np, dev, cur_stream, weights, xs, ys):
    out = {}
    GiB = 1 << 30

    def rotate_count(bytes_per_copy):
        return max(2, -(-GiB // bytes_per_copy))

    # -- the three decode shapes on their own, rotating through the stack's copies
    for name in synth.DECODE_7B_SHAPES:
        ws = [(W, cw) for nm, W, cw in weights if nm == name]
        W0 = ws[0][0]
        per = W0.n * W0.k + 4 * W0.n
        ws = ws[:rotate_count(per)]

        def mk(W, cw):
            def f():
                qg.qgemv_launch_raw(cw, qg.QG_ACT_FLOAT, xs[W.k].data_ptr(), qg.QG_BF16, ys[W.n].data_ptr(),
                                    qg.QG_BF16, cur_stream())
            return f
        t = Timed(torch, [mk(W, cw) for W, cw in ws])
        t.run(2)
        sec = t.run(10) / t.n
        out["decode_w8a16_" + name] = {"us": round(sec * 1e6, 3), "weight_GBps": round(per / sec / 1e9, 1),
                                       "hbm_frac": round(per / sec / 1e9 / HBM_PEAK_GBS, 4),
                                       "rotating_copies": len(ws)}
        log("%s: %.2f us, %.0f GB/s" % (name, sec * 1e6, per / sec / 1e9))

    # -- small-batch decode: the same 32-layer step for M tokens at once
    #    (weight-only int8 products of qg_qgemv_batch_grouped on bf16 MFMA)
    out.update(bench_small_batch(torch, qg, dev, weights))

    # -- tiny W8A8 GEMV (launch-latency bound)
    wl = synth.tiny_gemv()
    wq, s_w = qg.quantize_absmax(torch.from_numpy(wl.tensors["w"]).to(dev), per_row=True)
    Wt = qg.QWeight(qg.QG_WFMT_INT8, 256, 256, wq, s_w)
    cwt = Wt.c_struct()
    xt = torch.from_numpy(wl.tensors["x"]).to(dev)
    yt = torch.empty(256, dtype=torch.float32, device=dev)

    def tiny():
        qg.qgemv_launch_raw(cwt, qg.QG_ACT_INT8, xt.data_ptr(), qg.QG_F32, yt.data_ptr(), qg.QG_F32, cur_stream())
    t = Timed(torch, [tiny] * 100)
    t.run(2)
    sec = t.run(10) / t.n
    out["tiny_w8a8_256x256"] = {"us": round(sec * 1e6, 3), "weight_GBps": round((65536 + 1024) / sec / 1e9, 1),
                                "note": "launch-latency bound"}
    log("tiny: %.2f us" % (sec * 1e6))

    # -- ternary 11008 x 4096
    wl = synth.ternary_decode()
    q, gamma = qg.quantize_ternary(torch.from_numpy(wl.tensors["w"]).to(dev))
    packed = qg.pack(q, 2)
    per = packed.numel() + 4
    copies = [qg.QWeight(qg.QG_WFMT_TERNARY2, 11008, 4096, packed.clone(), gamma.clone())
              for _ in range(rotate_count(per))]
    xtn = torch.from_numpy(wl.tensors["x"]).to(dev)
    ytn = torch.empty(11008, dtype=torch.float32, device=dev)
    cws = [W.c_struct() for W in copies]

    def mkt(cw):
        def f():
            qg.qgemv_launch_raw(cw, qg.QG_ACT_INT8, xtn.data_ptr(), qg.QG_F32, ytn.data_ptr(), qg.QG_F32, cur_stream())
        return f
    t = Timed(torch, [mkt(cw) for cw in cws])
    t.run(2)
    sec = t.run(10) / t.n
    out["ternary_11008x4096"] = {"us": round(sec * 1e6, 3), "weight_GBps": round(per / sec / 1e9, 1),
                                 "hbm_frac": round(per / sec / 1e9 / HBM_PEAK_GBS, 4), "rotating_copies": len(copies)}
    log("ternary: %.2f us, %.0f GB/s" % (sec * 1e6, per / sec / 1e9))
    del copies, cws, packed

    # -- the same codes packed five per byte in base 3 (1.6 bits per weight)
    packed = qg.pack_base3(q)
    del q
    per = packed.numel() + 4
    copies = [qg.QWeight(qg.QG_WFMT_TERNARY3, 11008, 4096, packed.clone(), gamma.clone())
              for _ in range(rotate_count(per))]
    cws = [W.c_struct() for W in copies]
    t = Timed(torch, [mkt(cw) for cw in cws])
    t.run(2)
    sec = t.run(10) / t.n
    out["ternary_base3_11008x4096"] = {"us": round(sec * 1e6, 3), "weight_GBps": round(per / sec / 1e9, 1),
                                       "hbm_frac": round(per / sec / 1e9 / HBM_PEAK_GBS, 4),
                                       "bytes": per, "weights_per_ns": round(11008 * 4096 / sec / 1e9, 1),
                                       "rotating_copies": len(copies)}
    log("ternary base 3: %.2f us, %.0f GB/s" % (sec * 1e6, per / sec / 1e9))
    del copies, cws, packed
    torch.cuda.empty_cache()

    # -- group-wise 4-bit weights (two-level scales), W4A16, 11008 x 4096
    wl = synth.q4_decode()
    codes, meta = qg.quantize_q4k(torch.from_numpy(wl.tensors["w"]).to(dev))
    per = codes.numel() + meta.numel()
    copies = [qg.QWeight(qg.QG_WFMT_Q4K, 11008, 4096, codes.clone(), None, resid=meta.clone())
              for _ in range(rotate_count(per))]
    del codes, meta
    xq4 = torch.from_numpy(wl.tensors["x_bf16"]).to(dev).view(torch.bfloat16)
    yq4 = torch.empty(11008, dtype=torch.bfloat16, device=dev)
    cws = [W.c_struct() for W in copies]

    def mkq(cw):
        def f():
            qg.qgemv_launch_raw(cw, qg.QG_ACT_FLOAT, xq4.data_ptr(), qg.QG_BF16, yq4.data_ptr(), qg.QG_BF16,
                                cur_stream())
        return f
    t = Timed(torch, [mkq(cw) for cw in cws])
    t.run(2)
    sec = t.run(10) / t.n
    out["q4k_w4a16_11008x4096"] = {"us": round(sec * 1e6, 3), "weight_GBps": round(per / sec / 1e9, 1),
                                   "hbm_frac": round(per / sec / 1e9 / HBM_PEAK_GBS, 4),
                                   "bits_per_weight": 4.5, "rotating_copies": len(copies)}
    log("q4k: %.2f us, %.0f GB/s" % (sec * 1e6, per / sec / 1e9))
    del copies, cws
    torch.cuda.empty_cache()

    # -- sign backbone + int8 residual, 28672 x 8192
    wl = synth.sign_residual_decode()
    wdev = torch.from_numpy(wl.tensors["w"]).to(dev)
    sign, alpha, rq, s_r = qg.split_sign_residual(wdev)
    sp = qg.pack(sign, 1)
    del sign, wdev
    per = sp.numel() + rq.numel() + 8 * 28672
    copies = [qg.QWeight(qg.QG_WFMT_SIGN1_RES8, 28672, 8192, sp.clone(), alpha.clone(), resid=rq.clone(),
                         scale2=s_r.clone()) for _ in range(rotate_count(per))]
    xsr = torch.from_numpy(wl.tensors["x_bf16"]).to(dev).view(torch.bfloat16)
    ysr = torch.empty(28672, dtype=torch.bfloat16, device=dev)
    cws = [W.c_struct() for W in copies]

    def mks(cw):
        def f():
            qg.qgemv_launch_raw(cw, qg.QG_ACT_FLOAT, xsr.data_ptr(), qg.QG_BF16, ysr.data_ptr(), qg.QG_BF16,
                                cur_stream())
        return f
    t = Timed(torch, [mks(cw) for cw in cws])
    t.run(1)
    sec = t.run(5) / t.n
    out["sign1_res8_28672x8192"] = {"us": round(sec * 1e6, 3), "weight_GBps": round(per / sec / 1e9, 1),
                                    "hbm_frac": round(per / sec / 1e9 / HBM_PEAK_GBS, 4),
                                    "rotating_copies": len(copies)}
    log("sign+residual: %.2f us, %.0f GB/s" % (sec * 1e6, per / sec / 1e9))
    del copies, cws, sp, rq
    torch.cuda.empty_cache()

    # -- the same with the zero-point residual (asymmetric int8, z per row)
    wdev = torch.from_numpy(wl.tensors["w"]).to(dev)
    sign, alpha, rq, s_r, z_r = qg.split_sign_residual_zp(wdev)
    sp = qg.pack(sign, 1)
    del sign, wdev
    per = sp.numel() + rq.numel() + 9 * 28672
    copies = [qg.QWeight(qg.QG_WFMT_SIGN1_RES8Z, 28672, 8192, sp.clone(), alpha.clone(), resid=rq.clone(),
                         scale2=s_r.clone(), zero=z_r.clone()) for _ in range(rotate_count(per))]
    cws = [W.c_struct() for W in copies]
    t = Timed(torch, [mks(cw) for cw in cws])
    t.run(1)
    sec = t.run(5) / t.n
    out["sign1_res8z_28672x8192"] = {"us": round(sec * 1e6, 3), "weight_GBps": round(per / sec / 1e9, 1),
                                     "hbm_frac": round(per / sec / 1e9 / HBM_PEAK_GBS, 4),
                                     "rotating_copies": len(copies)}
    log("sign+zero-point residual: %.2f us, %.0f GB/s" % (sec * 1e6, per / sec / 1e9))
    del copies, cws, sp, rq
    torch.cuda.empty_cache()

    # -- thresholded separated weights (80th-percentile backbone, 50th-percentile
    #    zero class), int8 activations, same weights and x as the line above
    out.update(bench_sep_threshold(torch, qg, synth, dev, rotate_count))

    # -- W8A8 prefill GEMM with outlier split, 2048 x 4096 x 4096, 20 outlier channels
    full, split_only, dims, gemm_bytes = build_prefill(torch, qg, synth, dev, cur_stream)
    m, k, n, n_out = dims["m"], dims["k"], dims["n"], dims["n_out"]
    tf = Timed(torch, [full] * 20)
    tf.run(2)
    sec_full = tf.run(10) / 20
    ts = Timed(torch, [split_only] * 20)
    ts.run(2)
    sec_split = ts.run(10) / 20
    tg = Timed(torch, [dims["gemm_only"]] * 20)  # on the split outputs left by the runs above
    tg.run(2)
    sec_gemm = tg.run(10) / 20
    int8_ops = 2.0 * m * n * (k - n_out)
    bf16_ops = 2.0 * m * n * n_out
    tops = int8_ops / sec_gemm / 1e12
    out["prefill_w8a8_outlier"] = {
        "metric": "int8 TOPS of the W8A8 GEMM (2*M*N*(K-n_out) int8 ops / GEMM time)",
        "shape": "M=2048 K=4096 N=4096 n_out=20",
        "gemm_us": round(sec_gemm * 1e6, 2), "split_us": round(sec_split * 1e6, 2),
        "timing": "HIP-graph replays of 20 launches each, HIP events on the replay stream: "
                  "qg_qgemm_w8a8 (GEMM kernel alone), qg_quantize_absmax_split, qg_qgemm_w8a8_outlier (both)",
        "call_us": round(sec_full * 1e6, 2), "int8_TOPS": round(tops, 1),
        "mfma_frac": round(tops / INT8_MFMA_PEAK_TOPS, 4),
        "call_TOPS": round((int8_ops + bf16_ops) / sec_full / 1e12, 1),
        "roofline": {"bound": "mfma", "achieved": round(tops, 1), "peak": INT8_MFMA_PEAK_TOPS, "unit": "TFLOP/s",
                     "frac": round(tops / INT8_MFMA_PEAK_TOPS, 4), "traffic": recorded_traffic("qgemm"),
                     "algorithmic_bytes_per_launch": gemm_bytes},
        "vendor_int8_gemm_us": vendor_int8_gemm_us(torch, dims["xq"], dims["wq"]),
        "vendor_note": "torch._int_mm (vendor BLAS) on the same int8 operands: int32 product only, "
                       "no rescale or outlier path; context, not a target",
    }
    log("prefill: gemm %.1f us (%.0f TOPS), split %.1f us" % (sec_gemm * 1e6, tops, sec_split * 1e6))

    # -- format-separated prefill: the same activations and weights in MXFP4
    #    (E2M1 + E8M0 per 32) on the block-scaled FP4 matrix cores
    out["prefill_mxfp4"] = bench_mxfp4_prefill(torch, qg, synth, dev, sec_gemm)

    # -- outlier-channel detection on the same activations (run once, offline)
    xp = full.hold[3]
    idx_d = torch.empty(n_out, dtype=torch.int32, device=dev)
    import ctypes
    L = qg.lib()
    ws_d = torch.empty(L.qg_detect_outliers_workspace_bytes(k), dtype=torch.uint8, device=dev)

    def detect():
        st = L.qg_detect_outliers(ctypes.c_void_p(xp.data_ptr()), m, k, n_out, ctypes.c_void_p(idx_d.data_ptr()),
                                  ctypes.c_void_p(ws_d.data_ptr()), ws_d.numel(), ctypes.c_void_p(cur_stream()))
        if st != 0:
            raise RuntimeError("qg_detect_outliers failed: %s" % qg.status_str(st))
    td = Timed(torch, [detect] * 20)
    td.run(2)
    sec_det = td.run(10) / 20
    found = sorted(idx_d.cpu().tolist())
    out["detect_outliers_2048x4096"] = {"us": round(sec_det * 1e6, 2),
                                        "read_GBps": round(2.0 * m * k / sec_det / 1e9, 1),
                                        "finds_planted_channels": found == sorted(dims["idx"]),
                                        "note": "offline, once per model: per-channel ranges by row block, then a one-workgroup select"}
    log("detect: %.1f us" % (sec_det * 1e6))
    return out


def vendor_int8_gemm_us(torch, xq, wq):
    """Time of the vendor int8 GEMM (int32 out) on the same operands, or None."""
    try:
        b = wq.t()
        for _ in range(3):
            torch._int_mm(xq, b)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(50):
            torch._int_mm(xq, b)
        e1.record()
        e1.synchronize()
        return round(e0.elapsed_time(e1) * 1e3 / 50, 2)
    except Exception as e:  # not available in this torch build
        log("vendor int8 GEMM unavailable: %s" % e)
        return None


def cpu_baseline(np, synth):
    """The oracle as it stands (fp64 dequantize-then-multiply) on a bounded
    sample of the headline workload: the seven projections of a few layers."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # threadpoolctl missing: report the affinity size
        threads = len(os.sched_getaffinity(0))
    log("cpu baseline: preparing oracle operands")
    ops = {}
    for name, (n, k) in synth.DECODE_7B_SHAPES.items():
        wl = synth.decode_w8a16(n=n, k=k, seed=synth.DECODE_7B_SEEDS[name])
        wq, s_w = oracle.quantize_absmax(wl.tensors["w"], per_row=True)
        ops[name] = (wq, s_w, wl.tensors["x_bf16"])
    plan = ["attn_4096x4096"] * 4 + ["ffn_up_11008x4096"] * 2 + ["ffn_down_4096x11008"]
    done_bytes = 0
    layers = 0
    t0 = time.perf_counter()
    while True:  # whole layers, until about 12 s of CPU work
        for name in plan:
            wq, s_w, xb = ops[name]
            oracle.y_w8a16(wq, s_w, xb)
            done_bytes += wq.size + 4 * s_w.size
        layers += 1
        el = time.perf_counter() - t0
        if el > 12.0:
            break
    return {"value": round(done_bytes / el / 1e9, 3), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": "%d decode layers (%d projections: 4 x 4096x4096, 2 x 11008x4096, 1 x 4096x11008 each; "
                      "%.2f GB of int8 weights), fp64 dequantize-then-multiply, %.1f s" %
                      (layers, 7 * layers, done_bytes / 1e9, el),
            "host_cpus": os.cpu_count(), "affinity": len(os.sched_getaffinity(0))}


if __name__ == "__main__":
    main()
