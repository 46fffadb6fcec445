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

Also measured (in the same JSON line): the on-box streaming-read ceiling
(qg_probe_stream_read on 4 GiB, and the step's own launch sizes as pure
reads); each workload of the suite on its own (tiny W8A8, the three decode
shapes, ternary, base-3 ternary, 4-bit groups, sign + residual with and
without zero-points, thresholded separated weights, small batches, the W8A8
prefill GEMM with outlier split, the MXFP4 prefill, outlier detection); the
same 32-layer step with ternary, sign + residual and thresholded weights;
the roofline of the dominant kernel; and the CPU oracle's throughput on a
bounded sample of the headline workload plus its seconds on each of the five
workloads.

Recorded profiles (used only while the kernel sources hash as recorded):
  * kernel durations per config (rocprof median / p10 / p90): a rocprofv3
    --kernel-trace run of `bench.py --mark-configs ORDER`, whose separator
    launches split the trace into configs, then `--summarize-trace`;
  * HBM traffic and other counters per config: rocprofv3 --pmc passes over
    `--profile-workload` (FETCH_SIZE, then WRITE_SIZE, then MFMA counters),
    then `--summarize-counters`.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--layers L]
                       [--no-cpu-baseline] [--only-headline] [--mark-configs ORDER]
       python bench.py --profile-workload [--mark-configs ORDER]
       python bench.py --summarize-trace TRACE_DIR ORDER
       python bench.py --summarize-counters ORDER PMC_DIR [PMC_DIR ...]
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
KERNEL_SOURCES = {  # the recorded counters and durations hold while these hash as recorded
    "qgemv": ("qgemv.hip", "qg_device.h", "qg_launch.h"),
    "qgemm": ("qgemm.hip", "qg_gemm.h", "qg_device.h", "qg_launch.h"),
    "sepq": ("sepq.hip", "qg_device.h", "qg_launch.h"),
    "batch": ("qgemv_batch.hip", "qg_gemm.h", "qg_device.h", "qg_launch.h"),
    "mx": ("mx.hip", "qg_gemm.h", "qg_device.h", "qg_launch.h"),
    "quantize": ("quantize.hip", "exact_mean.h", "qg_device.h", "qg_launch.h"),
}
COPY_BYTES = 256 << 20           # calibration copy: bytes read and bytes written


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
    ap.add_argument("--mark-configs", metavar="ORDER_JSON",
                    help="launch a separator kernel before each timed config and write the config order to "
                         "ORDER_JSON (for a rocprofv3 --kernel-trace run of the bench)")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_DIR", "ORDER_JSON"),
                    help="turn the kernel trace of a --mark-configs run into per-config kernel durations "
                         "(median, p10, p90) in " + os.path.relpath(os.path.join(ROOT, "profiles", "kernel_durations.json"), ROOT))
    ap.add_argument("--summarize-counters", nargs="+", metavar="ORDER_JSON_THEN_PMC_DIRS",
                    help="ORDER_JSON of a --profile-workload run, then the rocprofv3 --pmc output folders of its "
                         "passes: per-config counter means (and HBM bytes from FETCH_SIZE / WRITE_SIZE) into "
                         + os.path.relpath(COUNTERS_FILE, ROOT))
    return ap.parse_args()


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


# --mark-configs: a separator launch (the per-tensor absmax quantizer on 8
# values) before each timed config, so that a rocprofv3 kernel trace of the
# run splits into configs; the order is written next to the trace
MARKS = None


def mark(torch, qg, name):
    if MARKS is None:
        return
    import ctypes
    x = MARKS["x"]
    st = qg.lib().qg_quantize_absmax_noalloc(ctypes.c_void_p(x.data_ptr()), qg.QG_F32, 1, 8, qg.QG_PER_TENSOR,
                                             ctypes.c_void_p(MARKS["q"].data_ptr()),
                                             ctypes.c_void_p(MARKS["s"].data_ptr()),
                                             ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    if st != 0:
        raise RuntimeError("separator launch failed: %s" % qg.status_str(st))
    torch.cuda.synchronize()
    MARKS["order"].append(name)


def src_hash(kernel):
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


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
    launch_bytes = [sum(weights[li * len(layer_plan) + i][1].n * weights[li * len(layer_plan) + i][1].k
                        for i in grp) for li in range(L) for grp in groups_per_layer]
    return dict(weights=weights, xs=xs, ys=ys, y_proj=y_proj, launches=launches, keep=keep,
                step_bytes=step_bytes, act_bytes=act_bytes, launch_bytes=launch_bytes)


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
    """Fixed workload for the rocprofv3 --pmc passes, in segments started by
    the separator launch (see mark()): two 256 MiB device copies (the
    calibration of FETCH_SIZE / WRITE_SIZE), then two runs of each kernel
    the bench reports: the W8A16 decode step, the prefill call, the MXFP4
    GEMM, the three W8A16 projection shapes alone, the thresholded (with and
    without the residual), sign + residual (with and without zero-points),
    ternary (2-bit and base 3) and 4-bit products, the small-batch steps at
    16 and 4 tokens, and the ternary, sign + residual and thresholded decode
    steps.
    Launches are eager (no graphs)."""
    import torch
    import quantized_gemv_amd as qg
    import synth
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    qg.lib()
    dev = torch.device("cuda:0")
    global MARKS
    MARKS = {"x": torch.zeros(8, device=dev), "q": torch.empty(8, dtype=torch.int8, device=dev),
             "s": torch.empty(1, device=dev), "order": []}

    def cur_stream():
        return torch.cuda.current_stream().cuda_stream

    def twice(name, fs):
        mark(torch, qg, name)
        for _ in range(2):
            for f in fs:
                f()
        torch.cuda.synchronize()
        mark(torch, qg, "setup")  # what runs until the next profiled config
    src = torch.ones(COPY_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    twice("calibration_copy", [lambda: dst.copy_(src)])
    del src, dst
    h = build_headline(torch, qg, synth, dev, args.layers)
    twice("decode_step_w8a16", h["launches"])
    # the three projection shapes alone (the first layer's copies)
    for name, idx in (("decode_w8a16_attn_4096x4096", 0), ("decode_w8a16_ffn_up_11008x4096", 4),
                      ("decode_w8a16_ffn_down_4096x11008", 6)):
        W1 = h["weights"][idx][1]
        y1 = torch.empty(W1.n, dtype=torch.bfloat16, device=dev)
        twice(name, [lambda W1=W1, y1=y1: qg.qgemv(W1, h["xs"][W1.k], act_int8=False, y=y1)])
    tiled = tiled_weights(qg, h["weights"])
    for m in (16, 4):
        twice("small_batch_decode_step_m%d" % m, small_batch_launches(torch, qg, dev, tiled, m))
    del h, tiled
    torch.cuda.empty_cache()
    full, _, _, _ = build_prefill(torch, qg, synth, dev, cur_stream)
    twice("prefill_w8a8_outlier", [full])
    del full
    wl = synth.prefill_outlier()
    xpf = torch.from_numpy(wl.tensors["x_bf16"]).to(dev).view(torch.bfloat16)
    wc, wsc = qg.quantize_mxfp4(torch.from_numpy(wl.tensors["w"]).to(dev))
    xc, xsc = qg.quantize_mxfp4(xpf)
    ypf = torch.empty((xpf.shape[0], wc.shape[0]), dtype=torch.float32, device=dev)
    twice("prefill_mxfp4", [lambda: qg.gemm_mxfp4(xc, xsc, wc, wsc, y=ypf)])
    del wl, xpf, wc, wsc, xc, xsc, ypf
    torch.cuda.empty_cache()
    wl = synth.sign_residual_decode()
    wdev = torch.from_numpy(wl.tensors["w"]).to(dev)
    xs = torch.from_numpy(wl.tensors["x_bf16"]).to(dev).view(torch.bfloat16)
    sw = qg.split_sep_threshold(wdev, 80, 50)
    twice("sep_threshold_28672x8192", [lambda: qg.qgemv_sep(sw, xs)])
    twice("sep_threshold_skip_residual_28672x8192", [lambda: qg.qgemv_sep(sw, xs, skip_residual=True)])
    del sw
    sign, alpha, rq, s_r, z_r = qg.split_sign_residual_zp(wdev)
    Wz = qg.QWeight(qg.QG_WFMT_SIGN1_RES8Z, 28672, 8192, qg.pack(sign, 1), alpha, resid=rq, scale2=s_r, zero=z_r)
    del sign
    twice("sign1_res8z_28672x8192", [lambda: qg.qgemv(Wz, xs, act_int8=False, y_dtype=torch.bfloat16)])
    del Wz, rq
    torch.cuda.empty_cache()
    sign, alpha, rq, s_r = qg.split_sign_residual(wdev)
    Wsr = qg.QWeight(qg.QG_WFMT_SIGN1_RES8, 28672, 8192, qg.pack(sign, 1), alpha, resid=rq, scale2=s_r)
    del sign, wdev
    twice("sign1_res8_28672x8192", [lambda: qg.qgemv(Wsr, xs, act_int8=False, y_dtype=torch.bfloat16)])
    del Wsr, rq
    torch.cuda.empty_cache()
    wl = synth.ternary_decode()
    q, gamma = qg.quantize_ternary(torch.from_numpy(wl.tensors["w"]).to(dev))
    Wt = qg.QWeight(qg.QG_WFMT_TERNARY2, 11008, 4096, qg.pack(q, 2), gamma)
    xt = torch.from_numpy(wl.tensors["x"]).to(dev)
    twice("ternary_11008x4096", [lambda: qg.qgemv(Wt, xt, act_int8=True)])
    W3 = qg.QWeight(qg.QG_WFMT_TERNARY3, 11008, 4096, qg.pack_base3(q), gamma)
    twice("ternary_base3_11008x4096", [lambda: qg.qgemv(W3, xt, act_int8=True)])
    del q, Wt, W3
    wl = synth.q4_decode()
    codes, meta = qg.quantize_q4k(torch.from_numpy(wl.tensors["w"]).to(dev))
    Wq4 = qg.QWeight(qg.QG_WFMT_Q4K, 11008, 4096, codes, None, resid=meta)
    xq4 = torch.from_numpy(wl.tensors["x_bf16"]).to(dev).view(torch.bfloat16)
    twice("q4k_w4a16_11008x4096", [lambda: qg.qgemv(Wq4, xq4, act_int8=False, y_dtype=torch.bfloat16)])
    del codes, meta, Wq4
    torch.cuda.empty_cache()
    for fmt in ("ternary2", "sign1_res8", "sep_threshold"):
        launches, _, keep, _ = build_format_step(torch, qg, synth, dev, args.layers, fmt)
        twice("decode_step_" + fmt, launches)
        del launches, keep
        torch.cuda.empty_cache()
    order = args.mark_configs or os.path.join(ROOT, "gpurun_out", "profile_order.json")
    with open(order, "w") as f:
        json.dump({"configs": MARKS["order"], "hashes": {k: src_hash(k) for k in KERNEL_SOURCES},
                   "command": "python bench.py " + " ".join(_rel(a) for a in sys.argv[1:])}, f, indent=1)
    log("profile workload done (%d segments, order in %s)" % (len(MARKS["order"]), order))


def _segments(rows, order_json):
    """Split (dispatch id, kernel, record) rows, in dispatch order, at the
    separator launches; returns [(config, [(kernel, record)])]."""
    with open(order_json) as f:
        order = json.load(f)
    segs, cur = [], None
    for _, name, rec in sorted(rows, key=lambda r: r[0]):
        if SEPARATOR_KERNEL in name:
            cur = []
            segs.append(cur)
        elif cur is not None and "absmax_apply_kernel" not in name:
            cur.append((name, rec))
    if len(segs) != len(order["configs"]):
        raise SystemExit("%d separators, %d configs in %s" % (len(segs), len(order["configs"]), order_json))
    return list(zip(order["configs"], segs)), order


def _rel(path):
    """A path under the repository, relative to its root (as printed in the
    profile summaries)."""
    ap, root = os.path.realpath(path), os.path.realpath(ROOT)
    return os.path.relpath(ap, root) if ap.startswith(root + os.sep) else path


def _pass_counters(d):
    """The counters one rocprofv3 --pmc output folder holds."""
    import csv
    import glob
    names = set()
    for fn in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(fn) as f:
            for r in csv.DictReader(f):
                names.add(r["Counter_Name"])
    return sorted(names)


def summarize_counters(order_json, dirs):
    """Per config and kernel, the mean of every counter collected in the
    rocprofv3 --pmc output folders `dirs` (one pass each) of a
    --profile-workload run.  FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are
    scaled to bytes by what they read for the calibration copies (256 MiB read
    and written each)."""
    import csv
    import glob
    per = {}  # config -> kernel -> counter -> [values]
    order = None
    for d in dirs:
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit("no *counter_collection.csv under %s" % d)
        disp = {}
        for fn in files:
            with open(fn) as f:
                for r in csv.DictReader(f):
                    did = int(r["Dispatch_Id"])
                    e = disp.setdefault(did, [r["Kernel_Name"], {}])
                    e[1][r["Counter_Name"]] = e[1].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        segs, order = _segments([(did, v[0], v[1]) for did, v in disp.items()], order_json)
        for cfg, recs in segs:
            for name, cnt in recs:
                k = per.setdefault(cfg, {}).setdefault(name, {})
                for c, v in cnt.items():
                    k.setdefault(c, []).append(v)
    # the calibration segment holds exactly the two 256 MiB copies (the
    # runtime may split each into several copy dispatches)
    cal = per.get("calibration_copy", {})
    fk = sum(v for c in cal.values() for v in c.get("FETCH_SIZE", []))
    wk = sum(v for c in cal.values() for v in c.get("WRITE_SIZE", []))
    f_fetch = 2 * COPY_BYTES / (fk * 1024.0) if fk else None
    f_write = 2 * COPY_BYTES / (wk * 1024.0) if wk else None
    out = {"source_hashes": order["hashes"], "command": order.get("command", ""),
           "calibration": {"copies": 2, "bytes_read_each": COPY_BYTES, "bytes_written_each": COPY_BYTES,
                           "fetch_kib_total": round(fk, 1), "write_kib_total": round(wk, 1),
                           "fetch_scale": f_fetch and round(f_fetch, 4), "write_scale": f_write and round(f_write, 4)},
           "configs": {}}
    for cfg, ks in per.items():
        if cfg in ("calibration_copy", "setup"):
            continue
        rec = {}
        for name, cnt in ks.items():
            if "copyBuffer" in name or "FillFunctor" in name or "elementwise" in name:
                continue
            r = {"dispatches": max(len(v) for v in cnt.values())}
            for c, v in sorted(cnt.items()):
                r[c] = round(sum(v) / len(v), 1)
            if "FETCH_SIZE" in r and "WRITE_SIZE" in r and f_fetch and f_write:
                r["hbm_bytes_per_dispatch"] = round(r["FETCH_SIZE"] * 1024.0 * f_fetch + r["WRITE_SIZE"] * 1024.0 * f_write)
            rec[name[:160]] = r
        out["configs"][cfg] = rec
    passes = []
    for d in dirs:  # one rocprofv3 pass per folder, with the counters it holds
        passes.append("rocprofv3 --pmc %s --output-format csv -d $R/%s -o run -- python3 $R/bench.py "
                      "--profile-workload --mark-configs $R/%s" % (" ".join(_pass_counters(d)), _rel(d), _rel(order_json)))
    out["commands"] = passes + ["python3 $R/bench.py --summarize-counters %s" % " ".join(
        "$R/" + _rel(x) for x in [order_json] + list(dirs))]
    with open(COUNTERS_FILE, "w") as f:
        json.dump(out, f, indent=1)
    cols = ["FETCH_SIZE", "WRITE_SIZE", "hbm_bytes_per_dispatch", "SQ_INSTS_VALU_MFMA_MOPS_I8",
            "SQ_INSTS_VALU_MFMA_MOPS_F6F4", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "SQ_INSTS_VALU",
            "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES"]
    md = ["# Counters per bench config (rocprofv3 --pmc over `bench.py --profile-workload`)", "",
          "Commands (R = the repository root; run from /tmp with TMPDIR=/tmp for rocprofv3's own files; one pass "
          "per counter group, then the summary):", ""] + ["    " + c for c in out["commands"]] + ["",
          "Calibration: %s" % json.dumps(out["calibration"]), "",
          "| config | kernel | dispatches | " + " | ".join(cols) + " |", "|---|---|---|" + "---|" * len(cols)]
    for cfg, ks in out["configs"].items():
        for name, r in ks.items():
            md.append("| %s | `%s` | %d | " % (cfg, name[:80], r["dispatches"]) +
                      " | ".join(str(r.get(c, "")) for c in cols) + " |")
    # the memory pipeline (address unit TA, data unit TD, vector L1 TCP, L2
    # TCC), where those passes were taken: cycles and requests summed over
    # the block instances, per dispatch
    mem = sorted({c for ks in out["configs"].values() for r in ks.values() for c in r
                  if c.split("_")[0] in ("TA", "TD", "TCP", "TCC") and c not in cols})
    if mem:
        md += ["", "Memory pipeline counters (summed over block instances, mean per dispatch):", "",
               "| config | kernel | " + " | ".join(mem) + " |", "|---|---|" + "---|" * len(mem)]
        for cfg, ks in out["configs"].items():
            for name, r in ks.items():
                md.append("| %s | `%s` | " % (cfg, name[:80]) + " | ".join(str(r.get(c, "")) for c in mem) + " |")
    with open(COUNTERS_FILE[:-5] + ".md", "w") as f:
        f.write("\n".join(md) + "\n")
    print("\n".join(md[:6]))


def config_sources(cfg):
    """The kernel sources (keys of KERNEL_SOURCES) whose kernels a bench config
    times: a recorded figure of that config holds while these are unchanged."""
    if cfg.startswith("small_batch"):
        return ("batch",)
    if "sep_threshold" in cfg:
        return ("sepq",)
    if cfg.startswith("prefill_w8a8"):
        return ("qgemm", "quantize")
    if cfg.startswith("prefill_mxfp4"):
        return ("mx",)
    if cfg.startswith(("decode_", "tiny_", "ternary", "q4k_", "sign1_")):
        return ("qgemv",)
    return tuple(KERNEL_SOURCES)


def recorded_traffic(cfg, key="qgemv_kernel"):
    """HBM bytes per dispatch of one config's kernels (those whose name holds
    `key`, averaged over their dispatches) from the recorded counters, or None
    when missing or taken on other kernel sources."""
    try:
        with open(COUNTERS_FILE) as f:
            cnt = json.load(f)
        if any(cnt["source_hashes"].get(k) != src_hash(k) for k in config_sources(cfg)):
            return None
        tot = n = 0
        for name, r in cnt["configs"][cfg].items():
            if key in name and "hbm_bytes_per_dispatch" in r and "absmax" not in name:
                tot += r["hbm_bytes_per_dispatch"] * r["dispatches"]
                n += r["dispatches"]
        return round(tot / n) if n else None
    except (OSError, ValueError, KeyError, TypeError, AttributeError):
        return None


DURATIONS_FILE = os.path.join(ROOT, "profiles", "kernel_durations.json")
SEPARATOR_KERNEL = "absmax_partial_kernel"


def summarize_trace(trace_dir, order_json):
    """Per-config kernel durations from a rocprofv3 kernel trace of a
    --mark-configs run: the dispatches between two separator launches belong
    to the config named in the order file; for every kernel with at least 10
    dispatches there, the median, p10, p90 and mean duration."""
    import csv
    import glob
    import numpy as np
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit("no *kernel_trace.csv under %s" % trace_dir)
    rows = []
    for fn in files:
        with open(fn) as f:
            for r in csv.DictReader(f):
                rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"]))
    rows.sort()
    with open(order_json) as f:
        order = json.load(f)
    segments, cur = [], None
    for st, en, name in rows:
        if SEPARATOR_KERNEL in name:
            cur = []
            segments.append(cur)
        elif cur is not None and "absmax_apply_kernel" not in name:
            cur.append((name, (en - st) / 1e3))
    if len(segments) != len(order["configs"]):
        raise SystemExit("%d separators in the trace, %d configs in the order file" % (len(segments), len(order["configs"])))
    out = {"source_hashes": order["hashes"], "command": order.get("command", ""), "configs": {},
           "commands": ["rocprofv3 --kernel-trace --stats --output-format csv -d $R/%s -o run -- python3 $R/%s"
                        % (_rel(trace_dir), order.get("command", "").replace("python ", "", 1).replace(
                            "--mark-configs ", "--mark-configs $R/")),
                        "python3 $R/bench.py --summarize-trace $R/%s $R/%s" % (_rel(trace_dir), _rel(order_json))]}
    for cfg, seg in zip(order["configs"], segments):
        by = {}
        for name, us in seg:
            by.setdefault(name, []).append(us)
        ks = {}
        for name, v in sorted(by.items(), key=lambda kv: -len(kv[1])):
            if len(v) < 10:
                continue
            a = np.array(v)
            ks[name[:160]] = {"dispatches": len(v), "median_us": round(float(np.median(a)), 3),
                              "p10_us": round(float(np.percentile(a, 10)), 3),
                              "p90_us": round(float(np.percentile(a, 90)), 3), "mean_us": round(float(a.mean()), 3)}
        out["configs"][cfg] = ks
    with open(DURATIONS_FILE, "w") as f:
        json.dump(out, f, indent=1)
    md = ["# Kernel durations per bench config (rocprofv3 --kernel-trace)", "",
          "Commands (R = the repository root; run from /tmp with TMPDIR=/tmp for rocprofv3's own files):",
          ""] + ["    " + c for c in out["commands"]] + ["",
          "| config | kernel | dispatches | median us | p10 us | p90 us | mean us |", "|---|---|---|---|---|---|---|"]
    for cfg, ks in out["configs"].items():
        for name, r in ks.items():
            md.append("| %s | `%s` | %d | %.3f | %.3f | %.3f | %.3f |" % (cfg, name[:90], r["dispatches"], r["median_us"],
                                                                      r["p10_us"], r["p90_us"], r["mean_us"]))
    with open(DURATIONS_FILE[:-5] + ".md", "w") as f:
        f.write("\n".join(md) + "\n")
    print("\n".join(md))
    stats = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    if stats:  # the --stats summary of the same run, top kernels by total time
        with open(stats[0]) as f:
            st = list(csv.DictReader(f))
        md = ["# Kernel statistics of the marked bench run (rocprofv3 --kernel-trace --stats)", "",
              "Command (R = the repository root): `%s` (the `*_kernel_stats.csv` it writes)" % out["commands"][0], "",
              "| kernel | calls | average us | min us | max us | share |", "|---|---|---|---|---|---|"]
        for r in st[:30]:
            md.append("| `%s` | %s | %.3f | %.3f | %.3f | %s%% |" % (r["Name"][:110], r["Calls"], float(r["AverageNs"]) / 1e3,
                                                                  float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3,
                                                                  r["Percentage"]))
        with open(os.path.join(ROOT, "profiles", "bench_kernel_stats.md"), "w") as f:
            f.write("\n".join(md) + "\n")


def recorded_durations(cfg):
    """rocprof durations of one config's kernels from the committed summary,
    or None when missing or taken on other kernel sources."""
    try:
        with open(DURATIONS_FILE) as f:
            d = json.load(f)
        if any(d["source_hashes"].get(k) != src_hash(k) for k in config_sources(cfg)):
            return None
        ks = d["configs"].get(cfg)
        return None if ks is None else {n: r for n, r in ks.items() if "qg::" in n}  # this library's kernels
    except (OSError, ValueError, KeyError, TypeError, AttributeError):
        return None


def main():
    args = parse()
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters[0], args.summarize_counters[1:])
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
    global MARKS
    if args.mark_configs:
        MARKS = {"x": torch.zeros(8, device=dev), "q": torch.empty(8, dtype=torch.int8, device=dev),
                 "s": torch.empty(1, device=dev), "order": []}

    def cur_stream():
        return torch.cuda.current_stream().cuda_stream

    # ---------------------------------------------------------------- headline stack
    L = args.layers
    h = build_headline(torch, qg, synth, dev, L)
    launches, step_bytes, act_bytes = h["launches"], h["step_bytes"], h["act_bytes"]
    launches_per_step = len(launches)

    log("capturing the decode step (%d launches, %.2f GB of weights)" % (launches_per_step, step_bytes / 1e9))
    mark(torch, qg, "decode_step_w8a16")
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
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": recorded_traffic("decode_step_w8a16", "qgemv_kernel"),
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

    result["roofline"]["rocprof"] = recorded_durations("decode_step_w8a16")
    mark(torch, qg, "hbm_read_ceiling")
    result["hbm_read_ceiling"] = hbm_read_ceiling(torch, qg, dev, h["launch_bytes"])
    log("HBM read ceiling: %s" % json.dumps(result["hbm_read_ceiling"]))
    if not args.only_headline:
        result["configs"] = bench_configs(torch, qg, synth, np, dev, cur_stream, h["weights"], h["xs"], h["ys"])
        result["prefill"] = result["configs"].pop("prefill_w8a8_outlier")
        del h, launches, step
        torch.cuda.empty_cache()
        result["decode_steps"] = bench_format_steps(torch, qg, synth, dev, L)
        for name, rec in list(result["configs"].items()) + list(result["decode_steps"].items()) + \
                [("prefill_w8a8_outlier", result["prefill"])]:
            if isinstance(rec, dict):
                rec["rocprof"] = recorded_durations(name)
                if "traffic" not in rec:
                    key = {"prefill_mxfp4": "gemm_mxfp4", "decode_step_sep_threshold": "sep_qgemv",
                           "prefill_w8a8_outlier": "qgemm_w8a8"}.get(name, "qgemv_kernel")
                    if name.startswith("small_batch"):
                        key = "qgemv_batch"
                    rec["traffic"] = recorded_traffic(name, key)
    result["context"] = {
        "note": "figures quoted from the pages for context; not targets",
        "fp16_7b_bytes_per_token_GB": 14, "fp16_7b_ms_per_token_at_2TBps": 7.0,
        "separated_quant_claimed_decode_speedup": 1.78,
        "qadd_prefill_speedup_dgx_spark": 1.49,
        "this_step_weight_GB": round(step_bytes / 1e9, 3),
    }
    if MARKS is not None:
        with open(args.mark_configs, "w") as f:
            json.dump({"configs": MARKS["order"], "hashes": {k: src_hash(k) for k in KERNEL_SOURCES},
                       "command": "python bench.py " + " ".join(_rel(a) for a in sys.argv[1:])}, f, indent=1)
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
        mark(torch, qg, "sep_threshold_skip_residual_28672x8192" if skip else "sep_threshold_28672x8192")
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
        out[name]["traffic"] = recorded_traffic(name, "sep_qgemv")
        log("%s: %.2f us, %.0f GB/s" % (name, sec * 1e6, per / sec / 1e9))
        del copies, t
        torch.cuda.empty_cache()
    return out


def small_batch_launches(torch, qg, dev, weights, m):
    """Launch closures of the decode step for a batch of m tokens: per layer
    (q, k, v) and (gate, up) grouped, o and down single launches through
    qg_qgemv_batch_ws (one shared workspace, the launches run in stream
    order; the library splits K where that pays, i.e. for down).  `weights`
    holds row-major or 16-row tiled matrices."""
    per_layer = 7
    layers = len(weights) // per_layer
    xs = {k: torch.randn(m, k, device=dev).to(torch.bfloat16) for k in (4096, 11008)}
    ys = [torch.empty((m, W.n), dtype=torch.bfloat16, device=dev) for _, W, _ in weights[:per_layer]]
    need = max(qg.batch_workspace_bytes(W.n, W.k, m) for _, W, _ in weights[:per_layer])
    wsb = torch.zeros(max(need, 16), dtype=torch.uint8, device=dev)
    launches = []
    for li in range(layers):
        for grp in [[0, 1, 2], [3], [4, 5], [6]]:
            ws_ = [weights[li * per_layer + i][1] for i in grp]
            yy = [ys[i] for i in grp]
            if len(grp) == 1:
                launches.append((lambda W, y: (lambda: qg.qgemv_batch(W, xs[W.k], y=y, ws=wsb)))(ws_[0], yy[0]))
            else:
                launches.append((lambda ws_, yy: (lambda: qg.qgemv_batch_grouped(ws_, xs[ws_[0].k], ys=yy)))(ws_, yy))
    return launches


def tiled_weights(qg, weights):
    """The step's matrices with their codes in 16-row tiles (qg_pack_tiles16)."""
    return [(name, qg.tiled16(W), x) for name, W, x in weights]


def bench_small_batch(torch, qg, dev, weights, batches=(4, 16)):
    """The headline's decode step (32 layers, the same weights and the same
    four launches per layer) for a batch of M tokens, on the weights in the
    16-row tiled layout (and, for reference, on the row-major codes)."""
    step_bytes = sum(W.n * W.k + 4 * W.n for _, W, _ in weights)
    tiled = tiled_weights(qg, weights)
    torch.cuda.synchronize()
    out = {}
    for m in batches:
        mark(torch, qg, "small_batch_decode_step_m%d" % m)
        secs = {}
        for lay, ws_ in (("tiled", tiled), ("row_major", weights)):
            t = Timed(torch, small_batch_launches(torch, qg, dev, ws_, m))
            t.run(1)
            secs[lay] = t.run(5)
            n_launch = t.n
            del t
        sec = secs["tiled"]
        out["small_batch_decode_step_m%d" % m] = {
            "tokens": m, "ms_per_step": round(sec * 1e3, 4), "tokens_per_s": round(m / sec, 1),
            "weight_GBps": round(step_bytes / sec / 1e9, 1), "hbm_frac": round(step_bytes / sec / 1e9 / HBM_PEAK_GBS, 4),
            "launches_per_step": n_launch,
            "ms_per_step_row_major_codes": round(secs["row_major"] * 1e3, 4),
            "note": "32 layers x (q,k,v grouped, o, (gate,up) grouped, down) on int8 codes in 16-row tiles "
                    "(qg_pack_tiles16), widened to bf16 in registers for the MFMAs; down with K split over "
                    "workgroups"}
        log("small batch m=%d: %.3f ms per step (%.3f on row-major codes), %.0f tokens/s"
            % (m, sec * 1e3, secs["row_major"] * 1e3, m / sec))
    del tiled
    torch.cuda.empty_cache()
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
        mark(torch, qg, "decode_w8a16_" + name)
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
    mark(torch, qg, "tiny_w8a8_256x256")
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
    mark(torch, qg, "ternary_11008x4096")
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
    mark(torch, qg, "ternary_base3_11008x4096")
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
    mark(torch, qg, "q4k_w4a16_11008x4096")
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
    mark(torch, qg, "sign1_res8_28672x8192")
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
    mark(torch, qg, "sign1_res8z_28672x8192")
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
    mark(torch, qg, "prefill_w8a8_outlier")
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
                     "frac": round(tops / INT8_MFMA_PEAK_TOPS, 4), "traffic": recorded_traffic("prefill_w8a8_outlier", "qgemm_w8a8"),
                     "algorithmic_bytes_per_launch": gemm_bytes},
        "vendor_int8_gemm_us": vendor_int8_gemm_us(torch, dims["xq"], dims["wq"]),
        "vendor_note": "torch._int_mm (vendor BLAS) on the same int8 operands: int32 product only, "
                       "no rescale or outlier path; context, not a target",
    }
    log("prefill: gemm %.1f us (%.0f TOPS), split %.1f us" % (sec_gemm * 1e6, tops, sec_split * 1e6))

    # -- format-separated prefill: the same activations and weights in MXFP4
    #    (E2M1 + E8M0 per 32) on the block-scaled FP4 matrix cores
    mark(torch, qg, "prefill_mxfp4")
    out["prefill_mxfp4"] = bench_mxfp4_prefill(torch, qg, synth, dev, sec_gemm)

    # -- outlier-channel detection on the same activations (run once, offline)
    mark(torch, qg, "detect_outliers_2048x4096")
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


def hbm_read_ceiling(torch, qg, dev, step_sizes):
    """The on-box streaming-read rate (qg_probe_stream_read: every byte read
    once with 128-bit non-temporal loads, nothing computed), on 4 GiB and as
    the headline step's own sequence of launch sizes replayed as a graph of
    pure reads over distinct buffers -- the floor the qgemv step is compared
    with."""
    import ctypes
    L = qg.lib()
    sink = torch.zeros(65536, dtype=torch.int32, device=dev)
    out = {}
    big = 4 << 30
    buf = torch.ones(big, dtype=torch.uint8, device=dev)
    for wgs in (256, 1024):
        nb = int(L.qg_probe_stream_read_bytes(big, wgs))

        def f():
            st = L.qg_probe_stream_read(ctypes.c_void_p(buf.data_ptr()), big, wgs, ctypes.c_void_p(sink.data_ptr()),
                                        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            if st != 0:
                raise RuntimeError("qg_probe_stream_read: %s" % qg.status_str(st))
        t = Timed(torch, [f] * 4)
        t.run(1)
        sec = t.run(5) / 4
        out["read_4GiB_%dwg_GBps" % wgs] = round(nb / sec / 1e9, 1)
    del buf
    torch.cuda.empty_cache()
    total = sum(step_sizes)
    region = torch.ones(total + (1 << 20), dtype=torch.uint8, device=dev)
    launches, offs, read = [], 0, 0
    for b in step_sizes:
        nb = int(L.qg_probe_stream_read_bytes(b, 256))
        read += nb
        base = region.data_ptr() + offs

        def f(base=base, b=b):
            st = L.qg_probe_stream_read(ctypes.c_void_p(base), b, 256, ctypes.c_void_p(sink.data_ptr()),
                                        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            if st != 0:
                raise RuntimeError("qg_probe_stream_read: %s" % qg.status_str(st))
        launches.append(f)
        offs += (b + 255) // 256 * 256
    t = Timed(torch, launches)
    t.run(2)
    sec = t.run(10)
    out["step_sequence_ms"] = round(sec * 1e3, 4)
    out["step_sequence_GBps"] = round(read / sec / 1e9, 1)
    out["step_sequence_note"] = ("the decode step's %d launch sizes as pure streaming reads (256 workgroups, "
                                 "HIP graph of distinct buffers)" % len(step_sizes))
    best = max(v for k, v in out.items() if k.startswith("read_4GiB"))
    out["ceiling_frac_of_peak"] = round(best / HBM_PEAK_GBS, 4)
    del region
    torch.cuda.empty_cache()
    return out


FORMAT_SEEDS = {"attn_4096x4096": 31, "ffn_up_11008x4096": 32, "ffn_down_4096x11008": 33}


def build_format_step(torch, qg, synth, dev, L, fmt):
    """The headline's 32-layer decode step (same shapes, launches grouped the
    same way, every layer its own weight copy) with the weights in a low-bit
    format: "ternary2" (2-bit ternary, int8 activations), "sign1_res8" (sign
    backbone + int8 residual, bf16 activations) or "sep_threshold"
    (thresholded separated weights, 80th / 50th percentiles, grouped with
    qg_qgemv_sep_grouped).  Returns (launches, weight bytes per step, objects to keep)."""
    shapes = synth.DECODE_7B_SHAPES
    plan = ["attn_4096x4096"] * 4 + ["ffn_up_11008x4096"] * 2 + ["ffn_down_4096x11008"]
    groups_per_layer = [[0, 1, 2], [3], [4, 5], [6]]
    base = {}
    for name, (n, k) in shapes.items():
        if fmt == "ternary2":
            w = torch.from_numpy(synth.ternary_decode(n=n, k=k, seed=FORMAT_SEEDS[name]).tensors["w"]).to(dev)
            q, gamma = qg.quantize_ternary(w)
            base[name] = (qg.pack(q, 2), gamma)
            del q
        else:
            w = torch.from_numpy(synth.sign_residual_decode(n=n, k=k, seed=FORMAT_SEEDS[name]).tensors["w"]).to(dev)
            if fmt == "sign1_res8":
                sign, alpha, rq, s_r = qg.split_sign_residual(w)
                base[name] = (qg.pack(sign, 1), alpha, rq, s_r)
                del sign
            else:
                base[name] = qg.split_sep_threshold(w, 80, 50)
        del w
    torch.cuda.synchronize()
    weights, nbytes = [], 0
    for _ in range(L):
        for name in plan:
            n, k = shapes[name]
            b = base[name]
            if fmt == "ternary2":
                W = qg.QWeight(qg.QG_WFMT_TERNARY2, n, k, b[0].clone(), b[1].clone())
                nbytes += b[0].numel() + 4
            elif fmt == "sign1_res8":
                W = qg.QWeight(qg.QG_WFMT_SIGN1_RES8, n, k, b[0].clone(), b[1].clone(), resid=b[2].clone(),
                               scale2=b[3].clone())
                nbytes += b[0].numel() + b[2].numel() + 8 * n
            else:
                W = qg.SepWeight(b.cls.clone(), b.rv.clone(), b.alpha.clone(), b.s_r.clone(), k)
                nbytes += sep_threshold_bytes(torch, b, False)[0]
            weights.append(W)
    del base
    if fmt == "ternary2":
        xs = {k: torch.randn(k, device=dev) for k in (4096, 11008)}
    else:
        xs = {k: torch.randn(k, device=dev).to(torch.bfloat16) for k in (4096, 11008)}
    launches, keep = [], [weights, xs]
    for li in range(L):
        for grp in groups_per_layer:
            ws_ = [weights[li * len(plan) + i] for i in grp]
            if fmt == "sep_threshold":
                ys_ = [torch.empty(W.n, dtype=torch.float32, device=dev) for W in ws_]
                gl = qg.SepGroupLaunch(ws_, xs[ws_[0].k], ys_)
            else:
                ydt = torch.float32 if fmt == "ternary2" else torch.bfloat16
                ys_ = [torch.empty(W.n, dtype=ydt, device=dev) for W in ws_]
                gl = qg.GroupLaunch(ws_, xs[ws_[0].k], ys_, act_int8=(fmt == "ternary2"))
            keep.append(gl)
            launches.append(gl.launch)
    weights_per_step = L * sum(shapes[nm][0] * shapes[nm][1] for nm in plan)
    return launches, nbytes, keep, weights_per_step


def bench_format_steps(torch, qg, synth, dev, L):
    """The 32-layer decode step in the low-bit formats (see build_format_step)."""
    out = {}
    for fmt in ("ternary2", "sign1_res8", "sep_threshold"):
        mark(torch, qg, "decode_step_" + fmt)
        launches, nbytes, keep, nw = build_format_step(torch, qg, synth, dev, L, fmt)
        t = Timed(torch, launches)
        t.run(2)
        sec = t.run(10)
        out["decode_step_%s" % fmt] = {
            "ms_per_step": round(sec * 1e3, 4), "tokens_per_s": round(1.0 / sec, 1),
            "weight_bytes_per_step": nbytes, "weight_GBps": round(nbytes / sec / 1e9, 1),
            "hbm_frac": round(nbytes / sec / 1e9 / HBM_PEAK_GBS, 4), "launches_per_step": len(launches),
            "bytes_per_weight": round(nbytes / nw, 4)}
        log("decode step %s: %.3f ms, %.0f GB/s of weights" % (fmt, sec * 1e3, nbytes / sec / 1e9))
        del t, launches, keep
        torch.cuda.empty_cache()
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
            "host_cpus": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)),
            "per_config": oracle_per_config(np, synth)}


def oracle_per_config(np, synth):
    """Seconds the oracle takes on each of the five workloads at full size:
    the offline quantization (codes and scales from the fp32 weights) and the
    product (integer sums and the fp64 reference output) timed apart; input
    generation excluded.  Beside each, the parity of the HIP path on the same
    inputs against those oracle outputs: codes and scales bit for bit, int32
    accumulators bit for bit where the path has them, and the fp32 output's
    normwise error against the 1e-5 tolerance."""
    import oracle
    import torch
    import quantized_gemv_amd as qg
    out = {}

    def timed(f):
        t0 = time.perf_counter()
        r = f()
        return r, round(time.perf_counter() - t0, 3)

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    def dev_bf16(bits):
        return dev(np.asarray(bits, np.uint16)).view(torch.bfloat16)

    def host(t):
        torch.cuda.synchronize()
        return t.cpu().numpy()

    def same(gpu, ref):
        return bool(np.array_equal(host(gpu), np.asarray(ref)))

    def parity(exact, y, y_ref):
        err = oracle.normwise_error(host(y), y_ref)
        exact = {k: bool(v) for k, v in exact.items()}
        return {**exact, "y_normwise_err": float("%.3g" % err), "tol": 1e-5,
                "ok": bool(all(exact.values()) and err <= 1e-5)}
    log("cpu baseline: oracle on the five workloads (and the HIP path's parity against it)")
    wl = synth.tiny_gemv()
    (wq, sw), tq = timed(lambda: oracle.quantize_absmax(wl.tensors["w"], per_row=True))
    (xq, sx), tx = timed(lambda: oracle.quantize_absmax(wl.tensors["x"], per_row=False))
    (acc, y_ref), tp = timed(lambda: (lambda a: (a, oracle.y_w8a8(a, sw, sx)))(oracle.int_dot_exact(wq, xq)))
    gq, gs = qg.quantize_absmax(dev(wl.tensors["w"]), per_row=True)
    gacc = torch.empty(256, dtype=torch.int32, device="cuda")
    gy = qg.qgemv(qg.QWeight(qg.QG_WFMT_INT8, 256, 256, gq, gs), dev(wl.tensors["x"]), act_int8=True, acc_out=gacc)
    out["tiny_w8a8_256x256"] = {"quantize_s": tq, "product_s": round(tx + tp, 3),
                                "product_note": "activation quantization + exact int32 dot + fp64 rescale",
                                "parity": parity({"codes_scales_exact": same(gq, wq) and same(gs, sw),
                                                  "acc_exact": same(gacc, acc.astype(np.int32))}, gy, y_ref)}
    for name, (n, k) in synth.DECODE_7B_SHAPES.items():
        wl = synth.decode_w8a16(n=n, k=k, seed=synth.DECODE_7B_SEEDS[name])
        (wq, sw), tq = timed(lambda: oracle.quantize_absmax(wl.tensors["w"], per_row=True))
        y_ref, tp = timed(lambda: oracle.y_w8a16(wq, sw, wl.tensors["x_bf16"]))
        gq, gs = qg.quantize_absmax(dev(wl.tensors["w"]), per_row=True)
        gy = qg.qgemv(qg.QWeight(qg.QG_WFMT_INT8, n, k, gq, gs), dev_bf16(wl.tensors["x_bf16"]), act_int8=False)
        out["decode_w8a16_" + name] = {"quantize_s": tq, "product_s": tp,
                                       "parity": parity({"codes_scales_exact": same(gq, wq) and same(gs, sw)},
                                                        gy, y_ref)}
        del gq, gy
    wl = synth.ternary_decode()
    (q, g), tq = timed(lambda: oracle.ternary_absmean(wl.tensors["w"]))

    def tern():
        xq, sx = oracle.quantize_absmax(wl.tensors["x"], per_row=False)
        acc = oracle.int_dot_exact(q, xq)
        return acc, oracle.y_ternary(acc, g, sx)
    (acc, y_ref), tp = timed(tern)
    gq, gg = qg.quantize_ternary(dev(wl.tensors["w"]))
    gacc = torch.empty(q.shape[0], dtype=torch.int32, device="cuda")
    gy = qg.qgemv(qg.QWeight(qg.QG_WFMT_TERNARY2, q.shape[0], q.shape[1], qg.pack(gq, 2), gg),
                  dev(wl.tensors["x"]), act_int8=True, acc_out=gacc)
    out["ternary_11008x4096"] = {"quantize_s": tq, "product_s": tp,
                                 "parity": parity({"codes_scales_exact": same(gq, q) and bool(host(gg)[0] == g),
                                                   "acc_exact": same(gacc, acc.astype(np.int32))}, gy, y_ref)}
    del q, gq, gy
    wl = synth.sign_residual_decode()
    (sgn, a, rq, sr), tq = timed(lambda: oracle.sign_residual_split(wl.tensors["w"]))
    y_ref, tp = timed(lambda: oracle.y_sign_residual(sgn, a, rq, sr, wl.tensors["x_bf16"]))
    n, k = sgn.shape
    gsg, ga, grq, gsr = qg.split_sign_residual(dev(wl.tensors["w"]))
    exact = {"codes_scales_exact": same(gsg, sgn) and same(ga, a) and same(grq, rq) and same(gsr, sr)}
    gy = qg.qgemv(qg.QWeight(qg.QG_WFMT_SIGN1_RES8, n, k, qg.pack(gsg, 1), ga, resid=grq, scale2=gsr),
                  dev_bf16(wl.tensors["x_bf16"]), act_int8=False)
    out["sign1_res8_28672x8192"] = {"quantize_s": tq, "product_s": tp, "parity": parity(exact, gy, y_ref)}
    del sgn, rq, wl, gsg, grq, gy
    torch.cuda.empty_cache()
    wl = synth.prefill_outlier()
    idx = wl.tensors["idx"]

    def wquant():
        wq, sw = oracle.quantize_absmax(wl.tensors["w"], per_row=True)
        return wq, sw, oracle.gather_outlier_weights(wl.tensors["w"], idx)
    (wq, sw, wo), tq = timed(wquant)

    def prefill():
        xq, sx, xo = oracle.outlier_split_quantize(wl.tensors["x_bf16"], idx)
        acc = oracle.int_gemm_exact(xq, wq)
        return acc, oracle.y_prefill(acc, sx, sw, xo, wo)
    (acc, y_ref), tp = timed(prefill)
    wdev = dev(wl.tensors["w"])
    gq, gs = qg.quantize_absmax(wdev, per_row=True)
    gwo = qg.gather_columns_bf16(wdev, idx.tolist())
    del wdev
    gacc = torch.empty(acc.shape, dtype=torch.int32, device="cuda")
    gy = qg.qgemm_w8a8_outlier(dev_bf16(wl.tensors["x_bf16"]), idx.tolist(), gq, gs, gwo, acc_out=gacc)
    out["prefill_w8a8_outlier_2048x4096x4096"] = {
        "quantize_s": tq, "product_s": tp,
        "product_note": "outlier split + per-token quantization, exact int32 GEMM (fp64 BLAS on integer values), "
                        "fp64 rescale and outlier GEMM",
        "parity": parity({"codes_scales_exact": same(gq, wq) and same(gs, sw),
                          "acc_exact": same(gacc, acc.astype(np.int32))}, gy, y_ref)}
    del gq, gwo, gacc, gy
    torch.cuda.empty_cache()
    return out


if __name__ == "__main__":
    main()
