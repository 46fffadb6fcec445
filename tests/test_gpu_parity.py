"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Bar: bit-exact on quantized codes, scales, packed bytes and int32
accumulators; float outputs within the normwise tolerances of gpu_util
(1e-5 on fp32-activation paths, 2e-3 on bf16-activation paths) against the
oracle's fp64 reference computed from the oracle's own codes.

Sizes: small shapes spanning several workgroups with ragged tails, the five
workloads at full size with every row checked, and edge cases (minimum /
maximum K, single rows, zero inputs).
"""
import sys

import ctypes

import numpy as np
import pytest
import torch

import oracle
import oracle.q4 as oq4
import synth
from gpu_util import (TOL_BF16, TOL_F32, bf16_to_f64, canaries_intact, check_bf16_output, dev, dev_bf16, guarded,
                      host)

pytestmark = pytest.mark.gpu


def note(msg):
    print("[case] " + msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def qg():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import quantized_gemv_amd as q
    q.lib()  # fails loudly if the HIP library is not built
    return q


# ------------------------------------------------------------------ quantizers

@pytest.mark.parametrize("rows,cols", [(1, 8), (7, 264), (33, 4096), (4, 11008)])
@pytest.mark.parametrize("bf16_in", [False, True])
def test_absmax_per_row(qg, rows, cols, bf16_in):
    note("absmax per_row %dx%d bf16=%s" % (rows, cols, bf16_in))
    g = synth.rng(rows * 1000 + cols)
    w = synth.gaussian(g, (rows, cols), 0.02)
    if rows > 2:
        w[2] = 0.0
    if bf16_in:
        bits = synth.to_bf16_bits(w)
        xin = dev_bf16(bits)
        w = synth.bf16_bits_to_f32(bits)
    else:
        xin = dev(w)
    q, s = qg.quantize_absmax(xin, per_row=True)
    q_ref, s_ref = oracle.quantize_absmax(w, per_row=True)
    assert np.array_equal(host(s), s_ref)
    assert np.array_equal(host(q), q_ref)


@pytest.mark.parametrize("n", [8, 256, 4096, 65536 + 8, 3 * 1024 * 1024])
def test_absmax_per_tensor(qg, n):
    note("absmax per_tensor n=%d" % n)
    g = synth.rng(n)
    x = synth.gaussian(g, (n,), 1.0)
    q, s = qg.quantize_absmax(dev(x), per_row=False)
    q_ref, s_ref = oracle.quantize_absmax(x, per_row=False)
    assert host(s)[0] == s_ref[0]
    assert np.array_equal(host(q), q_ref)


def test_absmax_tiny_groups(qg):
    # groups whose 127 / max|x| overflows fp32 (max|x| ~ 1e-37): the scale is
    # clamped to FLT_MAX on both sides, zeros stay 0
    note("absmax tiny groups")
    g = synth.rng(37)
    w = synth.gaussian(g, (6, 4096), 0.02)
    w[1] = w[1] * np.float32(1e-36)
    w[3] = w[3] * np.float32(2e-37)
    w[3, ::7] = 0.0
    q, s = qg.quantize_absmax(dev(w), per_row=True)
    q_ref, s_ref = oracle.quantize_absmax(w, per_row=True)
    assert s_ref[1] == np.finfo(np.float32).max and s_ref[3] == np.finfo(np.float32).max
    assert np.array_equal(host(s), s_ref) and np.array_equal(host(q), q_ref)
    x = np.ascontiguousarray(w[3])
    qt, st = qg.quantize_absmax(dev(x), per_row=False)
    qt_ref, st_ref = oracle.quantize_absmax(x, per_row=False)
    assert host(st)[0] == st_ref[0] and np.array_equal(host(qt), qt_ref)
    # the W8A8 product quantizes such an x inside the kernel: same codes, so
    # the int32 sums match exactly
    wq, s_w = qg.quantize_absmax(dev(w), per_row=True)
    W = qg.QWeight(qg.QG_WFMT_INT8, 6, 4096, wq, s_w)
    acc = torch.empty(6, dtype=torch.int32, device="cuda")
    qg.qgemv(W, dev(x), act_int8=True, acc_out=acc)
    assert np.array_equal(host(acc), oracle.int_dot_exact(q_ref, qt_ref).astype(np.int32))


def test_probe_stream_read_runs(qg):
    # the measurement aid: launches, returns, and leaves the sink untouched
    # (it is written only on an XOR value that ones never produce)
    note("probe stream read")
    import ctypes
    buf = torch.ones(4 << 20, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(8, dtype=torch.int32, device="cuda")
    st = qg.lib().qg_probe_stream_read(ctypes.c_void_p(buf.data_ptr()), buf.numel(), 8,
                                       ctypes.c_void_p(sink.data_ptr()),
                                       ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    assert not host(sink).any()


def test_absmax_worked_example_on_gpu(qg):
    note("absmax worked example")
    x = np.array([10.8, 3.08, 3.02, -7.59, 0, 0, 0, 0], np.float32)
    q, s = qg.quantize_absmax(dev(x), per_row=False)
    assert host(q).tolist()[:4] == [127, 36, 36, -89]
    assert host(s)[0] == np.float32(127) / np.float32(10.8)


@pytest.mark.parametrize("m,k,n_out", [(5, 64, 3), (64, 512, 6), (2048, 4096, 20), (3, 4096, 0), (2, 64, 64),
                                       (3, 40, 2),        # row length not a multiple of 32 columns
                                       (9, 6152, 7),      # four 16-byte pieces per thread
                                       (2, 16392, 5),     # row longer than the register window: two passes
                                       (65537, 8, 1)])    # more rows than workgroups: grid-stride rows
def test_outlier_split(qg, m, k, n_out):
    note("outlier split m=%d k=%d n_out=%d" % (m, k, n_out))
    wl = synth.prefill_outlier(m=m, k=k, n=8, n_out=n_out, seed=5)
    xb, idx = wl.tensors["x_bf16"], wl.tensors["idx"]
    xq, s, xo = qg.quantize_absmax_split(dev_bf16(xb), idx.tolist(), ld=n_out + 5)
    xq_ref, s_ref, xo_ref = oracle.outlier_split_quantize(xb, idx)
    assert np.array_equal(host(s), s_ref)
    assert np.array_equal(host(xq), xq_ref)
    if n_out:  # x_out is not touched when there are no outliers
        xo = host(xo)
        assert np.array_equal(xo[:, :n_out], xo_ref)
        assert not xo[:, n_out:].any()  # the padding columns are zero


@pytest.mark.parametrize("m,k,n_out,kind", [(2048, 4096, 20, "planted"), (64, 256, 4, "planted"),
                                            (7, 520, 37, "ties"), (5, 64, 64, "gauss"), (300, 1024, 256, "ties"),
                                            (3, 8, 1, "gauss"), (9, 128, 5, "zero"), (5000, 64, 17, "gauss"),
                                            (2, 262144, 256, "gauss"), (4, 96, 0, "gauss")])
def test_detect_outliers(qg, m, k, n_out, kind):
    note("detect outliers m=%d k=%d n_out=%d %s" % (m, k, n_out, kind))
    if kind == "planted":
        xb = synth.prefill_outlier(m=m, k=k, n=8, n_out=n_out, seed=5).tensors["x_bf16"]
    else:
        g = synth.rng(11)
        if kind == "gauss":
            x = synth.gaussian(g, (m, k), 1.0)
        elif kind == "ties":  # few distinct magnitudes: many equal ranges
            x = g.integers(-4, 5, (m, k)).astype(np.float32)
        else:
            x = np.zeros((m, k), np.float32)
        xb = synth.to_bf16_bits(x)
    idx = qg.detect_outliers(dev_bf16(xb), n_out)
    assert np.array_equal(host(idx), oracle.detect_outlier_channels(xb, n_out))


def test_gather_columns(qg):
    note("gather outlier weights")
    wl = synth.prefill_outlier(m=4, k=4096, n=4096, n_out=20, seed=5)
    w, idx = wl.tensors["w"], wl.tensors["idx"]
    wo = host(qg.gather_columns_bf16(dev(w), idx.tolist(), ld=29))
    assert np.array_equal(wo[:, :20], oracle.gather_outlier_weights(w, idx))
    assert not wo[:, 20:].any()


@pytest.mark.parametrize("n,k", [(3, 4), (64, 256), (11008, 4096)])
def test_ternary_quantize(qg, n, k):
    note("ternary quantize %dx%d" % (n, k))
    w = synth.ternary_decode(n=n, k=k, seed=3).tensors["w"]
    q, gamma = qg.quantize_ternary(dev(w))
    q_ref, g_ref = oracle.ternary_absmean(w)
    assert host(gamma)[0] == g_ref
    assert np.array_equal(host(q), q_ref)


def test_ternary_special_values(qg):
    note("ternary special values")
    for w in (np.array([[1.9486494, 5.8459477, 0, 0]], np.float32),
              np.zeros((2, 8), np.float32),
              np.array([[0.5, 1.5, 1.0, -1.0]], np.float32)):
        q, gamma = qg.quantize_ternary(dev(w))
        q_ref, g_ref = oracle.ternary_absmean(w)
        assert host(gamma)[0] == g_ref
        assert np.array_equal(host(q), q_ref)


@pytest.mark.parametrize("n,k", [(5, 8), (37, 520), (130, 8192)])
def test_split_sign_residual_small(qg, n, k):
    note("sign/residual split %dx%d" % (n, k))
    w = synth.sign_residual_decode(n=n, k=k, seed=4).tensors["w"]
    w[0, :4] = [0.0, -0.0, 1e-30, -1e-30]
    if n > 3:
        w[3] = 0
    sign, alpha, rq, s_r = qg.split_sign_residual(dev(w))
    s_ref, a_ref, rq_ref, sr_ref = oracle.sign_residual_split(w)
    assert np.array_equal(host(alpha), a_ref)
    assert np.array_equal(host(s_r), sr_ref)
    assert np.array_equal(host(sign), s_ref)
    assert np.array_equal(host(rq), rq_ref)


# ------------------------------------------------------------------ packing

@pytest.mark.parametrize("bits", [1, 2])
@pytest.mark.parametrize("n,k", [(1, 8), (9, 264), (300, 4096)])
def test_pack_unpack(qg, bits, n, k):
    note("pack bits=%d %dx%d" % (bits, n, k))
    g = synth.rng(bits * 7 + n)
    if bits == 2:
        c = (g.integers(0, 3, size=(n, k)) - 1).astype(np.int8)
    else:
        c = np.where(g.random((n, k)) < 0.5, -1, 1).astype(np.int8)
    p = qg.pack(dev(c), bits)
    p_ref = oracle.pack(c, bits)
    assert np.array_equal(host(p), p_ref)
    assert np.array_equal(host(qg.unpack(p, bits, k)), c)


def test_pack_exhaustive_bytes(qg):
    note("pack exhaustive")
    allbytes = np.arange(256, dtype=np.uint8)[None, :].repeat(2, axis=0)
    codes = oracle.unpack(allbytes, 1, 8 * 256)
    assert np.array_equal(host(qg.pack(dev(codes), 1)), allbytes)
    tern = oracle.unpack(np.array([[b for b in range(256) if all(((b >> (2 * j)) & 3) != 3 for j in range(4))]],
                                  np.uint8), 2, 4 * 81)
    assert np.array_equal(host(qg.pack(dev(tern), 2)), oracle.pack(tern, 2))


# ------------------------------------------------------------------ qgemv

def _int8_weight(qg, w):
    wq, s_w = qg.quantize_absmax(dev(w), per_row=True)
    return qg.QWeight(qg.QG_WFMT_INT8, w.shape[0], w.shape[1], wq, s_w), wq, s_w


@pytest.mark.parametrize("n,k", [(256, 256), (1, 128), (77, 1152), (300, 4096), (129, 11008)])
def test_qgemv_w8a8(qg, n, k):
    note("qgemv w8a8 %dx%d" % (n, k))
    wl = synth.tiny_gemv(n=n, k=k, seed=1)
    w, x = wl.tensors["w"], wl.tensors["x"]
    W, wq, s_w = _int8_weight(qg, w)
    wq_ref, sw_ref = oracle.quantize_absmax(w, per_row=True)
    assert np.array_equal(host(wq), wq_ref) and np.array_equal(host(s_w), sw_ref)
    xq_ref, sx_ref = oracle.quantize_absmax(x, per_row=False)
    acc_ref = oracle.int_dot_exact(wq_ref, xq_ref)
    y_ref = oracle.y_w8a8(acc_ref, sw_ref, sx_ref)
    acc_full, acc = guarded(n, torch.int32)
    y_full, y = guarded(n, torch.float32)
    qg.qgemv(W, dev(x), act_int8=True, y=y, acc_out=acc)
    assert np.array_equal(host(acc), acc_ref.astype(np.int32))
    assert oracle.normwise_error(host(y), y_ref) <= TOL_F32
    assert canaries_intact(acc_full, n) and canaries_intact(y_full, n)


@pytest.mark.parametrize("name", list(synth.DECODE_7B_SHAPES))
def test_qgemv_w8a16_decode_shapes(qg, name):
    n, k = synth.DECODE_7B_SHAPES[name]
    note("qgemv w8a16 %s" % name)
    wl = synth.decode_w8a16(n=n, k=k, seed=synth.DECODE_7B_SEEDS[name])
    w, xb = wl.tensors["w"], wl.tensors["x_bf16"]
    W, wq, s_w = _int8_weight(qg, w)
    wq_ref, sw_ref = oracle.quantize_absmax(w, per_row=True)
    assert np.array_equal(host(s_w), sw_ref)
    assert np.array_equal(host(wq), wq_ref)
    y_ref = oracle.y_w8a16(wq_ref, sw_ref, xb)
    y_full, y = guarded(n, torch.bfloat16)
    x = dev_bf16(xb)
    qg.qgemv(W, x, act_int8=False, y=y)
    yb = host(y)
    y32 = host(qg.qgemv(W, x, act_int8=False, y_dtype=torch.float32))
    check_bf16_output(yb, y32, y_ref)
    assert canaries_intact(y_full, n)
    # the fp32 result carries only the fp32 accumulation error
    assert oracle.normwise_error(y32, y_ref) <= 1e-5
    # determinism: a second launch is bit-identical
    y2 = qg.qgemv(W, x, act_int8=False, y_dtype=torch.bfloat16)
    assert np.array_equal(host(y2), yb)


# x in registers (K <= 4096: 128, 1152, 4096; two-row items once a
# workgroup owns 256 rows or more: 66000 x 4096), x staged in LDS as fp32
# (4096 < K <= 12288: 5120, 8192, 11008, 12288; 13000 x 8192 puts 51 rows in
# each workgroup, so the two ends of each SIMD's row pool meet after a dozen
# claims), x with every item (12416, 32768); 65600 x 256: hundreds of rows
# per workgroup on a one-chunk row
@pytest.mark.parametrize("n,k", [(8, 128), (77, 1152), (11008, 4096), (66000, 4096), (77, 5120), (300, 8192),
                                 (13000, 8192), (129, 12288), (40, 12416), (33, 32768), (65600, 256)])
def test_qgemv_w8a16_small_and_edges(qg, n, k):
    note("qgemv w8a16 %dx%d" % (n, k))
    wl = synth.decode_w8a16(n=n, k=k, seed=21)
    w, xb = wl.tensors["w"], wl.tensors["x_bf16"]
    W, wq, s_w = _int8_weight(qg, w)
    wq_ref, sw_ref = oracle.quantize_absmax(w, per_row=True)
    assert np.array_equal(host(wq), wq_ref)
    y_ref = oracle.y_w8a16(wq_ref, sw_ref, xb)
    y = qg.qgemv(W, dev_bf16(xb), act_int8=False, y_dtype=torch.float32)
    assert oracle.normwise_error(host(y), y_ref) <= 1e-5
    # fp32 activations take the same path (converted exactly to fp32 on chip)
    xf = synth.bf16_bits_to_f32(xb)
    y2 = qg.qgemv(W, dev(xf), act_int8=False, y_dtype=torch.float32)
    assert np.array_equal(host(y2), host(y))


def _ternary_case(qg, n, k, seed=3, x_bf16=False):
    wl = synth.ternary_decode(n=n, k=k, seed=seed)
    w, x = wl.tensors["w"], wl.tensors["x"]
    if x_bf16:
        xb = synth.to_bf16_bits(x)
        x = synth.bf16_bits_to_f32(xb)
        xin = dev_bf16(xb)
    else:
        xin = dev(x)
    q, gamma = qg.quantize_ternary(dev(w))
    packed = qg.pack(q, 2)
    q_ref, g_ref = oracle.ternary_absmean(w)
    p_ref = oracle.pack(q_ref, 2)
    assert host(gamma)[0] == g_ref
    assert np.array_equal(host(packed), p_ref)
    W = qg.QWeight(qg.QG_WFMT_TERNARY2, n, k, packed, gamma)
    xq_ref, sx_ref = oracle.quantize_absmax(x, per_row=False)
    acc_ref = oracle.int_dot_exact(q_ref, xq_ref)
    y_ref = oracle.y_ternary(acc_ref, g_ref, sx_ref)
    acc_full, acc = guarded(n, torch.int32)
    y_full, y = guarded(n, torch.float32)
    qg.qgemv(W, xin, act_int8=True, y=y, acc_out=acc)
    assert np.array_equal(host(acc), acc_ref.astype(np.int32))
    assert oracle.normwise_error(host(y), y_ref) <= TOL_F32
    assert canaries_intact(acc_full, n) and canaries_intact(y_full, n)


# one-row items with every item in flight (300, 11008 and 4096 rows; K =
# 11008 keeps x in two 16-column groups per thread, K = 32768 quantizes the
# groups past that window in a second pass), two-row items (30000 x 4096)
# and four-row items two at a time (40000 x 1024)
@pytest.mark.parametrize("n,k", [(1, 128), (13, 384), (300, 4096), (11008, 4096), (4096, 11008), (30000, 4096),
                                 (40000, 1024), (40, 32768)])
def test_qgemv_ternary(qg, n, k):
    note("qgemv ternary %dx%d" % (n, k))
    _ternary_case(qg, n, k)


def test_qgemv_ternary_bf16_activations(qg):
    note("qgemv ternary bf16 x")
    _ternary_case(qg, 100, 1024, x_bf16=True)


def _sr_case(qg, n, k, seed=4):
    """Split, pack and fused product on the GPU; every row of alpha, s_r, the
    sign bytes, the residual codes and y against the oracle."""
    wl = synth.sign_residual_decode(n=n, k=k, seed=seed)
    w, xb = wl.tensors["w"], wl.tensors["x_bf16"]
    sign, alpha, rq, s_r = qg.split_sign_residual(dev(w))
    sp = qg.pack(sign, 1)
    W = qg.QWeight(qg.QG_WFMT_SIGN1_RES8, n, k, sp, alpha, resid=rq, scale2=s_r)
    y_full, y = guarded(n, torch.bfloat16)
    qg.qgemv(W, dev_bf16(xb), act_int8=False, y=y)
    y32 = qg.qgemv(W, dev_bf16(xb), act_int8=False, y_dtype=torch.float32)
    s_ref, a_ref, rq_ref, sr_ref = oracle.sign_residual_split(w)
    assert np.array_equal(host(alpha), a_ref)
    assert np.array_equal(host(s_r), sr_ref)
    assert np.array_equal(host(sp), oracle.pack(s_ref, 1))
    assert np.array_equal(host(rq), rq_ref)
    y_ref = oracle.y_sign_residual(s_ref, a_ref, rq_ref, sr_ref, xb)
    check_bf16_output(host(y), host(y32), y_ref)
    assert oracle.normwise_error(host(y32), y_ref) <= 1e-5
    assert canaries_intact(y_full, n)


@pytest.mark.parametrize("n,k", [(1, 128), (9, 1152), (700, 8192), (31, 32768)])
def test_qgemv_sign_residual(qg, n, k):
    note("qgemv sign+residual %dx%d" % (n, k))
    _sr_case(qg, n, k)


# Shapes where a workgroup owns more row groups than the two per wave it takes
# first, so the rest are handed out through its LDS counter: 20 rows per
# workgroup, 38 (ragged: the last workgroup has fewer), and 24 rows of four
# segments each.  Every row is checked: a group skipped or taken twice in any
# workgroup leaves canary bytes or a wrong value in y.
@pytest.mark.parametrize("n,k", [(5120, 1152), (9477, 2048), (6144, 16384)])
def test_qgemv_sign_residual_dynamic_groups(qg, n, k):
    note("qgemv sign+residual %dx%d (dynamic row groups, every row)" % (n, k))
    _sr_case(qg, n, k)


def test_qgemv_sign_residual_full(qg):
    # the 70B-style FFN shape: 112 rows per workgroup, all through the LDS
    # counter after the first two groups of each wave; every row checked
    note("qgemv sign+residual 28672x8192 (every row)")
    _sr_case(qg, 28672, 8192)


@pytest.mark.parametrize("fmt", ["int8_f", "int8_i", "ternary", "sign_res"])
def test_qgemv_grouped_matches_single(qg, fmt):
    note("qgemv grouped %s" % fmt)
    shapes = [(4096, 4096), (1024, 4096), (777, 4096)] if fmt != "sign_res" else [(300, 4096), (64, 4096)]
    g = synth.rng(77)
    Ws, refs = [], []
    for i, (n, k) in enumerate(shapes):
        w = synth.gaussian(g, (n, k), 0.02)
        if fmt.startswith("int8"):
            Wd, wq, s_w = _int8_weight(qg, w)
            Ws.append(Wd)
            refs.append(oracle.quantize_absmax(w, per_row=True))
        elif fmt == "ternary":
            q, gamma = qg.quantize_ternary(dev(w))
            Ws.append(qg.QWeight(qg.QG_WFMT_TERNARY2, n, k, qg.pack(q, 2), gamma))
            refs.append(oracle.ternary_absmean(w))
        else:
            sign, alpha, rq, s_r = qg.split_sign_residual(dev(w))
            Ws.append(qg.QWeight(qg.QG_WFMT_SIGN1_RES8, n, k, qg.pack(sign, 1), alpha, resid=rq, scale2=s_r))
            refs.append(oracle.sign_residual_split(w))
    xf = synth.gaussian(g, (4096,), 1.0)
    xb = synth.to_bf16_bits(xf)
    act_int8 = fmt in ("int8_i", "ternary")
    x = dev(xf) if act_int8 else dev_bf16(xb)
    accs = [torch.empty(W.n, dtype=torch.int32, device="cuda") for W in Ws] if act_int8 else None
    ys = qg.qgemv_grouped(Ws, x, act_int8=act_int8, y_dtype=torch.float32, accs=accs)
    for i, W in enumerate(Ws):
        acc1 = torch.empty(W.n, dtype=torch.int32, device="cuda") if act_int8 else None
        y1 = qg.qgemv(W, x, act_int8=act_int8, y_dtype=torch.float32, acc_out=acc1)
        assert np.array_equal(host(ys[i]), host(y1)), "grouped output differs from the single launch"
        if act_int8:
            assert np.array_equal(host(accs[i]), host(acc1))
            xq_r, sx_r = oracle.quantize_absmax(xf, per_row=False)
            acc_r = oracle.int_dot_exact(refs[i][0], xq_r)
            assert np.array_equal(host(accs[i]), acc_r.astype(np.int32))
        elif fmt == "int8_f":
            assert oracle.normwise_error(host(ys[i]), oracle.y_w8a16(refs[i][0], refs[i][1], xb)) <= 1e-5
        else:
            assert oracle.normwise_error(host(ys[i]), oracle.y_sign_residual(*refs[i], xb)) <= 1e-5


@pytest.mark.parametrize("k,ns", [(11008, (4096, 777, 1500)), (1152, (4096, 777, 1500)),
                                  (4096, (4096, 300, 1000, 64, 2048))])
def test_qgemv_w8a16_grouped_matches_single(qg, k, ns):
    # a grouped launch of the W8A16 product at a K whose x is staged in LDS
    # (11008) and ones whose x sits in registers (1152, 4096; five matrices
    # take the 8-slot kernel argument): bit-identical to the single launches,
    # and within tolerance of the oracle
    note("qgemv w8a16 grouped k=%d, %d matrices" % (k, len(ns)))
    g = synth.rng(k)
    Ws, refs = [], []
    for n in ns:
        w = synth.gaussian(g, (n, k), 0.02)
        W, _, _ = _int8_weight(qg, w)
        Ws.append(W)
        refs.append(oracle.quantize_absmax(w, per_row=True))
    xb = synth.to_bf16_bits(synth.gaussian(g, (k,), 1.0))
    x = dev_bf16(xb)
    ys = qg.qgemv_grouped(Ws, x, act_int8=False, y_dtype=torch.float32)
    for i, W in enumerate(Ws):
        y1 = qg.qgemv(W, x, act_int8=False, y_dtype=torch.float32)
        assert np.array_equal(host(ys[i]), host(y1)), "grouped output differs from the single launch"
        assert oracle.normwise_error(host(ys[i]), oracle.y_w8a16(refs[i][0], refs[i][1], xb)) <= 1e-5


def test_qgemv_zero_inputs(qg):
    note("qgemv zero inputs")
    n, k = 70, 1024
    w = np.zeros((n, k), np.float32)
    W, wq, s_w = _int8_weight(qg, w)
    acc = torch.empty(n, dtype=torch.int32, device="cuda")
    y = qg.qgemv(W, dev(np.zeros(k, np.float32)), act_int8=True, acc_out=acc)
    assert not host(acc).any() and not host(y).any()
    q, gamma = qg.quantize_ternary(dev(w))
    Wt = qg.QWeight(qg.QG_WFMT_TERNARY2, n, k, qg.pack(q, 2), gamma)
    y = qg.qgemv(Wt, dev(np.ones(k, np.float32)), act_int8=True, acc_out=acc)
    assert not host(acc).any() and not host(y).any()


# ------------------------------------------------------------------ prefill GEMM

def _qgemm_case(qg, m, k, n, n_out, seed=5, check_acc=True):
    wl = synth.prefill_outlier(m=m, k=k, n=n, n_out=n_out, seed=seed)
    w, xb, idx = wl.tensors["w"], wl.tensors["x_bf16"], wl.tensors["idx"]
    wq, s_w = qg.quantize_absmax(dev(w), per_row=True)
    w_out = qg.gather_columns_bf16(dev(w), idx.tolist())
    acc = torch.empty((m, n), dtype=torch.int32, device="cuda") if check_acc else None
    y = qg.qgemm_w8a8_outlier(dev_bf16(xb), idx.tolist(), wq, s_w, w_out, acc_out=acc)
    xq_ref, sx_ref, xo_ref = oracle.outlier_split_quantize(xb, idx)
    wq_ref, sw_ref = oracle.quantize_absmax(w, per_row=True)
    wo_ref = oracle.gather_outlier_weights(w, idx)
    assert np.array_equal(host(wq), wq_ref) and np.array_equal(host(s_w), sw_ref)
    acc_ref = oracle.int_gemm_exact(xq_ref, wq_ref)
    if check_acc:
        assert np.array_equal(host(acc), acc_ref.astype(np.int32))
    y_ref = oracle.y_prefill(acc_ref, sx_ref, sw_ref, xo_ref, wo_ref)
    assert oracle.normwise_error(host(y), y_ref) <= TOL_F32

    # the GEMM alone on the split activations: the same bits as the full call
    xq, sx, xo = qg.quantize_absmax_split(dev_bf16(xb), idx.tolist())
    acc2 = torch.empty_like(acc) if check_acc else None
    y2 = qg.qgemm_w8a8(xq, sx, xo, wq, s_w, w_out, n_out, acc_out=acc2)
    assert torch.equal(y2.view(torch.int32), y.view(torch.int32))
    if check_acc:
        assert torch.equal(acc2, acc)
    if n_out:
        # wider row strides whose padding holds NaN: columns >= n_out are never used
        def nan_padded(t, ld):
            out = torch.full((t.shape[0], ld), 0x7FC0, dtype=torch.int16, device="cuda").view(torch.bfloat16)
            out[:, :n_out] = t[:, :n_out]
            return out
        xo_pad = nan_padded(xo, qg.out_ld(n_out) + 16)
        wo_pad = nan_padded(w_out, qg.out_ld(n_out) + 8)
        y3 = qg.qgemm_w8a8(xq, sx, xo_pad, wq, s_w, wo_pad, n_out)
        assert torch.equal(y3.view(torch.int32), y.view(torch.int32))


@pytest.mark.parametrize("m,k,n,n_out", [(32, 128, 32, 0), (64, 256, 96, 5), (130, 384, 200, 16), (1, 128, 1, 1),
                                         (257, 1024, 129, 20)])
def test_qgemm_small(qg, m, k, n, n_out):
    note("qgemm m=%d k=%d n=%d n_out=%d" % (m, k, n, n_out))
    _qgemm_case(qg, m, k, n, n_out)


def test_qgemm_max_k(qg):
    # the largest K the GEMM accepts, with ragged m and n tiles
    note("qgemm m=33 k=133120 n=65 n_out=3")
    _qgemm_case(qg, 33, qg.QG_QGEMM_MAX_K, 65, 3)


def test_qgemm_int32_bound(qg):
    # every product 127 * (+-127) over the largest K: sums of +-2,147,092,480,
    # just inside int32, exact
    note("qgemm extreme codes at k=133120")
    m, k, n = 17, qg.QG_QGEMM_MAX_K, 33
    xq = torch.full((m, k), 127, dtype=torch.int8, device="cuda")
    wq = torch.full((n, k), 127, dtype=torch.int8, device="cuda")
    wq[1::2] = -127
    ones_m = torch.ones(m, dtype=torch.float32, device="cuda")
    ones_n = torch.ones(n, dtype=torch.float32, device="cuda")
    acc = torch.empty((m, n), dtype=torch.int32, device="cuda")
    y = qg.qgemm_w8a8(xq, ones_m, None, wq, ones_n, None, 0, acc_out=acc)
    expect = np.where(np.arange(n) % 2 == 0, 1, -1)[None, :] * np.full((m, n), k * 127 * 127, np.int64)
    assert int(np.abs(expect).max()) < 2 ** 31
    assert np.array_equal(host(acc).astype(np.int64), expect)
    assert np.array_equal(host(y).astype(np.float64), expect.astype(np.float64))


def test_qgemm_full(qg):
    note("qgemm 2048x4096x4096 n_out=20")
    _qgemm_case(qg, 2048, 4096, 4096, 20)


# ---------------------------------------------------------------- 4-bit groups, two-level scales
def _q4_weights(n, k, seed):
    w = synth.q4_decode(n=n, k=k, seed=seed).tensors["w"]
    if n >= 6:
        w[0] = 0.0                                       # all-zero row
        w[1] = 0.125                                     # constant row
        w[2] = np.abs(w[2])                              # all positive
        w[3] = -np.abs(w[3]) - 0.01                      # all negative
        w[4, 32:64] *= 40.0                              # one group with large values
    return w


@pytest.mark.parametrize("n,k", [(6, 256), (37, 512), (64, 4096), (6, 11008), (11008, 4096)])
def test_quantize_q4k(qg, n, k):
    note("quantize q4k %dx%d" % (n, k))
    w = _q4_weights(n, k, 6)
    codes, meta = qg.quantize_q4k(dev(w))
    plane_ref, meta_ref = oq4.pack_q4k(*oq4.quantize_q4k(w))
    assert np.array_equal(host(codes), plane_ref)
    assert np.array_equal(host(meta), meta_ref)


@pytest.mark.parametrize("n,k", [(6, 256), (37, 512), (11008, 4096), (77, 11008), (33, 32768)])
def test_qgemv_q4k(qg, n, k):
    note("qgemv q4k %dx%d" % (n, k))
    w = _q4_weights(n, k, 6)
    xb = synth.q4_decode(n=1, k=k, seed=7).tensors["x_bf16"]
    codes, meta = qg.quantize_q4k(dev(w))
    parts = oq4.quantize_q4k(w)
    plane_ref, meta_ref = oq4.pack_q4k(*parts)
    assert np.array_equal(host(codes), plane_ref) and np.array_equal(host(meta), meta_ref)
    y_ref = oq4.y_q4k(*parts, xb)
    W = qg.QWeight(qg.QG_WFMT_Q4K, n, k, codes, None, resid=meta)
    x = dev_bf16(xb)
    y32 = host(qg.qgemv(W, x, act_int8=False, y_dtype=torch.float32))
    assert oracle.normwise_error(y32, y_ref) <= TOL_F32
    y_full, y = guarded(n, torch.bfloat16)
    qg.qgemv(W, x, act_int8=False, y=y)
    check_bf16_output(host(y), y32, y_ref)
    assert canaries_intact(y_full, n)


def test_qgemv_q4k_grouped_matches_single(qg):
    note("qgemv q4k grouped")
    k = 4096
    xb = synth.q4_decode(n=1, k=k, seed=7).tensors["x_bf16"]
    x = dev_bf16(xb)
    Ws, singles = [], []
    for i, n in enumerate((4096, 1000, 2304)):
        codes, meta = qg.quantize_q4k(dev(_q4_weights(n, k, 20 + i)))
        W = qg.QWeight(qg.QG_WFMT_Q4K, n, k, codes, None, resid=meta)
        Ws.append(W)
        singles.append(host(qg.qgemv(W, x, act_int8=False, y_dtype=torch.bfloat16)))
    ys = qg.qgemv_grouped(Ws, x, act_int8=False, y_dtype=torch.bfloat16)
    for y, ref in zip(ys, singles):
        assert np.array_equal(host(y), ref)
