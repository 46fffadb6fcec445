"""GPU parity on seeded random shapes, every format of the product.

The other GPU tests pin chosen shapes (tile and segment boundaries, the
workload sizes).  Here each format runs on shapes drawn from a fixed seed:
n log-uniform in [1, 20000], k a log-uniform multiple of the format's K
quantum up to its maximum, so that row counts that are not multiples of any
workgroup share meet K that is not a multiple of any item size.  Every case
keeps the full bar of the shape-specific tests (it calls the same case
functions): codes, scales and int32 sums bit-exact against the oracle, fp32
outputs within 1e-5 normwise, bf16 outputs the RNE of the fp32 result, and
canaries around every output intact.  The drawn shapes are in the test ids.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import TOL_F32, canaries_intact, check_bf16_output, dev, dev_bf16, guarded, host
from test_gpu_base3 import _tern3_case
from test_gpu_parity import _int8_weight, _sr_case, _ternary_case
from test_gpu_sep_threshold import _product_case
from test_gpu_zero_point import _zp_case

pytestmark = pytest.mark.gpu

_RNG = np.random.default_rng(20261204)


def note(msg):
    print("[case] " + msg, flush=True)
    sys.stdout.flush()


def _draw(count, quantum=128, kmax=32768, max_elems=12_000_000, nmax=20000):
    """count (n, k) pairs: n and k / quantum log-uniform, n * k capped so
    that the oracle stays within seconds."""
    out = []
    while len(out) < count:
        n = int(np.exp(_RNG.uniform(0.0, np.log(nmax))))
        k = quantum * max(1, int(np.exp(_RNG.uniform(0.0, np.log(kmax // quantum)))))
        if n * k <= max_elems:
            out.append((n, k))
    return out


W8A8_SHAPES = _draw(16)
W8A16_SHAPES = _draw(16)
TERNARY_SHAPES = _draw(16)
BASE3_SHAPES = _draw(12)
SR_SHAPES = _draw(12, max_elems=6_000_000)
ZP_SHAPES = _draw(10, max_elems=6_000_000)
Q4_SHAPES = _draw(12, quantum=256)
SEP_SHAPES = [(n, k, int(_RNG.integers(50, 101))) for n, k in _draw(10, kmax=65536, max_elems=6_000_000)]
BATCH_SHAPES = [(n, k, int(_RNG.integers(1, 17))) for n, k in _draw(16, kmax=65536, max_elems=12_000_000)]
GROUP_SHAPES = [(tuple(int(np.exp(_RNG.uniform(0.0, np.log(6000)))) for _ in range(int(_RNG.integers(2, 9)))),
                 128 * int(_RNG.integers(1, 65))) for _ in range(6)]


@pytest.fixture(scope="module")
def qg():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import quantized_gemv_amd as q
    q.lib()  # fails loudly if the HIP library is not built
    return q


@pytest.mark.parametrize("n,k", W8A8_SHAPES)
def test_random_w8a8(qg, n, k):
    note("random w8a8 %dx%d" % (n, k))
    wl = synth.tiny_gemv(n=n, k=k, seed=n + k)
    w, x = wl.tensors["w"], wl.tensors["x"]
    W, wq, s_w = _int8_weight(qg, w)
    wq_ref, sw_ref = oracle.quantize_absmax(w, per_row=True)
    assert np.array_equal(host(wq), wq_ref) and np.array_equal(host(s_w), sw_ref)
    xq_ref, sx_ref = oracle.quantize_absmax(x, per_row=False)
    acc_ref = oracle.int_dot_exact(wq_ref, xq_ref)
    acc_full, acc = guarded(n, torch.int32)
    y_full, y = guarded(n, torch.float32)
    qg.qgemv(W, dev(x), act_int8=True, y=y, acc_out=acc)
    assert np.array_equal(host(acc), acc_ref.astype(np.int32))
    assert oracle.normwise_error(host(y), oracle.y_w8a8(acc_ref, sw_ref, sx_ref)) <= TOL_F32
    assert canaries_intact(acc_full, n) and canaries_intact(y_full, n)


@pytest.mark.parametrize("n,k", W8A16_SHAPES)
def test_random_w8a16(qg, n, k):
    note("random w8a16 %dx%d" % (n, k))
    wl = synth.decode_w8a16(n=n, k=k, seed=n + 2 * k)
    w, xb = wl.tensors["w"], wl.tensors["x_bf16"]
    W, wq, s_w = _int8_weight(qg, w)
    wq_ref, sw_ref = oracle.quantize_absmax(w, per_row=True)
    assert np.array_equal(host(wq), wq_ref) and np.array_equal(host(s_w), sw_ref)
    y_ref = oracle.y_w8a16(wq_ref, sw_ref, xb)
    y_full, y = guarded(n, torch.float32)
    qg.qgemv(W, dev_bf16(xb), act_int8=False, y=y)
    yb_full, yb = guarded(n, torch.bfloat16)
    qg.qgemv(W, dev_bf16(xb), act_int8=False, y=yb)
    assert oracle.normwise_error(host(y), y_ref) <= TOL_F32
    check_bf16_output(host(yb), host(y), y_ref)
    assert canaries_intact(y_full, n) and canaries_intact(yb_full, n)


@pytest.mark.parametrize("n,k", TERNARY_SHAPES)
def test_random_ternary(qg, n, k):
    note("random ternary %dx%d" % (n, k))
    _ternary_case(qg, n, k, seed=n + 3 * k)


@pytest.mark.parametrize("n,k", BASE3_SHAPES)
def test_random_ternary_base3(qg, n, k):
    note("random ternary base-3 %dx%d" % (n, k))
    _tern3_case(qg, n, k, seed=n + 5 * k)


@pytest.mark.parametrize("n,k", SR_SHAPES)
def test_random_sign_residual(qg, n, k):
    note("random sign + residual %dx%d" % (n, k))
    _sr_case(qg, n, k, seed=n + 7 * k)


@pytest.mark.parametrize("n,k", ZP_SHAPES)
def test_random_sign_residual_zp(qg, n, k):
    note("random sign + zero-point residual %dx%d" % (n, k))
    _zp_case(qg, n, k, seed=n + 11 * k)


@pytest.mark.parametrize("n,k", Q4_SHAPES)
def test_random_q4k(qg, n, k):
    note("random q4k %dx%d" % (n, k))
    import oracle.q4 as oq4
    g = synth.rng(n + 13 * k)
    w = synth.gaussian(g, (n, k), 0.02)
    xb = synth.to_bf16_bits(synth.gaussian(g, (k,), 1.0))
    codes, meta = qg.quantize_q4k(dev(w))
    parts = oq4.quantize_q4k(w)
    plane_ref, meta_ref = oq4.pack_q4k(*parts)
    assert np.array_equal(host(codes), plane_ref) and np.array_equal(host(meta), meta_ref)
    W = qg.QWeight(qg.QG_WFMT_Q4K, n, k, codes, None, resid=meta)
    y_full, y = guarded(n, torch.float32)
    qg.qgemv(W, dev_bf16(xb), act_int8=False, y=y)
    assert oracle.normwise_error(host(y), oq4.y_q4k(*parts, xb)) <= TOL_F32
    assert canaries_intact(y_full, n)


@pytest.mark.parametrize("n,k,pb", SEP_SHAPES)
def test_random_sep_threshold(qg, n, k, pb):
    pz = pb // 2
    note("random thresholded %dx%d pb=%d pz=%d" % (n, k, pb, pz))
    _product_case(qg, n, k, pb, pz, x_bf16=bool((n + k) & 1), seed=n + 17 * k)


@pytest.mark.parametrize("n,k,m", BATCH_SHAPES)
def test_random_batch(qg, n, k, m):
    note("random batch %dx%d m=%d" % (n, k, m))
    g = synth.rng(n + 19 * k + m)
    w = synth.gaussian(g, (n, k), 0.02)
    xb = synth.to_bf16_bits(synth.gaussian(g, (m, k), 1.0))
    W, wq, s_w = _int8_weight(qg, w)
    q_ref, s_ref = oracle.quantize_absmax(w, per_row=True)
    y_ref = oracle.y_w8a16_batch(q_ref, s_ref, xb)
    for layout in ("row-major", "tiled"):
        Wl = W if layout == "row-major" else qg.tiled16(W)
        full = torch.empty(m * n + 128, dtype=torch.float32, device="cuda")
        full.view(torch.uint8).fill_(0x5A)
        y = full[64:64 + m * n].view(m, n)
        qg.qgemv_batch(Wl, dev_bf16(xb), y=y)
        assert oracle.normwise_error(host(y), y_ref) <= TOL_F32, layout
        assert canaries_intact(full, m * n), layout


@pytest.mark.parametrize("ns,k", GROUP_SHAPES)
def test_random_grouped_w8a16(qg, ns, k):
    # a grouped launch of 2..8 matrices of random heights equals its single
    # launches bit for bit, and each matrix the oracle
    note("random grouped w8a16 %s k=%d" % (ns, k))
    g = synth.rng(sum(ns) + k)
    xb = synth.to_bf16_bits(synth.gaussian(g, (k,), 1.0))
    x = dev_bf16(xb)
    Ws, refs = [], []
    for n in ns:
        w = synth.gaussian(g, (n, k), 0.02)
        W, _, _ = _int8_weight(qg, w)
        Ws.append(W)
        refs.append(oracle.quantize_absmax(w, per_row=True))
    ys = qg.qgemv_grouped(Ws, x, act_int8=False, y_dtype=torch.float32)
    for W, y, (q_ref, s_ref) in zip(Ws, ys, refs):
        y1 = qg.qgemv(W, x, act_int8=False, y_dtype=torch.float32)
        assert np.array_equal(host(y).view(np.uint32), host(y1).view(np.uint32))
        assert oracle.normwise_error(host(y), oracle.y_w8a16(q_ref, s_ref, xb)) <= TOL_F32


def _draw_gemm(count, quantum, kmax, nmax=1500, max_ops=3_000_000_000):
    out = []
    while len(out) < count:
        m = int(np.exp(_RNG.uniform(0.0, np.log(nmax))))
        n = int(np.exp(_RNG.uniform(0.0, np.log(nmax))))
        k = quantum * max(1, int(np.exp(_RNG.uniform(0.0, np.log(kmax // quantum)))))
        if m * n * k <= max_ops:
            out.append((m, k, n))
    return out


QGEMM_SHAPES = [(m, k, n, int(_RNG.integers(0, 41)) if _RNG.uniform() < 0.7 else 0)
                for m, k, n in _draw_gemm(10, 128, 8192)]
MX_SHAPES = _draw_gemm(10, 256, 8192)


@pytest.mark.parametrize("m,k,n,n_out", QGEMM_SHAPES)
def test_random_qgemm_outlier(qg, m, k, n, n_out):
    # the W8A8 prefill with outlier channels: split, int32 sums, rescale and
    # the bf16 outlier product (the fixed-shape case function)
    from test_gpu_parity import _qgemm_case
    n_out = min(n_out, k - 1)
    note("random qgemm m=%d k=%d n=%d n_out=%d" % (m, k, n, n_out))
    _qgemm_case(qg, m, k, n, n_out, seed=m + k + n)


@pytest.mark.parametrize("m,k,n", MX_SHAPES)
def test_random_gemm_mxfp4(qg, m, k, n):
    import oracle.mx as mx
    from test_gpu_mx import _guarded2 as mx_guarded, _operands
    note("random mxfp4 gemm %dx%dx%d" % (m, k, n))
    ca, ea, cb, eb = _operands(m, k, n, m * 3 + k + n)
    pa, sa = mx.pack_mxfp4(ca, ea)
    pb, sb = mx.pack_mxfp4(cb, eb)
    full, y = mx_guarded(m, n)
    qg.gemm_mxfp4(dev(pa), dev(sa), dev(pb), dev(sb), y=y)
    assert oracle.normwise_error(host(y), mx.gemm_mxfp4(ca, ea, cb, eb)) <= TOL_F32
    assert canaries_intact(full, m * n)


# ------------------------------------------------------------ quantizers and packing
def _draw_rc(count, quantum=8, cmax=262144, rmax=5000, max_elems=8_000_000):
    out = []
    while len(out) < count:
        r = int(np.exp(_RNG.uniform(0.0, np.log(rmax))))
        c = quantum * max(1, int(np.exp(_RNG.uniform(0.0, np.log(cmax // quantum)))))
        if r * c <= max_elems:
            out.append((r, c))
    return out


ABSMAX_SHAPES = [(r, c, bool(_RNG.integers(0, 2))) for r, c in _draw_rc(12)]
TENSOR_SIZES = [8 * int(np.exp(_RNG.uniform(0.0, np.log(1_000_000)))) for _ in range(8)]
ASYM_SHAPES = [(r, c, bool(_RNG.integers(0, 2))) for r, c in _draw_rc(8)]
TERNQ_SHAPES = _draw_rc(8, quantum=4, cmax=65536)
PACK_SHAPES = [(int(_RNG.integers(1, 3)), r, c) for r, c in _draw_rc(8, cmax=65536)]
MXQ_SHAPES = [(r, c, bool(_RNG.integers(0, 2))) for r, c in _draw_rc(8, quantum=256)]
DETECT_SHAPES = [(r, c, int(_RNG.integers(0, min(c, 256) + 1))) for r, c in _draw_rc(8, rmax=3000, max_elems=4_000_000)]


def _maybe_bf16(x, bf16):
    if bf16:
        bits = synth.to_bf16_bits(x)
        return synth.bf16_bits_to_f32(bits), dev_bf16(bits)
    return x, dev(x)


@pytest.mark.parametrize("rows,cols,bf16", ABSMAX_SHAPES)
def test_random_absmax_per_row(qg, rows, cols, bf16):
    note("random absmax per row %dx%d bf16=%s" % (rows, cols, bf16))
    x, xd = _maybe_bf16(synth.gaussian(synth.rng(rows + cols), (rows, cols), 0.02), bf16)
    q, s = qg.quantize_absmax(xd, per_row=True)
    q_ref, s_ref = oracle.quantize_absmax(x, per_row=True)
    assert np.array_equal(host(s), s_ref) and np.array_equal(host(q), q_ref)


@pytest.mark.parametrize("n", TENSOR_SIZES)
def test_random_absmax_per_tensor(qg, n):
    note("random absmax per tensor n=%d" % n)
    x = synth.gaussian(synth.rng(n), (n,), 1.0)
    q, s = qg.quantize_absmax(dev(x), per_row=False)
    q_ref, s_ref = oracle.quantize_absmax(x, per_row=False)
    assert host(s)[0] == s_ref[0] and np.array_equal(host(q), q_ref)


@pytest.mark.parametrize("rows,cols,bf16", ASYM_SHAPES)
def test_random_asym(qg, rows, cols, bf16):
    note("random asym %dx%d bf16=%s" % (rows, cols, bf16))
    x0 = (synth.gaussian(synth.rng(rows * 3 + cols), (rows, cols), 1.0) + np.float32(0.4)).astype(np.float32)
    x, xd = _maybe_bf16(x0, bf16)
    q, s, z = qg.quantize_asym(xd)
    q_ref, s_ref, z_ref = oracle.quantize_asym(x)
    assert np.array_equal(host(s), s_ref)
    assert np.array_equal(host(z).astype(np.int32), z_ref)
    assert np.array_equal(host(q), q_ref)


@pytest.mark.parametrize("n,k", TERNQ_SHAPES)
def test_random_ternary_quantize(qg, n, k):
    note("random ternary quantize %dx%d" % (n, k))
    w = synth.laplace(synth.rng(n + k), (n, k), 0.02)
    q, gamma = qg.quantize_ternary(dev(w))
    q_ref, g_ref = oracle.ternary_absmean(w)
    assert host(gamma)[0] == g_ref and np.array_equal(host(q), q_ref)


@pytest.mark.parametrize("bits,n,k", PACK_SHAPES)
def test_random_pack(qg, bits, n, k):
    note("random pack bits=%d %dx%d" % (bits, n, k))
    g = synth.rng(bits + n + k)
    if bits == 2:
        c = (g.integers(0, 3, size=(n, k)) - 1).astype(np.int8)
    else:
        c = np.where(g.random((n, k)) < 0.5, -1, 1).astype(np.int8)
    p = qg.pack(dev(c), bits)
    assert np.array_equal(host(p), oracle.pack(c, bits))
    assert np.array_equal(host(qg.unpack(p, bits, k)), c)


@pytest.mark.parametrize("rows,cols,bf16", MXQ_SHAPES)
def test_random_mxfp4_quantize(qg, rows, cols, bf16):
    import oracle.mx as mx
    note("random mxfp4 quantize %dx%d bf16=%s" % (rows, cols, bf16))
    x, xd = _maybe_bf16(synth.gaussian(synth.rng(rows + 5 * cols), (rows, cols), 1.0), bf16)
    codes, scales = qg.quantize_mxfp4(xd)
    p_ref, s_ref = mx.pack_mxfp4(*mx.quantize_mxfp4(x))
    assert np.array_equal(host(scales), s_ref) and np.array_equal(host(codes), p_ref)


@pytest.mark.parametrize("m,k,n_out", DETECT_SHAPES)
def test_random_detect_outliers(qg, m, k, n_out):
    note("random detect outliers m=%d k=%d n_out=%d" % (m, k, n_out))
    xb = synth.to_bf16_bits(synth.gaussian(synth.rng(m + k + n_out), (m, k), 1.0))
    idx = qg.detect_outliers(dev_bf16(xb), n_out)
    assert np.array_equal(host(idx), oracle.detect_outlier_channels(xb, n_out))


# ------------------------------------------------ K split with a workspace; thresholded split
SPLITK_SHAPES = [(int(np.exp(_RNG.uniform(0.0, np.log(4096)))), 128 * int(_RNG.integers(64, 129)),
                  int(_RNG.integers(2, 17))) for _ in range(8)]
SEP_SPLIT_SHAPES = [(n, k, int(_RNG.integers(50, 101))) for n, k in _draw(6, kmax=65536, max_elems=4_000_000)]


@pytest.mark.parametrize("n,k,m", SPLITK_SHAPES)
def test_random_batch_splitk(qg, n, k, m):
    # qg_qgemv_batch_ws (K split over workgroups through the caller's
    # workspace) on random row counts and 8192 <= K <= 16384; twice, since
    # the row-block counters must come back to zero
    note("random batch split-K %dx%d m=%d" % (n, k, m))
    g = synth.rng(n + 23 * k + m)
    w = synth.gaussian(g, (n, k), 0.02)
    xb = synth.to_bf16_bits(synth.gaussian(g, (m, k), 1.0))
    W, _, _ = _int8_weight(qg, w)
    q_ref, s_ref = oracle.quantize_absmax(w, per_row=True)
    y_ref = oracle.y_w8a16_batch(q_ref, s_ref, xb)
    need = qg.batch_workspace_bytes(n, k, m)
    ws = torch.zeros(max(need, 16), dtype=torch.uint8, device="cuda")
    xd = dev_bf16(xb)
    y1 = host(qg.qgemv_batch(W, xd, y_dtype=torch.float32, ws=ws))
    y2 = host(qg.qgemv_batch(W, xd, y_dtype=torch.float32, ws=ws))
    assert oracle.normwise_error(y1, y_ref) <= TOL_F32
    assert np.array_equal(y1, y2)


@pytest.mark.parametrize("n,k,pb", SEP_SPLIT_SHAPES)
def test_random_sep_split(qg, n, k, pb):
    # the thresholded split on the GPU: classes, residual stream (with its
    # zero tail), alpha and s_r against the oracle on every row
    from test_gpu_sep_threshold import _check_split, _weights
    note("random thresholded split %dx%d pb=%d" % (n, k, pb))
    _check_split(qg, _weights(n, k, n + 29 * k), pb, pb // 2)
