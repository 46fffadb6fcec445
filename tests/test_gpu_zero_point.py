"""GPU parity of the asymmetric (zero-point) quantizer, the sign backbone +
zero-point residual split and its fused qgemv, against the oracle.

Codes, scales and zero-points are compared bit for bit; the qgemv's fp32
output is held to 1e-5 normwise and its bf16 output to the bf16 rule of
gpu_util, against the oracle's fp64 product of the oracle's own codes."""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import canaries_intact, check_bf16_output, dev, dev_bf16, guarded, host

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


def _special_rows(x):
    r, c = x.shape
    if r > 5 and c >= 8:
        x[1] = 0.0                                   # empty range: s = 1, z = -128
        x[2] = np.abs(x[2]) + np.float32(0.25)       # positives only: z = -128
        x[3] = -np.abs(x[3]) - np.float32(0.25)      # negatives only: z = 127
        x[4] = np.float32(0.75)                      # a constant row
        x[5, :3] = [-7.59, 10.8, 0.0]                # the range of [VG] fig. 22 ...
        x[5, 3:] = np.clip(x[5, 3:], -7.0, 10.0)     # ... kept as the row's ends
    if r > 6:
        x[6] = x[6] * np.float32(1e-37)              # 255 / range overflows: s = FLT_MAX
    return x


@pytest.mark.parametrize("rows,cols", [(1, 8), (7, 264), (33, 4096), (6, 11008)])
@pytest.mark.parametrize("bf16_in", [False, True])
def test_quantize_asym(qg, rows, cols, bf16_in):
    note("asym quantize %dx%d bf16=%s" % (rows, cols, bf16_in))
    g = synth.rng(rows * 977 + cols)
    x = _special_rows((synth.gaussian(g, (rows, cols), 1.0) + np.float32(0.3)).astype(np.float32))
    if bf16_in:
        bits = synth.to_bf16_bits(x)
        xin = dev_bf16(bits)
        x = synth.bf16_bits_to_f32(bits)
    else:
        xin = dev(x)
    q, s, z = qg.quantize_asym(xin)
    q_ref, s_ref, z_ref = oracle.quantize_asym(x)
    assert np.array_equal(host(s), s_ref)
    assert np.array_equal(host(z).astype(np.int32), z_ref)
    assert np.array_equal(host(q), q_ref)


@pytest.mark.parametrize("n,k", [(5, 8), (37, 520), (130, 8192)])
def test_split_sign_residual_zp(qg, n, k):
    note("sign + zero-point residual split %dx%d" % (n, k))
    w = synth.sign_residual_decode(n=n, k=k, seed=4).tensors["w"]
    w[0, :4] = [0.0, -0.0, 1e-30, -1e-30]
    if n > 3:
        w[3] = 0
    sign, alpha, rq, s_r, z_r = qg.split_sign_residual_zp(dev(w))
    s_ref, a_ref, rq_ref, sr_ref, zr_ref = oracle.sign_residual_split_zp(w)
    assert np.array_equal(host(alpha), a_ref)
    assert np.array_equal(host(s_r), sr_ref)
    assert np.array_equal(host(z_r).astype(np.int32), zr_ref)
    assert np.array_equal(host(sign), s_ref)
    assert np.array_equal(host(rq), rq_ref)


def _zp_weight(qg, w):
    n, k = w.shape
    sign, alpha, rq, s_r, z_r = qg.split_sign_residual_zp(dev(w))
    sp = qg.pack(sign, 1)
    return qg.QWeight(qg.QG_WFMT_SIGN1_RES8Z, n, k, sp, alpha, resid=rq, scale2=s_r, zero=z_r), (sp, alpha, rq, s_r, z_r)


def _zp_case(qg, n, k, seed=4, x_scale=1.0, x_shift=0.0):
    wl = synth.sign_residual_decode(n=n, k=k, seed=seed)
    w = wl.tensors["w"]
    xf = (synth.bf16_bits_to_f32(wl.tensors["x_bf16"]) * np.float32(x_scale) + np.float32(x_shift)).astype(np.float32)
    xb = synth.to_bf16_bits(xf)
    W, (sp, alpha, rq, s_r, z_r) = _zp_weight(qg, w)
    y_full, y = guarded(n, torch.bfloat16)
    qg.qgemv(W, dev_bf16(xb), act_int8=False, y=y)
    y32 = qg.qgemv(W, dev_bf16(xb), act_int8=False, y_dtype=torch.float32)
    s_ref, a_ref, rq_ref, sr_ref, zr_ref = oracle.sign_residual_split_zp(w)
    assert np.array_equal(host(alpha), a_ref)
    assert np.array_equal(host(s_r), sr_ref)
    assert np.array_equal(host(z_r).astype(np.int32), zr_ref)
    assert np.array_equal(host(sp), oracle.pack(s_ref, 1))
    assert np.array_equal(host(rq), rq_ref)
    y_ref = oracle.y_sign_residual_zp(s_ref, a_ref, rq_ref, sr_ref, zr_ref, xb)
    check_bf16_output(host(y), host(y32), y_ref)
    assert oracle.normwise_error(host(y32), y_ref) <= 1e-5
    assert canaries_intact(y_full, n)


@pytest.mark.parametrize("n,k", [(1, 128), (9, 1152), (700, 8192), (31, 32768)])
def test_qgemv_sign_residual_zp(qg, n, k):
    note("qgemv sign + zero-point residual %dx%d" % (n, k))
    _zp_case(qg, n, k)


# more row groups per workgroup than the two per wave taken first: the rest
# come from the workgroup's LDS counter (every row is checked)
@pytest.mark.parametrize("n,k", [(5120, 1152), (9477, 2048), (6144, 16384)])
def test_qgemv_sign_residual_zp_dynamic_groups(qg, n, k):
    note("qgemv sign + zero-point residual %dx%d (dynamic row groups, every row)" % (n, k))
    _zp_case(qg, n, k)


def test_qgemv_sign_residual_zp_shifted_activations(qg):
    # activations with a large common offset: sum_k x[k] is large, so the
    # zero-point term z * sum_k x[k] matters in every row
    note("qgemv sign + zero-point residual 300x4096, x + 3")
    _zp_case(qg, 300, 4096, seed=8, x_shift=3.0)


def test_qgemv_sign_residual_zp_full(qg):
    note("qgemv sign + zero-point residual 28672x8192 (every row)")
    _zp_case(qg, 28672, 8192)


def test_qgemv_zp_grouped_matches_single(qg):
    note("qgemv grouped sign + zero-point residual")
    g = synth.rng(78)
    shapes = [(300, 4096), (64, 4096), (1000, 4096)]
    Ws, refs = [], []
    for n, k in shapes:
        w = synth.laplace(g, (n, k), 0.015)
        W, _ = _zp_weight(qg, w)
        Ws.append(W)
        refs.append(oracle.sign_residual_split_zp(w))
    xb = synth.to_bf16_bits(synth.gaussian(g, (4096,), 1.0))
    x = dev_bf16(xb)
    ys = qg.qgemv_grouped(Ws, x, act_int8=False, y_dtype=torch.float32)
    for i, W in enumerate(Ws):
        y1 = qg.qgemv(W, x, act_int8=False, y_dtype=torch.float32)
        assert np.array_equal(host(ys[i]), host(y1)), "grouped output differs from the single launch"
        assert oracle.normwise_error(host(ys[i]), oracle.y_sign_residual_zp(*refs[i], xb)) <= 1e-5


def test_qgemv_zp_zero_activations(qg):
    note("qgemv sign + zero-point residual, x = 0")
    n, k = 70, 1024
    w = synth.gaussian(synth.rng(5), (n, k), 0.02)
    W, _ = _zp_weight(qg, w)
    x = torch.zeros(k, dtype=torch.bfloat16, device="cuda")
    y = qg.qgemv(W, x, act_int8=False, y_dtype=torch.float32)
    assert np.all(host(y) == 0.0)
