"""GPU parity of the MXFP4 format-separated prefill against the oracle.

The quantizer is compared byte for byte (codes and E8M0 scales); the GEMM is
run on the oracle's own packed operands and compared with the oracle's fp64
product within 1e-5 normwise (the products are exact; only the fp32
summation order differs); the fused prefill is checked end to end."""
import sys

import numpy as np
import pytest
import torch

import oracle
import oracle.mx as mx
import synth
from gpu_util import TOL_F32, canaries_intact, dev, dev_bf16, host

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
    r, k = x.shape
    if r >= 5 and k >= 64:
        x[1, :32] = 0.0                                     # all-zero block
        x[2, :32] = np.float32(-0.0)                        # negative zeros
        x[3, :32] = np.array(list(mx.E2M1) * 4, np.float32) * 0.25 * np.float32(3.0)  # ties after scaling
        x[3, 32:64] *= np.float32(1e30)                     # huge
        x[4, 32:64] *= np.float32(1e-30)                    # tiny
    return x


@pytest.mark.parametrize("rows,cols,bf16", [(1, 256, False), (7, 1024, False), (7, 1024, True), (256, 4096, True),
                                            (301, 768, False), (3, 262144, True)])
def test_quantize_mxfp4(qg, rows, cols, bf16):
    note("mxfp4 quantize %dx%d bf16=%s" % (rows, cols, bf16))
    g = synth.rng(rows + cols)
    x = _special_rows(synth.gaussian(g, (rows, cols), 1.0))
    if bf16:
        bits = synth.to_bf16_bits(x)
        xd = dev_bf16(bits)
        x = synth.bf16_bits_to_f32(bits)
    else:
        xd = dev(x)
    codes, scales = qg.quantize_mxfp4(xd)
    c_ref, e_ref = mx.quantize_mxfp4(x)
    p_ref, s_ref = mx.pack_mxfp4(c_ref, e_ref)
    assert np.array_equal(host(scales), s_ref)
    assert np.array_equal(host(codes), p_ref)


def _operands(m, k, n, seed):
    g = synth.rng(seed)
    a = synth.gaussian(g, (m, k), 1.0)
    b = synth.gaussian(g, (n, k), 0.02)
    ca, ea = mx.quantize_mxfp4(a)
    cb, eb = mx.quantize_mxfp4(b)
    return ca, ea, cb, eb


def _guarded2(m, n, guard=64):
    full = torch.empty(m * n + 2 * guard, dtype=torch.float32, device="cuda")
    full.view(torch.uint8).fill_(0x5A)
    return full, full[guard:guard + m * n].view(m, n)


@pytest.mark.parametrize("m,k,n", [(1, 256, 1), (33, 512, 65), (256, 1024, 128), (300, 768, 200),
                                   (257, 2304, 129), (512, 4096, 512), (3, 262144, 5)])
def test_gemm_mxfp4(qg, m, k, n):
    note("mxfp4 gemm %dx%dx%d" % (m, k, n))
    ca, ea, cb, eb = _operands(m, k, n, m * 7 + k + n)
    pa, sa = mx.pack_mxfp4(ca, ea)
    pb, sb = mx.pack_mxfp4(cb, eb)
    full, y = _guarded2(m, n)
    qg.gemm_mxfp4(dev(pa), dev(sa), dev(pb), dev(sb), y=y)
    y_ref = mx.gemm_mxfp4(ca, ea, cb, eb)
    assert oracle.normwise_error(host(y), y_ref) <= TOL_F32
    assert canaries_intact(full, m * n)


def test_prefill_mxfp4_full_shape(qg):
    # the prefill workload: X 2048x4096 bf16 with 20 channels x50, W 4096x4096;
    # rows of Y sampled for the fp64 reference
    note("mxfp4 prefill 2048x4096x4096 (sampled rows)")
    wl = synth.prefill_outlier()
    xb, w = wl.tensors["x_bf16"], wl.tensors["w"]
    m, k = xb.shape
    n = w.shape[0]
    wc, ws = qg.quantize_mxfp4(dev(w))
    cw, ew = mx.quantize_mxfp4(w)
    pw, sw = mx.pack_mxfp4(cw, ew)
    assert np.array_equal(host(wc), pw) and np.array_equal(host(ws), sw)
    y = qg.prefill_mxfp4(dev_bf16(xb), wc, ws)
    rows = np.unique(np.concatenate([[0, 1, m - 1], synth.rng(9).choice(m, 45, replace=False)]))
    cx, ex = mx.quantize_mxfp4(synth.bf16_bits_to_f32(xb[rows]))
    y_ref = mx.gemm_mxfp4(cx, ex, cw, ew)
    assert oracle.normwise_error(host(y)[rows], y_ref) <= TOL_F32
