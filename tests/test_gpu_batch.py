"""GPU parity of the small-batch weight-only product (qg_qgemv_batch,
qg_qgemv_batch_grouped) against the oracle's fp64 reference computed from
the oracle's own int8 codes.

fp32 outputs: within 1e-5 normwise (the products are exact; only the fp32
summation order differs).  bf16 outputs: the kernel's fp32 result within
2e-3 and its bf16 output exactly RNE of that result (gpu_util)."""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import TOL_F32, canaries_intact, check_bf16_output, dev, dev_bf16, host

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


def _case(n, k, m, seed):
    g = synth.rng(seed)
    w = synth.gaussian(g, (n, k), 0.02)
    synth.boost_entries(g, w, 0.001, 10.0)
    if n > 3:
        w[3] = 0.0  # all-zero row: s_w = 1, codes 0
    x = synth.gaussian(g, (m, k), 1.0)
    if m > 2:
        x[1] = 0.0  # an all-zero token
    return w, synth.to_bf16_bits(x)


def _weight(qg, w):
    wq, s_w = qg.quantize_absmax(dev(w), per_row=True)
    return qg.QWeight(qg.QG_WFMT_INT8, w.shape[0], w.shape[1], wq, s_w), wq, s_w


def _guarded2(m, n, dtype, guard=64):
    full = torch.empty(m * n + 2 * guard, dtype=dtype, device="cuda")
    full.view(torch.uint8).fill_(0x5A)
    return full, full[guard:guard + m * n].view(m, n)


@pytest.mark.parametrize("n,k,m", [(16, 128, 1), (7, 256, 16), (40, 1152, 2), (300, 4096, 5), (4096, 4096, 16),
                                   (11008, 4096, 8), (4096, 11008, 3), (33, 32768, 16), (1000, 128, 9),
                                   (2000, 2176, 4),
                                   # more 16-row tiles than CUs, K <= 4608: activations kept in LDS
                                   # (ragged units per wave; the largest K that fits; the first that does not)
                                   (5000, 2176, 16), (4200, 4608, 7), (4200, 4736, 16),
                                   # the largest K
                                   (16, 262144, 4)])
def test_qgemv_batch(qg, n, k, m):
    note("qgemv batch %dx%d m=%d" % (n, k, m))
    w, xb = _case(n, k, m, n + 3 * k + m)
    W, wq, s_w = _weight(qg, w)
    wq_h, s_h = host(wq), host(s_w)
    q_ref, s_ref = oracle.quantize_absmax(w, per_row=True)
    assert np.array_equal(wq_h, q_ref) and np.array_equal(s_h, s_ref)
    y_ref = oracle.y_w8a16_batch(q_ref, s_ref, xb)
    full32, y32 = _guarded2(m, n, torch.float32)
    qg.qgemv_batch(W, dev_bf16(xb), y=y32)
    fullb, yb = _guarded2(m, n, torch.bfloat16)
    qg.qgemv_batch(W, dev_bf16(xb), y=yb)
    y32_h, yb_h = host(y32), host(yb)
    assert oracle.normwise_error(y32_h, y_ref) <= TOL_F32
    check_bf16_output(yb_h.ravel(), y32_h.ravel(), y_ref.ravel())
    assert canaries_intact(full32, m * n) and canaries_intact(fullb, m * n)


def test_qgemv_batch_one_token_matches_batch1(qg):
    # m = 1 runs the batch-1 kernel: bit-identical to qg_qgemv
    note("qgemv batch m=1 vs qg_qgemv")
    w, xb = _case(4096, 4096, 1, 77)
    W, _, _ = _weight(qg, w)
    y1 = qg.qgemv(W, dev_bf16(xb[0]), act_int8=False, y_dtype=torch.float32)
    yb = qg.qgemv_batch(W, dev_bf16(xb))
    assert np.array_equal(host(y1), host(yb)[0])


def test_qgemv_batch_one_token_large_k(qg):
    # m = 1 beyond the batch-1 kernel's K: the MFMA kernel
    note("qgemv batch m=1 k=65536")
    w, xb = _case(64, 65536, 1, 78)
    W, wq, s_w = _weight(qg, w)
    q_ref, s_ref = oracle.quantize_absmax(w, per_row=True)
    y = qg.qgemv_batch(W, dev_bf16(xb))
    assert oracle.normwise_error(host(y), oracle.y_w8a16_batch(q_ref, s_ref, xb)) <= TOL_F32


def test_qgemv_batch_grouped_matches_single(qg):
    note("qgemv batch grouped (3 matrices, m=8)")
    k, m = 4096, 8
    shapes = [4096, 1024, 777]
    Ws = []
    g = synth.rng(91)
    xb = synth.to_bf16_bits(synth.gaussian(g, (m, k), 1.0))
    for j, n in enumerate(shapes):
        w = synth.gaussian(synth.rng(100 + j), (n, k), 0.02)
        Ws.append(_weight(qg, w)[0])
    xd = dev_bf16(xb)
    ys = qg.qgemv_batch_grouped(Ws, xd, y_dtype=torch.bfloat16)
    for W, y in zip(Ws, ys):
        y1 = qg.qgemv_batch(W, xd, y_dtype=torch.bfloat16)
        assert np.array_equal(host(y), host(y1))


def test_qgemv_batch_grouped_qkv_16_tokens(qg):
    # the grouped launch (768 tiles) keeps the activations in LDS; each
    # single 4096-row launch (256 tiles) reads them per tile: bit-identical
    note("qgemv batch grouped 3 x 4096x4096, m=16, vs single launches and the oracle")
    k, m = 4096, 16
    g = synth.rng(92)
    xb = synth.to_bf16_bits(synth.gaussian(g, (m, k), 1.0))
    xd = dev_bf16(xb)
    Ws, refs = [], []
    for j in range(3):
        w = synth.gaussian(synth.rng(200 + j), (4096, k), 0.02)
        W, _, _ = _weight(qg, w)
        Ws.append(W)
        refs.append(w)
    ys = qg.qgemv_batch_grouped(Ws, xd, y_dtype=torch.float32)
    rows = np.unique(np.concatenate([[0, 1, 4095], synth.rng(93).choice(4096, 61, replace=False)]))
    for W, y, w in zip(Ws, ys, refs):
        y1 = qg.qgemv_batch(W, xd, y_dtype=torch.float32)
        assert np.array_equal(host(y), host(y1))
        q_ref, s_ref = oracle.quantize_absmax(np.ascontiguousarray(w[rows]), per_row=True)
        y_ref = oracle.y_w8a16_batch(q_ref, s_ref, xb)
        assert oracle.normwise_error(host(y)[:, rows], y_ref) <= TOL_F32
