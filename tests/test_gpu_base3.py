"""GPU parity of base-3 ternary packing (five digits per byte) and of the
qgemv on base-3 packed weights, against the oracle.

Packed bytes and int32 accumulators are compared bit for bit; the fp32
output is held to 1e-5 normwise against the oracle's fp64 product."""
import itertools
import sys

import numpy as np
import pytest
import torch

import oracle
import oracle.base3 as b3
import synth
from gpu_util import TOL_F32, canaries_intact, dev, dev_bf16, guarded, host

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


def test_pack_base3_all_tuples(qg):
    note("base-3 pack: all 243 digit tuples")
    codes = np.array(list(itertools.product((-1, 0, 1), repeat=5)), np.int8)  # 243 rows of k = 5
    packed = qg.pack_base3(dev(codes))
    assert np.array_equal(host(packed), b3.pack_base3(codes))
    assert np.array_equal(host(qg.unpack_base3(packed, 5)), codes)


@pytest.mark.parametrize("n,k", [(1, 5), (3, 80), (7, 333), (64, 4096), (5, 32768)])
def test_pack_unpack_base3(qg, n, k):
    note("base-3 pack/unpack %dx%d" % (n, k))
    codes = synth.rng(n * 31 + k).integers(-1, 2, size=(n, k)).astype(np.int8)
    packed = qg.pack_base3(dev(codes))
    assert packed.shape == (n, b3.row_bytes(k))
    assert np.array_equal(host(packed), b3.pack_base3(codes))
    assert np.array_equal(host(qg.unpack_base3(packed, k)), codes)


def _tern3_case(qg, n, k, seed=3, x_bf16=False):
    wl = synth.ternary_decode(n=n, k=k, seed=seed)
    w, x = wl.tensors["w"], wl.tensors["x"]
    if x_bf16:
        xb = synth.to_bf16_bits(x)
        x = synth.bf16_bits_to_f32(xb)
        xin = dev_bf16(xb)
    else:
        xin = dev(x)
    q, gamma = qg.quantize_ternary(dev(w))
    packed = qg.pack_base3(q)
    q_ref, g_ref = oracle.ternary_absmean(w)
    assert host(gamma)[0] == g_ref
    assert np.array_equal(host(packed), b3.pack_base3(q_ref))
    W = qg.QWeight(qg.QG_WFMT_TERNARY3, n, k, packed, gamma)
    xq_ref, sx_ref = oracle.quantize_absmax(x, per_row=False)
    acc_ref = oracle.int_dot_exact(q_ref, xq_ref)
    y_ref = oracle.y_ternary(acc_ref, g_ref, sx_ref)
    acc_full, acc = guarded(n, torch.int32)
    y_full, y = guarded(n, torch.float32)
    qg.qgemv(W, xin, act_int8=True, y=y, acc_out=acc)
    assert np.array_equal(host(acc), acc_ref.astype(np.int32))
    assert oracle.normwise_error(host(y), y_ref) <= TOL_F32
    assert canaries_intact(acc_full, n) and canaries_intact(y_full, n)


@pytest.mark.parametrize("n,k", [(1, 128), (13, 384), (300, 4096), (11008, 4096), (40, 32768), (9, 5120)])
def test_qgemv_ternary_base3(qg, n, k):
    note("qgemv base-3 ternary %dx%d" % (n, k))
    _tern3_case(qg, n, k)


def test_qgemv_ternary_base3_bf16_activations(qg):
    note("qgemv base-3 ternary 100x1024, bf16 x")
    _tern3_case(qg, 100, 1024, x_bf16=True)


def test_qgemv_base3_matches_two_bit(qg):
    # the same codes packed both ways give the same int32 sums
    note("qgemv base-3 vs 2-bit, 777x4096")
    g = synth.rng(91)
    w = synth.laplace(g, (777, 4096), 0.02)
    x = synth.gaussian(g, (4096,), 1.0)
    q, gamma = qg.quantize_ternary(dev(w))
    a2 = torch.empty(777, dtype=torch.int32, device="cuda")
    a3 = torch.empty(777, dtype=torch.int32, device="cuda")
    qg.qgemv(qg.QWeight(qg.QG_WFMT_TERNARY2, 777, 4096, qg.pack(q, 2), gamma), dev(x), act_int8=True, acc_out=a2)
    qg.qgemv(qg.QWeight(qg.QG_WFMT_TERNARY3, 777, 4096, qg.pack_base3(q), gamma), dev(x), act_int8=True, acc_out=a3)
    assert np.array_equal(host(a2), host(a3))


def test_qgemv_base3_grouped_matches_single(qg):
    note("qgemv grouped base-3 ternary")
    g = synth.rng(92)
    shapes = [(1000, 4096), (64, 4096), (333, 4096)]
    Ws = []
    for n, k in shapes:
        q, gamma = qg.quantize_ternary(dev(synth.laplace(g, (n, k), 0.02)))
        Ws.append(qg.QWeight(qg.QG_WFMT_TERNARY3, n, k, qg.pack_base3(q), gamma))
    x = dev(synth.gaussian(g, (4096,), 1.0))
    accs = [torch.empty(W.n, dtype=torch.int32, device="cuda") for W in Ws]
    ys = qg.qgemv_grouped(Ws, x, act_int8=True, y_dtype=torch.float32, accs=accs)
    for i, W in enumerate(Ws):
        acc1 = torch.empty(W.n, dtype=torch.int32, device="cuda")
        y1 = qg.qgemv(W, x, act_int8=True, y_dtype=torch.float32, acc_out=acc1)
        assert np.array_equal(host(ys[i]), host(y1)) and np.array_equal(host(accs[i]), host(acc1))
