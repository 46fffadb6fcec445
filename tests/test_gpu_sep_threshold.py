"""GPU parity of the thresholded separated format against the oracle.

The split is compared byte for byte (classes, the residual stream with its
zero tail, alpha and s_r); the product is run on the oracle's own packed
bytes, its int32 accumulators compared exactly and its fp32 output within
1e-5 normwise of the oracle's fp64 value ([SEP] sections 2.1, 3.3, 5.2 and
5.3)."""
import sys

import numpy as np
import pytest
import torch

import oracle
import oracle.threshold as th
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


def _weights(n, k, seed, special=True):
    g = synth.rng(seed)
    w = synth.laplace(g, (n, k), 0.015)
    synth.boost_entries(g, w, 0.005, 20.0)
    if special and n >= 4:
        w[1] = 0.0                                   # all zero
        w[2] = np.float32(0.03)                      # one magnitude everywhere
        w[3, ::3] = -w[3, ::3]
        w[3, : k // 2] = np.round(w[3, : k // 2] * 200) / 200  # many ties
    return w


def _check_split(qg, w, pb, pz):
    """GPU split against the oracle on every row: scales, class plane and
    residual stream."""
    n, k = w.shape
    sw = qg.split_sep_threshold(dev(w), pb, pz)
    assert sw.ld == th.resid_ld(k, pz) or (sw.ld == 16 and th.resid_ld(k, pz) < 16)
    f, a, rq, sr = th.threshold_split(w, pb, pz)
    plane, stream = th.pack_threshold(f, rq, sw.ld)
    assert np.array_equal(host(sw.alpha), a)
    assert np.array_equal(host(sw.s_r), sr)
    assert np.array_equal(host(sw.cls), plane)
    assert np.array_equal(host(sw.rv), stream)
    return sw, (f, a, rq, sr)


@pytest.mark.parametrize("n,k,pb,pz", [(1, 128, 80, 50), (7, 1152, 80, 50), (33, 4096, 70, 40), (6, 8192, 90, 0),
                                       (5, 1024, 60, 60), (4, 2048, 100, 0), (5, 640 * 2, 80, 1), (3, 65536, 80, 50)])
def test_split_sep_threshold(qg, n, k, pb, pz):
    note("split thresholded %dx%d pb=%d pz=%d" % (n, k, pb, pz))
    _check_split(qg, _weights(n, k, n * 7 + k), pb, pz)


def test_split_sep_threshold_full(qg):
    note("split thresholded 28672x8192 (every row)")
    wl = synth.sign_residual_decode()
    _check_split(qg, wl.tensors["w"], 80, 50)


def _product_case(qg, n, k, pb, pz, x_bf16, skip=False, seed=0, zero_x=False):
    w = _weights(n, k, seed + n + k)
    g = synth.rng(seed + 99)
    x = synth.gaussian(g, (k,), 1.0)
    if zero_x:
        x[:] = 0
    if x_bf16:
        xb = synth.to_bf16_bits(x)
        x = synth.bf16_bits_to_f32(xb)
        xd = dev_bf16(xb)
    else:
        xd = dev(x)
    f, a, rq, sr = th.threshold_split(w, pb, pz)
    ld = th.resid_ld(k, pz)
    ld = max(ld, 16)
    plane, stream = th.pack_threshold(f, rq, ld)
    sw = qg.SepWeight(dev(plane), dev(stream), dev(a), dev(sr), k)
    y_full, y = guarded(n, torch.float32)
    acc_full, acc = guarded(2 * n, torch.int32)
    qg.qgemv_sep(sw, xd, skip_residual=skip, y=y, acc_out=acc)
    xq, s_x = oracle.quantize_absmax(x, per_row=False)
    acc_b, acc_r = th.int_products(f, rq, xq)
    acc_h = host(acc)
    assert np.array_equal(acc_h[:n], acc_b)
    assert np.array_equal(acc_h[n:], np.zeros(n, np.int64) if skip else acc_r)
    y_ref = th.y_threshold(acc_b, acc_r, a, sr, s_x, skip_residual=skip)
    assert oracle.normwise_error(host(y), y_ref) <= TOL_F32
    assert canaries_intact(y_full, n) and canaries_intact(acc_full, 2 * n)


@pytest.mark.parametrize("n,k", [(1, 128), (9, 1152), (77, 4096), (300, 8192), (13, 11008), (8, 65536)])
@pytest.mark.parametrize("x_bf16", [False, True])
def test_qgemv_sep(qg, n, k, x_bf16):
    note("qgemv thresholded %dx%d bf16=%s" % (n, k, x_bf16))
    _product_case(qg, n, k, 80, 50, x_bf16)


@pytest.mark.parametrize("pb,pz", [(100, 0), (60, 60), (90, 0), (70, 10)])
def test_qgemv_sep_class_mixes(qg, pb, pz):
    # all residual (every step's slice is 1024 codes), no residual, no zeros
    note("qgemv thresholded mixes pb=%d pz=%d" % (pb, pz))
    _product_case(qg, 40, 3072, pb, pz, True)


@pytest.mark.parametrize("n,k", [(9, 1152), (300, 8192)])
def test_qgemv_sep_skip_residual(qg, n, k):
    note("qgemv thresholded skip residual %dx%d" % (n, k))
    _product_case(qg, n, k, 80, 50, True, skip=True)


# more row groups per workgroup than the two per wave taken first, so the
# rest come from the workgroup's LDS counter: 24 rows per workgroup (one step
# per row; two steps and a ragged last workgroup), and 24 groups of two rows
# in the skip-residual mode
@pytest.mark.parametrize("n,k,skip", [(8800, 1152, False), (8300, 8192, False), (17000, 1152, True)])
def test_qgemv_sep_dynamic_groups(qg, n, k, skip):
    note("qgemv thresholded %dx%d skip=%s (dynamic row groups)" % (n, k, skip))
    _product_case(qg, n, k, 80, 50, True, skip=skip)


def test_qgemv_sep_zero_activations(qg):
    note("qgemv thresholded zero x")
    _product_case(qg, 16, 1024, 80, 50, False, zero_x=True)


def test_qgemv_sep_full(qg):
    # the bench workload end to end on the GPU: split, then product, with
    # every row's classes, residual stream, scales, int32 sums and y checked
    note("qgemv thresholded 28672x8192 (every row)")
    wl = synth.sign_residual_decode()
    w, xb = wl.tensors["w"], wl.tensors["x_bf16"]
    sw, (f, a, rq, sr) = _check_split(qg, w, 80, 50)
    n = w.shape[0]
    acc_full, acc = guarded(2 * n, torch.int32)
    y_full, y = guarded(n, torch.float32)
    qg.qgemv_sep(sw, dev_bf16(xb), y=y, acc_out=acc)
    x = synth.bf16_bits_to_f32(xb)
    xq, s_x = oracle.quantize_absmax(x, per_row=False)
    acc_b, acc_r = th.int_products(f, rq, xq)
    acc_h = host(acc)
    assert np.array_equal(acc_h[:n], acc_b) and np.array_equal(acc_h[n:], acc_r)
    y_ref = th.y_threshold(acc_b, acc_r, a, sr, s_x)
    assert oracle.normwise_error(host(y), y_ref) <= TOL_F32
    assert canaries_intact(y_full, n) and canaries_intact(acc_full, 2 * n)


# Several matrices on the same x in one launch (qg_qgemv_sep_grouped): every
# row is computed by the kernel code of a single launch, so each matrix's y
# and int32 sums must equal its own qg_qgemv_sep call bit for bit, and the
# oracle's ([SEP] section 3.3: projections sharing an input in one launch).
@pytest.mark.parametrize("ns,k,x_bf16,skip", [
    ((300, 64, 1000), 1152, False, False),
    ((4096, 4096, 4096), 4096, True, False),     # q, k, v shapes: row groups from the LDS counter
    ((1, 17, 33, 200, 5, 64, 9, 130), 1024, True, True),
    ((8, 3), 65536, False, False),               # x transposed in registers (K > 32768)
])
def test_qgemv_sep_grouped(qg, ns, k, x_bf16, skip):
    note("qgemv thresholded grouped %s k=%d bf16=%s skip=%s" % (ns, k, x_bf16, skip))
    g = synth.rng(4242 + k)
    x = synth.gaussian(g, (k,), 1.0)
    if x_bf16:
        xb = synth.to_bf16_bits(x)
        x = synth.bf16_bits_to_f32(xb)
        xd = dev_bf16(xb)
    else:
        xd = dev(x)
    xq, s_x = oracle.quantize_absmax(x, per_row=False)
    ld = max(th.resid_ld(k, 50), 16)
    ws, refs, ys, accs, guards = [], [], [], [], []
    for i, n in enumerate(ns):
        w = _weights(n, k, 77 * i + n, special=(i == 0))
        f, a, rq, sr = th.threshold_split(w, 80, 50)
        plane, stream = th.pack_threshold(f, rq, ld)
        ws.append(qg.SepWeight(dev(plane), dev(stream), dev(a), dev(sr), k))
        refs.append((f, a, rq, sr))
        y_full, y = guarded(n, torch.float32)
        acc_full, acc = guarded(2 * n, torch.int32)
        ys.append(y)
        accs.append(acc)
        guards.append((y_full, acc_full))
    qg.SepGroupLaunch(ws, xd, ys, skip_residual=skip, accs=accs).launch()
    for i, n in enumerate(ns):
        f, a, rq, sr = refs[i]
        acc_b, acc_r = th.int_products(f, rq, xq)
        acc_h = host(accs[i])
        assert np.array_equal(acc_h[:n], acc_b), "matrix %d" % i
        assert np.array_equal(acc_h[n:], np.zeros(n, np.int64) if skip else acc_r), "matrix %d" % i
        y_ref = th.y_threshold(acc_b, acc_r, a, sr, s_x, skip_residual=skip)
        assert oracle.normwise_error(host(ys[i]), y_ref) <= TOL_F32, "matrix %d" % i
        assert canaries_intact(guards[i][0], n) and canaries_intact(guards[i][1], 2 * n), "matrix %d" % i
        # the same matrix alone
        y1 = torch.empty(n, dtype=torch.float32, device="cuda")
        a1 = torch.empty(2 * n, dtype=torch.int32, device="cuda")
        qg.qgemv_sep(ws[i], xd, skip_residual=skip, y=y1, acc_out=a1)
        assert np.array_equal(host(y1).view(np.uint32), host(ys[i]).view(np.uint32)), "matrix %d" % i
        assert np.array_equal(host(a1), acc_h), "matrix %d" % i
