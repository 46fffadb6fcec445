"""QG_DEBUG=1: the outlier-path calls run their device-side checks (the
index list as the kernels received it, the gathered outlier values, zero
codes at the outlier columns, zero padding), wait for the stream and report
a failed check as QG_ERR_DEVICE_CHECK.  On correct kernels the checks must
pass silently and change nothing: every output is bit-identical to the same
call without QG_DEBUG, and matches the oracle.  Page: "1-bit quantization is
not magic", section 2.2 (the outlier channels kept apart)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import TOL_F32, dev, dev_bf16, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qg():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import quantized_gemv_amd as q
    q.lib()
    return q


def _run(qg, w, xb, idx):
    wq, s_w = qg.quantize_absmax(dev(w), per_row=True)
    w_out = qg.gather_columns_bf16(dev(w), idx)
    xq, sx, xo = qg.quantize_absmax_split(dev_bf16(xb), idx)
    acc = torch.empty((xb.shape[0], w.shape[0]), dtype=torch.int32, device="cuda")
    y = qg.qgemm_w8a8_outlier(dev_bf16(xb), idx, wq, s_w, w_out, acc_out=acc)
    return [host(t) for t in (w_out, xq, sx, xo, acc, y)]


@pytest.mark.parametrize("m,k,n,n_out", [(64, 512, 256, 5), (300, 4096, 512, 20), (33, 1024, 128, 0)])
def test_debug_checks_pass_and_change_nothing(qg, monkeypatch, m, k, n, n_out):
    print("[case] QG_DEBUG outlier path m=%d k=%d n=%d n_out=%d" % (m, k, n, n_out), flush=True)
    wl = synth.prefill_outlier(m=m, k=k, n=n, n_out=n_out, seed=9)
    w, xb, idx = wl.tensors["w"], wl.tensors["x_bf16"], wl.tensors["idx"].tolist()
    monkeypatch.delenv("QG_DEBUG", raising=False)
    plain = _run(qg, w, xb, idx)
    monkeypatch.setenv("QG_DEBUG", "1")
    checked = _run(qg, w, xb, idx)  # raises on any status but QG_OK
    monkeypatch.delenv("QG_DEBUG")
    for a, b in zip(plain, checked):
        assert np.array_equal(a, b)
    # and the checked call against the oracle
    w_out, xq, sx, xo, acc, y = checked
    xq_ref, sx_ref, xo_ref = oracle.outlier_split_quantize(xb, np.asarray(idx, np.int64))
    assert np.array_equal(xq, xq_ref) and np.array_equal(sx, sx_ref)
    wq_ref, sw_ref = oracle.quantize_absmax(w, per_row=True)
    acc_ref = oracle.int_gemm_exact(xq_ref, wq_ref)
    assert np.array_equal(acc, acc_ref.astype(np.int32))
    wo_ref = oracle.gather_outlier_weights(w, np.asarray(idx, np.int64))
    y_ref = oracle.y_prefill(acc_ref, sx_ref, sw_ref, xo_ref, wo_ref)
    assert oracle.normwise_error(y, y_ref) <= TOL_F32


def test_debug_self_test_reports_and_clears(qg, monkeypatch):
    """QG_DEBUG=2 makes the checks expect every gathered value with its
    lowest bit flipped: a correct call with outliers must come back with
    QG_ERR_DEVICE_CHECK (the failure is reported, not swallowed), and the
    flag it left is cleared, so the next checked call passes."""
    print("[case] QG_DEBUG self-test", flush=True)
    wl = synth.prefill_outlier(m=40, k=256, n=64, n_out=6, seed=11)
    w, xb, idx = wl.tensors["w"], wl.tensors["x_bf16"], wl.tensors["idx"].tolist()
    monkeypatch.setenv("QG_DEBUG", "2")
    with pytest.raises(qg.QgError) as e1:
        qg.quantize_absmax_split(dev_bf16(xb), idx)
    assert e1.value.status == qg.QG_ERR_DEVICE_CHECK
    with pytest.raises(qg.QgError) as e2:
        qg.gather_columns_bf16(dev(w), idx)
    assert e2.value.status == qg.QG_ERR_DEVICE_CHECK
    # no outliers: nothing to flip, nothing to report
    qg.quantize_absmax_split(dev_bf16(xb), [])
    monkeypatch.setenv("QG_DEBUG", "1")
    xq, sx, xo = qg.quantize_absmax_split(dev_bf16(xb), idx)
    monkeypatch.delenv("QG_DEBUG")
    xq_ref, sx_ref, xo_ref = oracle.outlier_split_quantize(xb, np.asarray(idx, np.int64))
    assert np.array_equal(host(xq), xq_ref) and np.array_equal(host(sx), sx_ref)
    assert np.array_equal(host(xo)[:, :len(idx)], xo_ref)
