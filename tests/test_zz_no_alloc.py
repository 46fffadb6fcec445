"""The no-allocation per-tensor quantizer against the workspace entry point.

qg_quantize_absmax_noalloc keeps its partial maxima in a file-scope device
array shared by every call on the device; it must give, bit for bit, what
qg_quantize_absmax gives with a caller workspace, also on a second call with
a smaller input (whose fewer partials must not be mixed with the first
call's) and with a smaller range (a stale partial would raise the max)."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import dev, dev_bf16, host

pytestmark = pytest.mark.gpu


def note(msg):
    print("[case] " + msg, flush=True)
    sys.stdout.flush()


def _noalloc(qg, x, rows, cols, per_row):
    q = torch.empty((rows, cols), dtype=torch.int8, device=x.device)
    s = torch.empty(rows if per_row else 1, dtype=torch.float32, device=x.device)
    xt = qg.QG_BF16 if x.dtype == torch.bfloat16 else qg.QG_F32
    gran = qg.QG_PER_ROW if per_row else qg.QG_PER_TENSOR
    st = qg.lib().qg_quantize_absmax_noalloc(ctypes.c_void_p(x.data_ptr()), xt, rows, cols, gran,
                                             ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(s.data_ptr()),
                                             ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, qg.status_str(st)
    return q, s


@pytest.mark.parametrize("bf16", [False, True])
def test_noalloc_matches_workspace_entry_point(bf16):
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import quantized_gemv_amd as qg
    qg.lib()
    # first a large tensor with a wide range, then a smaller one with a
    # narrow range: 1024 partial maxima, then 3
    for rows, cols, sigma, seed in ((1024, 4096, 100.0, 1), (3, 2048, 1.0, 2)):
        note("noalloc per-tensor %dx%d bf16=%s" % (rows, cols, bf16))
        x = synth.gaussian(synth.rng(seed), (rows, cols), sigma)
        if bf16:
            bits = synth.to_bf16_bits(x)
            xd = dev_bf16(bits)
            x = synth.bf16_bits_to_f32(bits)
        else:
            xd = dev(x)
        q_ws, s_ws = qg.quantize_absmax(xd, per_row=False)
        q_na, s_na = _noalloc(qg, xd, rows, cols, per_row=False)
        assert host(s_na)[0] == host(s_ws)[0]
        assert np.array_equal(host(q_na), host(q_ws))
        q_ref, s_ref = oracle.quantize_absmax(x, per_row=False)
        assert host(s_na)[0] == s_ref[0] and np.array_equal(host(q_na), q_ref)


def test_noalloc_per_row():
    import quantized_gemv_amd as qg
    note("noalloc per-row 33x1024")
    x = synth.gaussian(synth.rng(3), (33, 1024), 0.02)
    q_ws, s_ws = qg.quantize_absmax(dev(x), per_row=True)
    q_na, s_na = _noalloc(qg, dev(x), 33, 1024, per_row=True)
    assert np.array_equal(host(s_na), host(s_ws)) and np.array_equal(host(q_na), host(q_ws))
