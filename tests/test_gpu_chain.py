"""GPU parity of the chained decode step (qg_chain_plan / qg_qgemv_chain).

Every stage's outputs are compared, element by element, with the oracle's
W8A16 product evaluated on the x that the stage read: the output of its
dependency as the GPU wrote it (read back after the call).  A stage that
read its x before the producer had finished writing it would disagree with
that oracle.  Page: "1-bit quantization is not magic", section 3.1 (decode
reads every weight once per token) and 3.3 (launch overhead)."""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemv_amd as qg
from gpu_util import bf16_to_f64, dev, host

pytestmark = pytest.mark.gpu

TOL = 1e-5  # on the fp32 sum before the bf16 rounding (fp32 path)


def check_stage(y_bits, y_ref):
    """bf16 output against the fp64 oracle: within half a bf16 ulp of the
    reference plus TOL * max|reference| (the fp32 accumulation)."""
    y_ref = np.asarray(y_ref, np.float64)
    yb = bf16_to_f64(y_bits)
    den = np.max(np.abs(y_ref))
    half_ulp = np.ldexp(1.0, np.frexp(np.abs(y_ref))[1] - 9)
    bad = np.abs(yb - y_ref) > half_ulp * (1 + 1e-6) + TOL * den
    assert not bad.any(), "rows %s differ: %s vs %s" % (np.nonzero(bad)[0][:8], yb[bad][:4], y_ref[bad][:4])


def make_weight(g, n, k):
    codes = g.integers(-127, 128, size=(n, k), dtype=np.int8)
    s_w = (127.0 / g.uniform(0.01, 0.2, size=n)).astype(np.float32)
    return codes, s_w


def build(spec, seed):
    """spec: list of (shapes [(n, k)], dep, x_from) where x_from is None (an
    input vector) or the stage whose first output x is.  Returns the ChainStep
    and the host copies needed by the oracle."""
    g = np.random.default_rng(seed)
    stages, host_w, ys_all, xs = [], [], [], []
    for si, (shapes, dep, x_from) in enumerate(spec):
        k = shapes[0][1]
        if x_from is None:
            xb = oracle.f32_to_bf16_bits(g.standard_normal(k).astype(np.float32))
            x = dev(xb).view(torch.bfloat16)
        else:
            x = ys_all[x_from][0]
            assert x.numel() == k
        ws, hw, ys = [], [], []
        for n, kk in shapes:
            assert kk == k
            codes, s_w = make_weight(g, n, k)
            ws.append(qg.QWeight(qg.QG_WFMT_INT8, n, k, dev(codes), dev(s_w)))
            hw.append((codes, s_w))
            ys.append(torch.full((n,), float("nan"), dtype=torch.bfloat16, device="cuda"))
        stages.append((ws, x, ys, dep))
        host_w.append(hw)
        ys_all.append(ys)
        xs.append(x)
    return qg.ChainStep(stages), host_w, ys_all, xs


def check_all(host_w, ys_all, xs):
    for s, hw in enumerate(host_w):
        xb = host(xs[s])
        for m, (codes, s_w) in enumerate(hw):
            check_stage(host(ys_all[s][m]), oracle.y_w8a16(codes, s_w, xb))


def layer_spec(layers, h=4096, f=11008):
    """The linear layers of a 4096-hidden / 11008-FFN decoder: per layer
    (q, k, v), o, (gate, up), down; each stage reads the first output of the
    one before it (o reads q, gate/up read o, down reads gate, the next
    layer's q, k, v read down)."""
    spec = []
    for li in range(layers):
        prev = len(spec) - 1
        spec.append(([(h, h)] * 3, prev if li else -1, prev if li else None))
        spec.append(([(h, h)], len(spec) - 1, len(spec) - 1))
        spec.append(([(f, h)] * 2, len(spec) - 1, len(spec) - 1))
        spec.append(([(h, f)], len(spec) - 1, len(spec) - 1))
    return spec


def test_chain_decode_layers_every_row():
    step, host_w, ys_all, xs = build(layer_spec(2), seed=101)
    step.launch()
    torch.cuda.synchronize()
    assert step.error() == 0
    check_all(host_w, ys_all, xs)
    first = [host(y).copy() for ys in ys_all for y in ys]
    # the call left its control words reset: a second call gives the same bits
    step.launch()
    torch.cuda.synchronize()
    assert step.error() == 0
    again = [host(y) for ys in ys_all for y in ys]
    for a, b in zip(first, again):
        assert np.array_equal(a, b)


def test_chain_ragged_shapes_and_dependencies():
    # ragged rows (slots cut short), 1-4 item segments per row, groups of up
    # to 8 matrices, a dependency that skips stages and an independent stage
    spec = [
        ([(1024, 384), (7, 384), (1, 384)], -1, None),  # 0: input x
        ([(8320, 1024), (33, 1024)], 0, 0),               # 1: k = 1024
        ([(4224, 8320)], 1, 1),                           # 2: k = 8320 (3 segments, the last ragged)
        ([(16384, 4224)], 2, 2),                          # 3: k = 4224 (2 segments)
        ([(100, 16384)] * 8, 3, 3),                       # 4: k = 16384 (4 segments), 8 matrices
        ([(257, 1024)], 0, 0),                            # 5: reads stage 0 again
        ([(640, 128)], -1, None),                         # 6: an independent input
        ([(256, 640)], 6, 6),                             # 7: reads stage 6
    ]
    step, host_w, ys_all, xs = build(spec, seed=102)
    step.launch()
    torch.cuda.synchronize()
    assert step.error() == 0
    check_all(host_w, ys_all, xs)


def test_chain_graph_replays():
    step, host_w, ys_all, xs = build(layer_spec(1), seed=103)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step.launch()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    ref = [host(y).copy() for ys in ys_all for y in ys]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step.launch()
    for _ in range(3):
        for ys in ys_all:
            for y in ys:
                y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert step.error() == 0
        got = [host(y) for ys in ys_all for y in ys]
        for a, b in zip(ref, got):
            assert np.array_equal(a, b)
        step.launch()  # eager work between the replays
        torch.cuda.synchronize()
    check_all(host_w, ys_all, xs)


def test_chain_time_bound_gives_up_and_recovers():
    """A time bound of zero ticks makes every wait that is not already
    satisfied give up: the call must end normally with the error word set;
    after the plan is restored, the next call is correct."""
    step, host_w, ys_all, xs = build(layer_spec(1), seed=104)
    normal = step.image.copy()
    step.image[48:56] = np.frombuffer(np.uint64(0).tobytes(), np.uint8)  # Header.timeout_ticks
    step.restore()
    step.launch()
    torch.cuda.synchronize()
    assert step.error() != 0
    step.image[:] = normal
    step.restore()
    step.launch()
    torch.cuda.synchronize()
    assert step.error() == 0
    check_all(host_w, ys_all, xs)
