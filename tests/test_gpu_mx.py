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


def _check_quantize(qg, x, xd):
    codes, scales = qg.quantize_mxfp4(xd)
    c_ref, e_ref = mx.quantize_mxfp4(x)
    p_ref, s_ref = mx.pack_mxfp4(c_ref, e_ref)
    assert np.array_equal(host(scales), s_ref)
    assert np.array_equal(host(codes), p_ref)


def _finite_bf16_bits():
    b = np.arange(65536, dtype=np.uint32)
    return b[((b >> 7) & 0xFF) != 0xFF].astype(np.uint16)  # 65280 values: no inf or NaN


def _rows_of_blocks(blocks, pad_value):
    """Blocks of 32 values -> rows of 256 (the last row padded with whole blocks)."""
    blocks = list(blocks)
    while len(blocks) % 8:
        blocks.append(np.full(32, pad_value, blocks[0].dtype))
    return np.concatenate(blocks).reshape(-1, 256)


@pytest.mark.parametrize("order", ["sorted", "shuffled"])
def test_quantize_mxfp4_every_bf16_value(qg, order):
    # every finite bf16 value (subnormals and both zeros included), in blocks
    # of neighbouring values or of random magnitudes
    note("mxfp4 quantize: all finite bf16 values, %s" % order)
    bits = _finite_bf16_bits()
    if order == "shuffled":
        bits = synth.rng(77).permutation(bits)
    bits = bits.reshape(255, 256)
    _check_quantize(qg, synth.bf16_bits_to_f32(bits), dev_bf16(bits))


# block exponents from the lowest (-127, the clamp) to the highest a finite
# value reaches (125 = floor(log2 max bf16) - 2)
_EXPONENTS = [-127, -126, -125, -124, -110, -60, -3, 0, 1, 7, 64, 120, 124, 125]


def test_quantize_mxfp4_bf16_against_each_block_exponent(qg):
    # blocks led by M = 7.75 * 2^e, so the block exponent is e and the other
    # 31 values, every bf16 value of magnitude up to M and at least 2^(e - 4),
    # land on every E2M1 code, tie and the saturated range
    note("mxfp4 quantize: bf16 values against block exponents")
    allb = _finite_bf16_bits()
    allv = synth.bf16_bits_to_f32(allb).astype(np.float64)
    blocks = []
    for e in _EXPONENTS:
        lead = synth.to_bf16_bits(np.array([7.75 * 2.0 ** e], np.float32))[0]
        assert synth.bf16_bits_to_f32(np.array([lead]))[0] == 7.75 * 2.0 ** e
        a = np.abs(allv)
        vals = allb[(a <= 7.75 * 2.0 ** e) & ((a >= 2.0 ** (e - 4)) | (a == 0))]
        vals = synth.rng(e + 500).permutation(vals)
        for i in range(0, len(vals), 31):
            chunk = vals[i:i + 31]
            blk = np.zeros(32, np.uint16)
            blk[0] = lead ^ (0x8000 if (i // 31) % 2 else 0)  # the lead value's sign alternates
            blk[1:1 + len(chunk)] = chunk
            blocks.append(blk)
    bits = _rows_of_blocks(blocks, 0)
    _check_quantize(qg, synth.bf16_bits_to_f32(bits), dev_bf16(bits))


def test_quantize_mxfp4_f32_ties_neighbours_and_subnormals(qg):
    # fp32 inputs: each block exponent e with the E2M1 midpoints (ties) and
    # their neighbours one ulp either side, the grid values, random values in
    # the binades around, and fp32 subnormals where e is at the bottom
    note("mxfp4 quantize: fp32 ties, neighbours, subnormals")
    g = synth.rng(123)
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0], np.float32)
    grid = np.array(mx.E2M1, np.float32)
    blocks = []
    for e in _EXPONENTS:
        scale = np.float32(2.0 ** e) if e > -127 else np.float32(2.0 ** -126) / np.float32(2.0)
        lead = np.float32(7.75) * scale
        assert float(lead) == 7.75 * 2.0 ** e
        t = ties * scale
        near = np.concatenate([t, np.nextafter(t, np.float32(0)), np.nextafter(t, np.float32(np.inf)),
                               grid * scale])
        rnd = (g.uniform(1.0, 2.0, 400) * 2.0 ** g.integers(e - 4, e + 3, 400)).astype(np.float32)
        rnd = rnd[np.abs(rnd) <= lead]
        vals = np.concatenate([near, rnd])
        vals = vals * np.where(g.random(len(vals)) < 0.5, -1, 1).astype(np.float32)
        vals = vals[np.isfinite(vals)]
        for i in range(0, len(vals), 31):
            blk = np.zeros(32, np.float32)
            blk[0] = lead
            blk[1:1 + len(vals[i:i + 31])] = vals[i:i + 31]
            blocks.append(blk)
    sub = np.arange(1, 1 + 31 * 64, dtype=np.uint32).view(np.float32)  # the smallest fp32 subnormals
    for i in range(0, len(sub), 31):
        blk = np.zeros(32, np.float32)
        blk[1:] = sub[i:i + 31] * np.float32(-1 if i % 2 else 1)
        blocks.append(blk)
    x = _rows_of_blocks(blocks, np.float32(0))
    assert np.all(np.isfinite(x))
    _check_quantize(qg, x, dev(x))


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
    # every row of Y against the fp64 reference
    note("mxfp4 prefill 2048x4096x4096 (every row)")
    wl = synth.prefill_outlier()
    xb, w = wl.tensors["x_bf16"], wl.tensors["w"]
    m, k = xb.shape
    n = w.shape[0]
    wc, ws = qg.quantize_mxfp4(dev(w))
    cw, ew = mx.quantize_mxfp4(w)
    pw, sw = mx.pack_mxfp4(cw, ew)
    assert np.array_equal(host(wc), pw) and np.array_equal(host(ws), sw)
    y = qg.prefill_mxfp4(dev_bf16(xb), wc, ws)
    cx, ex = mx.quantize_mxfp4(synth.bf16_bits_to_f32(xb))
    y_ref = mx.gemm_mxfp4(cx, ex, cw, ew)
    assert oracle.normwise_error(host(y), y_ref) <= TOL_F32  # a max-norm: one wrong row fails it
