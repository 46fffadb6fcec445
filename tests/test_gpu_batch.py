"""GPU parity of the small-batch weight-only product (qg_qgemv_batch,
qg_qgemv_batch_grouped, qg_qgemv_batch_ws) against the oracle's fp64 reference computed from
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
    for W, y, w in zip(Ws, ys, refs):
        y1 = qg.qgemv_batch(W, xd, y_dtype=torch.float32)
        assert np.array_equal(host(y), host(y1))
        q_ref, s_ref = oracle.quantize_absmax(w, per_row=True)  # every row
        y_ref = oracle.y_w8a16_batch(q_ref, s_ref, xb)
        assert oracle.normwise_error(host(y), y_ref) <= TOL_F32


def _workspace(qg, n, k, m):
    need = qg.batch_workspace_bytes(n, k, m)
    return need, torch.zeros(max(need, 16), dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("n,k,m", [(4096, 11008, 16), (4096, 11008, 4), (4096, 8192, 2),
                                   # ragged rows: 49 tiles, one per row block; 250 tiles in row
                                   # blocks of 4, the last of 2 tiles, its last tile of 6 rows
                                   (777, 8192, 7), (3990, 8192, 16), (16, 8192, 3),
                                   # ragged units per wave (130 units: 33, 33, 33, 31 per split)
                                   (100, 8320, 9),
                                   # the largest K with register-resident activations: 8 units per wave
                                   (4096, 16384, 16)])
def test_qgemv_batch_splitk(qg, n, k, m):
    note("qgemv batch split-K %dx%d m=%d" % (n, k, m))
    need, ws = _workspace(qg, n, k, m)
    assert need > 0
    w, xb = _case(n, k, m, 5 * n + k + m)
    W, wq, s_w = _weight(qg, w)
    q_ref, s_ref = oracle.quantize_absmax(w, per_row=True)
    assert np.array_equal(host(wq), q_ref) and np.array_equal(host(s_w), s_ref)
    y_ref = oracle.y_w8a16_batch(q_ref, s_ref, xb)
    xd = dev_bf16(xb)
    full32, y32 = _guarded2(m, n, torch.float32)
    qg.qgemv_batch(W, xd, y=y32, ws=ws)
    fullb, yb = _guarded2(m, n, torch.bfloat16)
    qg.qgemv_batch(W, xd, y=yb, ws=ws)
    y32_h, yb_h = host(y32), host(yb)
    assert oracle.normwise_error(y32_h, y_ref) <= TOL_F32
    check_bf16_output(yb_h.ravel(), y32_h.ravel(), y_ref.ravel())
    assert canaries_intact(full32, m * n) and canaries_intact(fullb, m * n)
    # every call leaves the row-block counters at zero (they follow the
    # partial tiles: 4 splits x tiles x 64 lanes x 16 B)
    tiles = (n + 15) // 16
    assert not host(ws)[4 * tiles * 64 * 16:].any()
    # deterministic: the partials are added in split order whichever
    # workgroup finishes last
    again = qg.qgemv_batch(W, xd, y_dtype=torch.float32, ws=ws)
    assert np.array_equal(host(again), y32_h)
    # the same definition as the unsplit launch, to rounding
    y_plain = host(qg.qgemv_batch(W, xd, y_dtype=torch.float32))
    assert oracle.normwise_error(y_plain, y_ref) <= TOL_F32


def test_qgemv_batch_splitk_shapes_alternate(qg):
    # one workspace, calls of two shapes in turn (4096 x 8192 and the down
    # projection 4096 x 11008) and two token counts
    note("qgemv batch split-K alternating shapes on one workspace")
    need = max(qg.batch_workspace_bytes(4096, 8192, 16), qg.batch_workspace_bytes(4096, 11008, 16))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    cases = []
    for j, (k, m) in enumerate([(8192, 16), (11008, 16), (8192, 5), (11008, 3)]):
        w, xb = _case(4096, k, m, 300 + j)
        W, _, _ = _weight(qg, w)
        q_ref, s_ref = oracle.quantize_absmax(w, per_row=True)
        cases.append((W, dev_bf16(xb), oracle.y_w8a16_batch(q_ref, s_ref, xb)))
    for rep in range(2):
        for W, xd, y_ref in cases:
            y = qg.qgemv_batch(W, xd, y_dtype=torch.float32, ws=ws)
            assert oracle.normwise_error(host(y), y_ref) <= TOL_F32
    assert not host(ws)[4 * 256 * 64 * 16:].any()


@pytest.mark.parametrize("n,k,m", [(5000, 11008, 16), (4096, 11008, 1), (64, 32768, 8), (4096, 4096, 16)])
def test_qgemv_batch_ws_without_split(qg, n, k, m):
    # shapes with no split (more tiles than CUs, one token, k beyond the
    # register-resident fragments, k below 8192) run qg_qgemv_batch: bit-identical
    note("qgemv batch ws fallback %dx%d m=%d" % (n, k, m))
    assert qg.batch_workspace_bytes(n, k, m) == 0
    w, xb = _case(n, k, m, 400 + m)
    W, _, _ = _weight(qg, w)
    xd = dev_bf16(xb)
    ws = torch.zeros(16, dtype=torch.uint8, device="cuda")
    y1 = qg.qgemv_batch(W, xd, y_dtype=torch.float32, ws=ws)
    y0 = qg.qgemv_batch(W, xd, y_dtype=torch.float32)
    assert np.array_equal(host(y1), host(y0))


# ---------------------------------------------------------------- 16-row tiles
def _tiles16_expected(codes):
    """The tiled layout written out with numpy: tile t, unit c, lane
    L = 16 g + i holds codes[16 t + i][64 c + 16 g .. + 15]; rows past n are 0."""
    n, k = codes.shape
    T, C = (n + 15) // 16, k // 64
    pad = np.zeros((T * 16, k), np.int8)
    pad[:n] = codes
    return pad.reshape(T, 16, C, 4, 16).transpose(0, 2, 3, 1, 4).reshape(-1)


@pytest.mark.parametrize("n,k", [(16, 128), (777, 1152), (4096, 4096), (33, 32768)])
def test_pack_tiles16_layout(qg, n, k):
    note("pack tiles16 %dx%d" % (n, k))
    codes = synth.rng(n + k).integers(-127, 128, size=(n, k), dtype=np.int64).astype(np.int8)
    full, out = torch.empty(qg.lib().qg_tiles16_bytes(n, k) + 128, dtype=torch.int8, device="cuda"), None
    full.view(torch.uint8).fill_(0x5A)
    out = full[64:-64]
    qg.pack_tiles16(dev(codes), out=out)
    assert np.array_equal(host(out), _tiles16_expected(codes))
    raw = host(full).view(np.uint8)
    assert np.all(raw[:64] == 0x5A) and np.all(raw[-64:] == 0x5A)


@pytest.mark.parametrize("n,k,m,same_order", [
    # the tile loop (K beyond the LDS-resident activations, or few tiles):
    # the same kernel as the row-major codes, bit-identical results
    (300, 4096, 5, True), (33, 32768, 16, True), (4200, 4736, 16, True), (16, 128, 1, False),
    # more tiles than CUs, fewer than three per CU (or units per tile not a
    # multiple of 8): the eight waves share each tile (activations in
    # registers; the summation order of the row-major kernel, to rounding);
    # ragged last tile
    (5000, 2176, 16, False), (4200, 4608, 7, False), (9000, 2176, 3, False),
    # three or four tiles per CU, units per tile a multiple of 8: two waves
    # per tile, one half of K each (2 to 4 tiles in a workgroup; 9
    # phases at K = 4608, 2 at K = 1024); ragged last tile
    (11008, 4096, 16, False), (11008, 4096, 3, False), (12288, 4608, 9, False), (12290, 1024, 16, False),
    (16384, 4096, 1, False),
    # five or more tiles per CU: one tile per wave over all of K; ring
    # depths 2 (34 units per tile) and 4 (72, 64); ragged last tile
    (20000, 2176, 5, False), (21000, 4608, 16, False), (22016, 4096, 16, False), (20007, 4096, 2, False)])
def test_qgemv_batch_tiles16_matches_row_major(qg, n, k, m, same_order):
    note("qgemv batch tiles16 %dx%d m=%d" % (n, k, m))
    w, xb = _case(n, k, m, 7 * n + k + m)
    W, _, _ = _weight(qg, w)
    Wt = qg.tiled16(W)
    xd = dev_bf16(xb)
    q_ref, s_ref = oracle.quantize_absmax(w, per_row=True)
    y_ref = oracle.y_w8a16_batch(q_ref, s_ref, xb)
    full32, y32 = _guarded2(m, n, torch.float32)
    qg.qgemv_batch(Wt, xd, y=y32)
    fullb, yb = _guarded2(m, n, torch.bfloat16)
    qg.qgemv_batch(Wt, xd, y=yb)
    assert canaries_intact(full32, m * n) and canaries_intact(fullb, m * n)
    y32_h = host(y32)
    assert oracle.normwise_error(y32_h, y_ref) <= TOL_F32
    check_bf16_output(host(yb).ravel(), y32_h.ravel(), y_ref.ravel())
    if same_order:
        assert np.array_equal(host(qg.qgemv_batch(W, xd, y_dtype=torch.float32)), y32_h)
    # deterministic
    assert np.array_equal(host(qg.qgemv_batch(Wt, xd, y_dtype=torch.float32)), y32_h)


@pytest.mark.parametrize("n,k,m", [(4096, 11008, 16), (4096, 11008, 4), (3990, 8192, 16), (100, 8320, 9)])
def test_qgemv_batch_splitk_tiles16(qg, n, k, m):
    note("qgemv batch split-K tiles16 %dx%d m=%d" % (n, k, m))
    need, ws = _workspace(qg, n, k, m)
    w, xb = _case(n, k, m, 11 * n + k + m)
    W, _, _ = _weight(qg, w)
    Wt = qg.tiled16(W)
    xd = dev_bf16(xb)
    y0 = qg.qgemv_batch(W, xd, y_dtype=torch.float32, ws=ws)
    full, y1 = _guarded2(m, n, torch.float32)
    qg.qgemv_batch(Wt, xd, y=y1, ws=ws)
    assert canaries_intact(full, m * n)
    assert np.array_equal(host(y0), host(y1))
    tiles = (n + 15) // 16
    assert not host(ws)[4 * tiles * 64 * 16:].any()


@pytest.mark.parametrize("rows", [[4096, 1024, 777], [11008, 11008]])
def test_qgemv_batch_grouped_tiles16(qg, rows):
    note("qgemv batch grouped tiles16 %s, m=16" % rows)
    k, m = 4096, 16
    xb = synth.to_bf16_bits(synth.gaussian(synth.rng(94), (m, k), 1.0))
    xd = dev_bf16(xb)
    ws = [synth.gaussian(synth.rng(300 + j), (n, k), 0.02) for j, n in enumerate(rows)]
    Wts = [qg.tiled16(_weight(qg, w)[0]) for w in ws]
    # 368 tiles (the waves share each tile) and 1376 (a tile per wave);
    # every matrix against the oracle
    ys = qg.qgemv_batch_grouped(Wts, xd, y_dtype=torch.float32)
    for w, y in zip(ws, ys):
        q_ref, s_ref = oracle.quantize_absmax(w, per_row=True)
        assert oracle.normwise_error(host(y), oracle.y_w8a16_batch(q_ref, s_ref, xb)) <= TOL_F32


@pytest.mark.parametrize("rows,k,m", [([9000, 8000], 4224, 16), ([20000, 777], 1152, 3), ([10000, 7001], 4608, 7),
                                      ([4096, 4096, 4096], 4096, 16), ([4096, 4096, 4100], 2048, 5)])
def test_qgemv_batch_grouped_tiles16_wave_tiles(qg, rows, k, m):
    """The kernel whose waves multiply whole tiles, or halves of K of a tile,
    against activations taken in phases of 8 units.  Whole tiles (five or
    more tiles per CU): short last phases (K = 4224 and 1152: 66 and 18
    units, with 2-unit rings), the largest K it takes (4608, 9 phases),
    waves without a tile.  Halves (three or four tiles per CU): the grouped
    q, k, v launch at 16 tokens and a ragged third matrix.  Ragged last
    tiles and fewer than 16 tokens; every row of every matrix, fp32 and
    bf16 outputs, against the oracle; nothing is written past the
    outputs."""
    note("qgemv batch grouped tiles16 wave tiles %s k=%d m=%d" % (rows, k, m))
    tiles = sum((n + 15) // 16 for n in rows)
    assert -(-tiles // 256) >= 3  # three or more tiles for some workgroups on 256 CUs
    xb = synth.to_bf16_bits(synth.gaussian(synth.rng(95 + k), (m, k), 1.0))
    xd = dev_bf16(xb)
    ws = [synth.gaussian(synth.rng(400 + j + k), (n, k), 0.02) for j, n in enumerate(rows)]
    Wts = [qg.tiled16(_weight(qg, w)[0]) for w in ws]
    y32s = qg.qgemv_batch_grouped(Wts, xd, y_dtype=torch.float32)
    guarded = [_guarded2(m, n, torch.bfloat16) for n in rows]
    qg.qgemv_batch_grouped(Wts, xd, ys=[y for _, y in guarded])
    for w, y32, (full, yb), n in zip(ws, y32s, guarded, rows):
        q_ref, s_ref = oracle.quantize_absmax(w, per_row=True)
        y_ref = oracle.y_w8a16_batch(q_ref, s_ref, xb)
        y32_h = host(y32)
        assert oracle.normwise_error(y32_h, y_ref) <= TOL_F32
        check_bf16_output(host(yb).ravel(), y32_h.ravel(), y_ref.ravel())
        assert canaries_intact(full, m * n)
