"""Host-side checks of the chained decode step's plan (qg_chain_plan runs on
the host only; nothing here touches a device): the image's tables cover
every output row exactly once, in the order the kernel hands slots out, and
every argument error is reported before anything is written or launched."""
import ctypes

import numpy as np
import pytest

import quantized_gemv_amd as qg

A = 1 << 20  # 16-B aligned fake device addresses: the plan never dereferences them


def stage(shapes, dep, base, x=None, fmt=qg.QG_WFMT_INT8):
    """One stage of fake device pointers (distinct per matrix)."""
    cw = (qg.CWeight * len(shapes))()
    yp = (ctypes.c_void_p * len(shapes))()
    for i, (n, k) in enumerate(shapes):
        cw[i].fmt, cw[i].n, cw[i].k = fmt, n, k
        cw[i].codes = base + 0x100000 * i
        cw[i].scale = base + 0x100000 * i + 0x80000
        yp[i] = base + 0x100000 * i + 0xC0000
    return (cw, len(shapes), A if x is None else x, yp, dep)


def layers(n_layers, h=4096, f=11008):
    st = []
    for li in range(n_layers):
        b = A * (16 + 8 * li)
        st.append(stage([(h, h)] * 3, len(st) - 1 if li else -1, b))
        st.append(stage([(h, h)], len(st) - 1, b + A))
        st.append(stage([(f, h)] * 2, len(st) - 1, b + 2 * A))
        st.append(stage([(h, f)], len(st) - 1, b + 4 * A))
    return st


def parse(img):
    hdr = np.frombuffer(img[:64].tobytes(), dtype=np.dtype([
        ("magic", "<u4"), ("version", "<u4"), ("nstages", "<i4"), ("total", "<i4"), ("max_k", "<i4"),
        ("stride", "<i4"), ("nc", "<i4"), ("grid", "<i4"), ("stages_off", "<u8"), ("slots_off", "<u8"),
        ("timeout", "<u8"), ("bytes", "<u8")]))[0]
    sdt = np.dtype([("x", "<u8"), ("k", "<i4"), ("dep", "<i4"), ("slot0", "<i4"), ("nslots", "<i4"),
                    ("nseg", "<i4"), ("pad", "<i4")])
    tdt = np.dtype([("codes", "<u8"), ("scale", "<u8"), ("y", "<u8"), ("rows", "<i4"), ("k", "<i4"),
                    ("nseg", "<i4"), ("stage", "<i4"), ("pad", "<i4", 2)])
    so, to = int(hdr["stages_off"]), int(hdr["slots_off"])
    stages = np.frombuffer(img[so:so + sdt.itemsize * int(hdr["nstages"])].tobytes(), sdt)
    slots = np.frombuffer(img[to:to + tdt.itemsize * int(hdr["total"])].tobytes(), tdt)
    return hdr, stages, slots


def test_plan_covers_every_row_once():
    st = layers(2)
    img, status = qg.chain_plan_image(st, 256)
    assert status == 0
    hdr, stages, slots = parse(img)
    assert hdr["magic"] == 0x48434751 and hdr["nstages"] == 8 and hdr["grid"] == 256
    assert hdr["timeout"] == qg.QG_CHAIN_TIMEOUT_TICKS and hdr["max_k"] == 11008 and hdr["bytes"] == img.size
    assert hdr["stride"] % 32 == 0 and hdr["stride"] >= 8
    assert hdr["slots_off"] % 64 == 0 and hdr["slots_off"] + 48 * hdr["total"] == hdr["bytes"]
    # control words (error, ticket, exit count, completion counters) start at zero
    assert not img[64:int(hdr["stages_off"])].any()
    slot = 0
    rows_per_slot = []
    for s, d in enumerate(stages):
        cw, count, x, yp, dep = st[s]
        assert d["dep"] == dep and d["x"] == x and d["k"] == cw[0].k
        assert d["slot0"] == slot
        assert d["nseg"] == -(-d["k"] // 4096)
        assert hdr["nc"] >= d["nseg"] * 256
        recs = slots[slot:slot + d["nslots"]]
        assert (recs["stage"] == s).all() and (recs["k"] == d["k"]).all() and (recs["nseg"] == d["nseg"]).all()
        r = int(recs["rows"].max())
        rows_per_slot.append(r)
        assert r % 8 == 0 and 8 <= r <= 128  # whole rows for each of the 8 workers
        i = 0
        for m in range(count):
            # the matrix's rows in slots of r (the last one ragged), in order
            n, k = cw[m].n, cw[m].k
            for row0 in range(0, n, r):
                t = recs[i]
                assert t["codes"] == cw[m].codes + row0 * k
                assert t["scale"] == cw[m].scale + 4 * row0
                assert t["y"] == yp[m] + 2 * row0
                assert t["rows"] == min(r, n - row0)
                i += 1
        assert i == d["nslots"]
        slot += i
    assert slot == hdr["total"]
    # about one slot per workgroup and stage at these sizes
    assert rows_per_slot[:4] == [48, 16, 88, 16]


def test_plan_bytes_query():
    l = qg.lib()
    st = layers(1)
    img, status = qg.chain_plan_image(st, 256)
    assert status == 0
    cs = (qg.CChainStage * 4)()
    for i, (cw, count, x, yp, dep) in enumerate(st):
        cs[i].count, cs[i].dep, cs[i].x = count, dep, x
        cs[i].w = ctypes.cast(cw, ctypes.POINTER(qg.CWeight))
        cs[i].y = ctypes.cast(yp, ctypes.POINTER(ctypes.c_void_p))
    assert l.qg_chain_plan_bytes(cs, 4, 256) == img.size
    assert l.qg_chain_plan_bytes(cs, 0, 256) == 0
    assert l.qg_chain_plan_bytes(cs, 4, 0) == 0
    assert l.qg_chain_plan_bytes(None, 4, 256) == 0
    cs[1].dep = 1                                               # invalid stages: 0 bytes
    assert l.qg_chain_plan_bytes(cs, 4, 256) == 0


@pytest.mark.parametrize("case,expect", [
    ("count0", 4), ("count9", 4), ("dep_self", 4), ("dep_below", 4), ("fmt", 4),
    ("k_small", 2), ("k_big", 2), ("k_ragged", 2), ("k_mismatch", 2), ("n0", 2),
    ("null_codes", 1), ("null_scale", 1), ("null_y", 1), ("null_x", 1),
    ("codes_misaligned", 3), ("x_misaligned", 3), ("y_odd", 3),
])
def test_plan_validation(case, expect):
    st = layers(1)
    cw, count, x, yp, dep = st[1]
    if case == "count0":
        st[1] = (cw, 0, x, yp, dep)
    elif case == "count9":
        st[1] = (cw, 9, x, yp, dep)
    elif case == "dep_self":
        st[1] = (cw, count, x, yp, 1)
    elif case == "dep_below":
        st[1] = (cw, count, x, yp, -2)
    elif case == "fmt":
        cw[0].fmt = qg.QG_WFMT_TERNARY2
    elif case == "k_small":
        st[1] = stage([(64, 64)], 0, 16 * A)
    elif case == "k_big":
        st[1] = stage([(64, qg.QG_CHAIN_MAX_K + 128)], 0, 16 * A)
    elif case == "k_ragged":
        st[1] = stage([(64, 4160)], 0, 16 * A)
    elif case == "k_mismatch":
        st[1] = stage([(64, 4096), (64, 4224)], 0, 16 * A)
    elif case == "n0":
        cw[0].n = 0
    elif case == "null_codes":
        cw[0].codes = None
    elif case == "null_scale":
        cw[0].scale = None
    elif case == "null_y":
        yp[0] = None
    elif case == "null_x":
        st[1] = (cw, count, None, yp, dep)
    elif case == "codes_misaligned":
        cw[0].codes = cw[0].codes + 8
    elif case == "x_misaligned":
        st[1] = (cw, count, A + 8, yp, dep)
    elif case == "y_odd":
        yp[0] = yp[0] + 1
    img, status = qg.chain_plan_image(st, 256)
    assert status == expect


def test_plan_argument_errors():
    st = layers(1)
    img, status = qg.chain_plan_image(st, 0)
    assert status == 4                                               # workgroups
    img, status = qg.chain_plan_image(st, 65536)
    assert status == 4
    l = qg.lib()
    cs = (qg.CChainStage * 1)()
    buf = np.zeros(4096 + 16, np.uint8)
    p = buf.ctypes.data + (-buf.ctypes.data) % 16
    assert l.qg_chain_plan(None, 1, 256, ctypes.c_void_p(p), 4096) == 1
    assert l.qg_chain_plan(cs, 0, 256, ctypes.c_void_p(p), 4096) == 4
    assert l.qg_chain_plan(cs, 1, 256, None, 4096) == 1
    # an image too small for the stages, or misaligned
    cw, count, x, yp, dep = stage([(64, 128)], -1, 16 * A)
    cs[0].count, cs[0].dep, cs[0].x = count, dep, x
    cs[0].w = ctypes.cast(cw, ctypes.POINTER(qg.CWeight))
    cs[0].y = ctypes.cast(yp, ctypes.POINTER(ctypes.c_void_p))
    need = l.qg_chain_plan_bytes(cs, 1, 256)
    assert 0 < need <= 4096
    assert l.qg_chain_plan(cs, 1, 256, ctypes.c_void_p(p + 8), 4096) == 3
    assert l.qg_chain_plan(cs, 1, 256, ctypes.c_void_p(p), need - 1) == 5
    assert l.qg_chain_plan(cs, 1, 256, ctypes.c_void_p(p), need) == 0


def test_chain_call_rejects_bad_images_before_launch():
    l = qg.lib()
    img, status = qg.chain_plan_image(layers(1), 256)
    assert status == 0
    bad = img.copy()
    ip = ctypes.c_void_p(img.ctypes.data)
    assert l.qg_qgemv_chain(None, ctypes.c_void_p(A), None) == 1
    assert l.qg_qgemv_chain(ip, None, None) == 1
    assert l.qg_qgemv_chain(ip, ctypes.c_void_p(A + 8), None) == 3
    raw = np.zeros(bad.size + 16, np.uint8)
    b = raw[(-raw.ctypes.data) % 16:][:bad.size]
    b[:] = bad
    b[0] ^= 1  # not an image that qg_chain_plan wrote
    assert l.qg_qgemv_chain(ctypes.c_void_p(b.ctypes.data), ctypes.c_void_p(A), None) == 4
