"""Host-side checks of the C-ABI library (CPU only, no GPU needed).

* libqgemv.so loads and exports every function include/qgemv.h declares;
* argument validation returns the documented status codes before anything
  touches a device (no call here reaches a kernel launch);
* the library's exact-mean arithmetic, built for the host from the same
  header, agrees with the oracle's correctly rounded mean.
"""
import ctypes
import os
import re
import struct
import subprocess

import numpy as np
import pytest
import torch

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qgemv.h")


@pytest.fixture(scope="module")
def qg():
    import quantized_gemv_amd as q
    if not os.path.exists(q.LIB_PATH):
        from quantized_gemv_amd.build import build
        build()
    return q


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qg_[a-z0-9_]+)\s*\(", src)))


def test_library_resolves_all_symbols(qg):
    # RTLD_NOW: every symbol (including kernel host stubs) must resolve at load
    ctypes.CDLL(qg.LIB_PATH, mode=os.RTLD_NOW | os.RTLD_LOCAL)


def test_header_symbols_exported(qg):
    decl = header_functions()
    assert len(decl) >= 14
    l = ctypes.CDLL(qg.LIB_PATH)
    for name in decl:
        assert hasattr(l, name), name
    assert set(decl) == set(qg.EXPORTED)
    assert qg.lib().qg_abi_version() == 20600
    for st in range(0, 8):
        assert qg.status_str(st)
    # every status of the header has its own text
    assert len({qg.status_str(st) for st in range(0, 8)}) == 8
    assert qg.status_str(qg.QG_ERR_DEVICE_CHECK) != qg.status_str(99)


A = 4096  # a 16-B aligned fake address: validation rejects before any use
U = 4097  # misaligned

# Every call below that passes A or U must be rejected by the library's
# argument checks: a call that got through would launch a kernel on a fake
# device address.  On a machine with a visible GPU that would fault the card,
# so these tests run only where no GPU is visible (device_count() does not
# initialise the runtime).
needs_no_gpu = pytest.mark.skipif(torch.cuda.device_count() > 0,
                                  reason="passes fake device addresses; runs where no GPU is visible")


@needs_no_gpu
def test_validation_quantize_absmax(qg):
    l = qg.lib()
    f = l.qg_quantize_absmax
    assert f(None, 0, 4, 64, 1, A, A, None, 0, None) == 1
    assert f(A, 7, 4, 64, 1, A, A, None, 0, None) == 4
    assert f(A, 0, 4, 64, 9, A, A, None, 0, None) == 4
    assert f(A, 0, 0, 64, 1, A, A, None, 0, None) == 2
    assert f(A, 0, 4, 60, 1, A, A, None, 0, None) == 2
    assert f(U, 0, 4, 64, 1, A, A, None, 0, None) == 3
    need = l.qg_quantize_absmax_workspace_bytes(4, 64, 0)
    assert need > 0 and l.qg_quantize_absmax_workspace_bytes(4, 64, 1) == 0
    assert f(A, 0, 4, 64, 0, A, A, None, 0, None) == 5
    assert f(A, 0, 4, 64, 0, A, A, A, need - 1, None) == 5


@needs_no_gpu
def test_validation_quantize_absmax_noalloc(qg):
    # the same checks as qg_quantize_absmax, with no workspace to check
    f = qg.lib().qg_quantize_absmax_noalloc
    assert f(None, 0, 4, 64, 1, A, A, None) == 1
    assert f(A, 0, 4, 64, 1, None, A, None) == 1
    assert f(A, 7, 4, 64, 1, A, A, None) == 4
    assert f(A, 0, 4, 64, 9, A, A, None) == 4
    assert f(A, 0, 0, 64, 1, A, A, None) == 2
    assert f(A, 0, 4, 60, 1, A, A, None) == 2
    assert f(A, 0, 1 << 20, 1 << 21, 0, A, A, None) == 2
    assert f(U, 0, 4, 64, 0, A, A, None) == 3
    assert f(A, 0, 4, 64, 0, U, A, None) == 3


def test_probe_stream_read_sizes(qg):
    # the probe reads the largest prefix that splits into equal blocks of
    # whole passes (512 threads x 16 B x 8 loads = 64 KiB) per workgroup
    f = qg.lib().qg_probe_stream_read_bytes
    assert f(256 << 16, 256) == 256 << 16
    assert f((256 << 16) + 5, 256) == 256 << 16
    assert f((256 << 16) - 1, 256) == 0
    assert f(4 << 30, 1024) == 4 << 30
    assert f(1 << 40, 1) == 0 and f(1 << 20, 0) == 0 and f(1 << 20, 70000) == 0


@needs_no_gpu
def test_validation_probe_stream_read(qg):
    f = qg.lib().qg_probe_stream_read
    assert f(None, 1 << 20, 4, A, None) == 1
    assert f(A, 1 << 20, 4, None, None) == 1
    assert f(A, 100, 4, A, None) == 2
    assert f(U, 1 << 20, 4, A, None) == 3


@needs_no_gpu
def test_validation_split_and_gather(qg):
    l = qg.lib()
    f = l.qg_quantize_absmax_split
    good = (ctypes.c_int32 * 3)(1, 5, 9)
    unsorted = (ctypes.c_int32 * 3)(5, 1, 9)
    dup = (ctypes.c_int32 * 3)(1, 1, 9)
    oob = (ctypes.c_int32 * 3)(1, 5, 64)
    neg = (ctypes.c_int32 * 3)(-1, 5, 9)
    # (x, rows, cols, idx, n_out, q, s, x_out, x_out_ld, stream)
    assert f(A, 2, 64, unsorted, 3, A, A, A, 8, None) == 4
    assert f(A, 2, 64, dup, 3, A, A, A, 8, None) == 4
    assert f(A, 2, 64, oob, 3, A, A, A, 8, None) == 4
    assert f(A, 2, 64, neg, 3, A, A, A, 8, None) == 4
    assert f(A, 2, 64, good, 3, A, A, None, 8, None) == 1
    assert f(A, 2, 64, None, 3, A, A, A, 8, None) == 1
    assert f(A, 2, 64, good, 257, A, A, A, 300, None) == 4
    assert f(A, 2, 63, good, 3, A, A, A, 8, None) == 2
    assert f(A, 2, 8 * 40000, good, 3, A, A, A, 8, None) == 2
    assert f(A, 2, 64, good, 3, A, A, A, 2, None) == 2           # stride below n_out
    assert f(A, 2, 64, good, 3, A, A, A, 65537, None) == 2       # stride above QG_MAX_OUT_LD
    assert f(U, 2, 64, good, 3, A, A, A, 8, None) == 3
    g = l.qg_gather_columns_bf16
    # (w, n, k, idx, n_out, w_out, w_out_ld, stream)
    assert g(A, 4, 64, oob, 3, A, 8, None) == 4
    assert g(A, 4, 64, good, 3, None, 8, None) == 1
    assert g(None, 4, 64, good, 3, A, 8, None) == 1
    assert g(A, 4, 64, good, 3, A, 2, None) == 2


@needs_no_gpu
def test_validation_ternary_split_pack(qg):
    l = qg.lib()
    ws = l.qg_ternary_workspace_bytes(4, 64)
    assert ws == 2048
    t = l.qg_quantize_ternary
    assert t(A, 4, 64, A, A, None, 0, None) == 5
    assert t(A, 4, 64, A, A, A, ws - 8, None) == 5
    assert t(A, 1, 3, A, A, A, ws, None) == 2
    assert t(U, 4, 64, A, A, A, ws, None) == 3
    assert t(A, 4, 64, A, A, A + 4, ws, None) == 3
    assert t(None, 4, 64, A, A, A, ws, None) == 1
    s = l.qg_split_sign_residual
    assert s(A, 4, 12, A, A, A, A, None) == 2
    assert s(A, 4, 64, A, None, A, A, None) == 1
    assert s(A, 4, 64, U, A, A, A, None) == 3
    p = l.qg_pack
    assert p(A, 4, 64, 3, A, None) == 4
    assert p(A, 4, 6, 2, A, None) == 2
    assert p(A, 4, 12, 1, A, None) == 2
    assert p(U, 4, 64, 2, A, None) == 3
    assert l.qg_unpack(A, 4, 64, 0, A, None) == 4


@needs_no_gpu
def test_validation_qgemv(qg):
    l = qg.lib()

    def call(fmt=0, n=64, k=256, amode=1, xt=1, yt=1, acc=None, codes=A, resid=A, scale=A, scale2=A, x=A, zero=A):
        w = qg.CWeight(fmt, 0, n, k, codes, resid, scale, scale2, zero)
        return l.qg_qgemv(ctypes.byref(w), amode, x, xt, A, yt, acc, None)

    assert l.qg_qgemv(None, 1, A, 1, A, 1, None, None) == 1
    assert call(codes=None) == 1
    assert call(x=None) == 1
    assert call(fmt=5) == 4
    assert call(fmt=1, amode=1) == 4          # ternary needs int8 activations
    assert call(fmt=2, amode=0) == 4          # sign+residual needs float activations
    assert call(fmt=2, xt=0) == 4             # ... in bf16
    assert call(fmt=2, resid=None) == 1
    assert call(amode=1, acc=A) == 4          # no integer accumulators in float mode
    assert call(k=200) == 2
    assert call(k=64) == 2
    assert call(k=32768 + 128) == 2
    assert call(n=0) == 2
    assert call(codes=U) == 3
    assert call(x=U) == 3
    assert call(xt=3) == 4 and call(yt=3) == 4 and call(amode=2) == 4
    # 4-bit groups: bf16 float activations, a metadata plane, k in whole super-blocks
    assert call(fmt=3, amode=0) == 4
    assert call(fmt=3, xt=0) == 4
    assert call(fmt=3, resid=None) == 1
    assert call(fmt=3, resid=U) == 3
    assert call(fmt=3, k=384) == 2
    q4 = qg.QG_WFMT_Q4K
    assert q4 == 3
    # sign + zero-point residual: as sign + residual, and the zero-points are required
    z = qg.QG_WFMT_SIGN1_RES8Z
    assert call(fmt=z, amode=0) == 4
    assert call(fmt=z, xt=0) == 4
    assert call(fmt=z, zero=None) == 1
    assert call(fmt=z, scale2=None) == 1
    assert call(fmt=z, resid=U) == 3
    # zero is required by SIGN1_RES8Z only: with a bad k the symmetric format
    # gets past the pointer checks to the shape check (no launch either way)
    assert call(fmt=2, zero=None, k=200) == 2
    assert call(fmt=z, zero=None, k=200) == 1
    # base-3 ternary: int8 activations only
    assert call(fmt=qg.QG_WFMT_TERNARY3, amode=1) == 4
    assert call(fmt=qg.QG_WFMT_TERNARY3, scale=None) == 1
    assert call(fmt=qg.QG_WFMT_TERNARY3, k=200, amode=0) == 2


@needs_no_gpu
def test_base3_row_bytes_and_validation(qg):
    l = qg.lib()
    import oracle.base3 as b3
    for k in (1, 5, 79, 80, 81, 4096, 11008, 32768):
        assert l.qg_base3_row_bytes(k) == b3.row_bytes(k)
    assert l.qg_base3_row_bytes(0) == 0
    assert l.qg_pack_base3(None, 4, 64, A, None) == 1
    assert l.qg_pack_base3(A, 0, 64, A, None) == 2
    assert l.qg_unpack_base3(A, 4, 0, A, None) == 2
    assert l.qg_unpack_base3(A, 4, 64, None, None) == 1


@needs_no_gpu
def test_validation_asym_and_zp_split(qg):
    l = qg.lib()
    q = l.qg_quantize_asym
    assert q(None, 0, 4, 64, A, A, A, None) == 1
    assert q(A, 0, 4, 64, A, A, None, None) == 1
    assert q(A, 2, 4, 64, A, A, A, None) == 4
    assert q(A, 0, 4, 12, A, A, A, None) == 2
    assert q(A, 0, 0, 64, A, A, A, None) == 2
    assert q(U, 1, 4, 64, A, A, A, None) == 3
    assert q(A, 1, 4, 64, U, A, A, None) == 3
    s = l.qg_split_sign_residual_zp
    assert s(A, 4, 12, A, A, A, A, A, None) == 2
    assert s(A, 4, 64, A, A, A, A, None, None) == 1
    assert s(A, 4, 64, U, A, A, A, A, None) == 3


@needs_no_gpu
def test_validation_quantize_q4k(qg):
    f = qg.lib().qg_quantize_q4k
    # (w, n, k, codes, meta, stream)
    assert f(None, 4, 256, A, A, None) == 1
    assert f(A, 4, 256, None, A, None) == 1
    assert f(A, 4, 256, A, None, None) == 1
    assert f(A, 0, 256, A, A, None) == 2
    assert f(A, 4, 384, A, A, None) == 2          # k not a multiple of 256
    assert f(A, 4, 128, A, A, None) == 2
    assert f(U, 4, 256, A, A, None) == 3
    assert f(A, 4, 256, A, U, None) == 3


@needs_no_gpu
def test_validation_qgemv_grouped(qg):
    l = qg.lib()
    W = qg.CWeight * 3
    ws = W(qg.CWeight(0, 0, 64, 256, A, A, A, A), qg.CWeight(0, 0, 32, 256, A, A, A, A),
           qg.CWeight(0, 0, 16, 256, A, A, A, A))
    ys = (ctypes.c_void_p * 3)(A, A, A)
    f = l.qg_qgemv_grouped
    assert f(None, 3, 1, A, 1, ys, 1, None, None) == 1
    assert f(ws, 3, 1, A, 1, None, 1, None, None) == 1
    assert f(ws, 0, 1, A, 1, ys, 1, None, None) == 4
    assert f(ws, 9, 1, A, 1, ys, 1, None, None) == 4
    ys_null = (ctypes.c_void_p * 3)(A, None, A)
    assert f(ws, 3, 1, A, 1, ys_null, 1, None, None) == 1
    mixed_k = W(qg.CWeight(0, 0, 64, 256, A, A, A, A), qg.CWeight(0, 0, 32, 384, A, A, A, A),
                qg.CWeight(0, 0, 16, 256, A, A, A, A))
    assert f(mixed_k, 3, 1, A, 1, ys, 1, None, None) == 2
    mixed_fmt = W(qg.CWeight(0, 0, 64, 256, A, A, A, A), qg.CWeight(1, 0, 32, 256, A, A, A, A),
                  qg.CWeight(0, 0, 16, 256, A, A, A, A))
    assert f(mixed_fmt, 3, 0, A, 1, ys, 1, None, None) == 4
    bad_n = W(qg.CWeight(0, 0, 64, 256, A, A, A, A), qg.CWeight(0, 0, 0, 256, A, A, A, A),
              qg.CWeight(0, 0, 16, 256, A, A, A, A))
    assert f(bad_n, 3, 1, A, 1, ys, 1, None, None) == 2
    accs = (ctypes.c_void_p * 3)(A, None, A)
    assert f(ws, 3, 1, A, 1, ys, 1, accs, None) == 4  # accumulators only in integer mode
    assert f(ws, 3, 1, U, 1, ys, 1, None, None) == 3


@needs_no_gpu
def test_validation_qgemm(qg):
    l = qg.lib()
    f = l.qg_qgemm_w8a8_outlier
    idx = (ctypes.c_int32 * 2)(3, 7)
    need = l.qg_qgemm_workspace_bytes(16, 256, 2)
    assert need >= 16 * 256 + 16 * 4 + 16 * 8 * 2  # xq, s_x, x_out [m][8]
    assert l.qg_qgemm_workspace_bytes(16, 256, 300) == 0
    assert l.qg_qgemm_workspace_bytes(0, 256, 2) == 0
    # K past the int32-exact bound is refused
    kmax = qg.QG_QGEMM_MAX_K
    assert kmax % 128 == 0 and kmax * 127 * 127 < 2 ** 31 and (kmax + 128) * 127 * 127 >= 2 ** 31
    assert l.qg_qgemm_workspace_bytes(16, kmax, 2) > 0 and l.qg_qgemm_workspace_bytes(16, kmax + 128, 2) == 0
    # (x, m, k, idx, n_out, wq, s_w, w_out, w_out_ld, n, y, acc_out, ws, ws_bytes, stream)
    assert f(A, 16, 256, idx, 2, A, A, A, 8, 32, A, None, A, need - 1, None) == 5
    assert f(A, 16, 256, idx, 2, A, A, None, 8, 32, A, None, A, need, None) == 1
    assert f(A, 16, 200, idx, 2, A, A, A, 8, 32, A, None, A, need, None) == 2
    assert f(A, 0, 256, idx, 2, A, A, A, 8, 32, A, None, A, need, None) == 2
    assert f(A, 16, kmax + 128, idx, 2, A, A, A, 8, 32, A, None, A, 1 << 40, None) == 2
    assert l.qg_qgemm_w8a8(A, A, A, 8, 16, kmax + 128, 2, A, A, A, 8, 32, A, None, None) == 2
    assert f(A, 16, 256, idx, 2, A, A, A, 2, 32, A, None, A, need, None) == 2    # w_out_ld not a multiple of 8
    assert f(A, 16, 256, idx, 2, A, A, A, 0, 32, A, None, A, need, None) == 2    # w_out_ld below n_out
    assert f(A, 16, 256, idx, 2, A, A, U, 8, 32, A, None, A, need, None) == 3    # w_out not 16-B aligned
    assert f(U, 16, 256, idx, 2, A, A, A, 8, 32, A, None, A, need, None) == 3
    bad = (ctypes.c_int32 * 2)(7, 3)
    assert f(A, 16, 256, bad, 2, A, A, A, 8, 32, A, None, A, need, None) == 4


def _run_driver(groups):
    exe = os.path.join(ROOT, "tests", "host", "_exact_mean_driver")
    src = os.path.join(ROOT, "tests", "host", "exact_mean_driver.cpp")
    if not os.path.exists(exe) or os.path.getmtime(exe) < max(os.path.getmtime(src), os.path.getmtime(
            os.path.join(ROOT, "quantized_gemv_amd", "csrc", "exact_mean.h"))):
        subprocess.run(["g++", "-O2", "-std=c++17", src, "-o", exe], check=True)
    blob = struct.pack("<Q", len(groups))
    for g in groups:
        g = np.ascontiguousarray(g, np.float32).ravel()
        blob += struct.pack("<Q", g.size) + g.tobytes()
    out = subprocess.run([exe], input=blob, capture_output=True, check=True).stdout.decode().split()
    return [np.array(int(v), np.uint32).view(np.float32) for v in out]


def test_library_exact_mean_matches_oracle():
    g = np.random.default_rng(0)
    groups = [
        g.laplace(0, 0.02, 4096).astype(np.float32),
        g.standard_normal(8192).astype(np.float32) * np.float32(1e-30),
        (g.standard_normal(777) * np.exp(g.uniform(-80, 80, 777))).astype(np.float32),
        np.array([1.9486494, 5.8459477], np.float32),
        np.array([1.0, 2.0, 2.0], np.float32),
        np.array([2.0 ** -149, 0.0, -0.0], np.float32),
        np.full(1000, np.finfo(np.float32).max, np.float32),
        np.zeros(16, np.float32),
    ]
    for _ in range(40):
        n = int(g.integers(1, 300))
        groups.append((g.standard_normal(n) * np.exp(g.uniform(-30, 30))).astype(np.float32))
    got = _run_driver(groups)
    for grp, r in zip(groups, got):
        assert r == oracle.mean_abs_f32(grp), (grp[:4], r, oracle.mean_abs_f32(grp))


@needs_no_gpu
def test_validation_qgemm_presplit(qg):
    f = qg.lib().qg_qgemm_w8a8
    # (xq, s_x, x_out, x_out_ld, m, k, n_out, wq, s_w, w_out, w_out_ld, n, y, acc_out, stream)
    assert f(None, A, A, 8, 16, 256, 2, A, A, A, 8, 32, A, None, None) == 1
    assert f(A, A, None, 8, 16, 256, 2, A, A, A, 8, 32, A, None, None) == 1   # x_out needed when n_out > 0
    assert f(A, A, A, 8, 16, 256, 2, A, A, None, 8, 32, A, None, None) == 1   # so is w_out
    assert f(A, A, A, 0, 16, 256, 2, A, A, A, 8, 32, A, None, None) == 2      # x_out_ld < n_out
    assert f(A, A, A, 4, 16, 256, 2, A, A, A, 8, 32, A, None, None) == 2      # x_out_ld not a multiple of 8
    assert f(A, A, A, 8, 16, 256, 2, A, A, A, 12, 32, A, None, None) == 2     # w_out_ld not a multiple of 8
    assert f(A, A, A, 8, 16, 200, 2, A, A, A, 8, 32, A, None, None) == 2      # k not a multiple of 128
    assert f(A, A, A, 8, 0, 256, 2, A, A, A, 8, 32, A, None, None) == 2
    assert f(A, A, A, 8, 16, 256, 2, A, A, A, 8, 0, A, None, None) == 2
    assert f(A, A, A, 304, 16, 256, 300, A, A, A, 304, 32, A, None, None) == 4  # more than QG_MAX_OUTLIERS
    assert f(A, A, A, 8, 16, 256, -1, A, A, A, 8, 32, A, None, None) == 4
    assert f(U, A, A, 8, 16, 256, 2, A, A, A, 8, 32, A, None, None) == 3
    assert f(A, A, A, 8, 16, 256, 2, U, A, A, 8, 32, A, None, None) == 3
    assert f(A, A, U, 8, 16, 256, 2, A, A, A, 8, 32, A, None, None) == 3      # x_out rows must be 16-B aligned


def test_header_constants_match_binding(qg):
    """Every #define QG_* value in the header equals the binding's constant."""
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    defs = dict(re.findall(r"#define\s+(QG_[A-Z0-9_]+)\s+(-?\d+)", src))
    assert len(defs) >= 20
    for name, val in defs.items():
        if name.startswith("QG_ERR_") or name == "QG_OK":
            continue
        assert hasattr(qg, name), name
        assert getattr(qg, name) == int(val), name


@needs_no_gpu
def test_validation_detect_outliers(qg):
    l = qg.lib()
    f = l.qg_detect_outliers
    need = l.qg_detect_outliers_workspace_bytes(64)
    assert need >= 64 * 4 and need % (64 * 4) == 0  # partial ranges of whole row blocks
    assert l.qg_detect_outliers_workspace_bytes(0) == 0
    # (x, rows, cols, n_out, idx, ws, ws_bytes, stream)
    assert f(None, 4, 64, 3, A, A, need, None) == 1
    assert f(A, 4, 64, 3, None, A, need, None) == 1
    assert f(A, 0, 64, 3, A, A, need, None) == 2
    assert f(A, 4, 60, 3, A, A, need, None) == 2          # cols not a multiple of 8
    assert f(A, 4, 64, 65, A, A, need, None) == 4         # more than cols
    assert f(A, 4, 512, 257, A, A, 2048, None) == 4       # more than QG_MAX_OUTLIERS
    assert f(A, 4, 64, -1, A, A, need, None) == 4
    assert f(U, 4, 64, 3, A, A, need, None) == 3
    assert f(A, 4, 64, 3, A, A, need - 1, None) == 5
    assert f(A, 4, 64, 3, A, None, need, None) == 5
    assert f(A, 4, 64, 3, A, A + 4, need, None) == 3     # workspace not 16-B aligned
    assert f(A, 4, 64, 0, None, None, 0, None) == 0       # nothing to find: no launch


@needs_no_gpu
def test_validation_sep_threshold(qg):
    l = qg.lib()
    import oracle.threshold as th
    # the smallest residual stride: the oracle's bound, rounded up to 16
    for k, pz in ((1024, 50), (1152, 0), (4096, 30), (128, 100), (8192, 40)):
        assert l.qg_sep_resid_ld(k, pz) == max(16, th.resid_ld(k, pz))
    assert l.qg_sep_resid_ld(1024, 101) == 0 and l.qg_sep_resid_ld(1024, -1) == 0
    f = l.qg_split_sep_threshold
    ld = l.qg_sep_resid_ld(1024, 50)
    # (w, n, k, pct_b, pct_z, cls, rv, rv_ld, alpha, s_r, stream)
    assert f(None, 4, 1024, 80, 50, A, A, ld, A, A, None) == 1
    assert f(A, 4, 1024, 80, 50, A, A, ld, None, A, None) == 1
    assert f(A, 0, 1024, 80, 50, A, A, ld, A, A, None) == 2
    assert f(A, 4, 1000, 80, 50, A, A, ld, A, A, None) == 2        # k not a multiple of 128
    assert f(A, 4, 65536 + 128, 80, 50, A, A, 65536, A, A, None) == 2  # beyond QG_SEP_MAX_K
    assert f(A, 4, 1024, 0, 0, A, A, ld, A, A, None) == 4          # pct_backbone < 1
    assert f(A, 4, 1024, 50, 60, A, A, ld, A, A, None) == 4        # pct_zero > pct_backbone
    assert f(A, 4, 1024, 101, 50, A, A, ld, A, A, None) == 4
    assert f(A, 4, 1024, 80, 50, A, A, ld - 16, A, A, None) == 2   # stride below the bound
    assert f(A, 4, 1024, 80, 50, A, A, ld + 8, A, A, None) == 2    # not a multiple of 16
    assert f(U, 4, 1024, 80, 50, A, A, ld, A, A, None) == 3
    assert f(A, 4, 1024, 80, 50, A, U, ld, A, A, None) == 3
    g = l.qg_qgemv_sep
    # (cls, rv, rv_ld, alpha, s_r, n, k, x, xt, skip, y, acc_out, stream)
    assert g(None, A, ld, A, A, 4, 1024, A, 0, 0, A, None, None) == 1
    assert g(A, None, ld, A, A, 4, 1024, A, 0, 0, A, None, None) == 1  # residual needed unless skipped
    assert g(A, A, ld, A, None, 4, 1024, A, 0, 0, A, None, None) == 1
    assert g(A, A, ld, A, A, 4, 1024, None, 0, 0, A, None, None) == 1
    assert g(A, A, ld, A, A, 0, 1024, A, 0, 0, A, None, None) == 2
    assert g(A, A, ld, A, A, 4, 1000, A, 0, 0, A, None, None) == 2
    assert g(A, A, 8, A, A, 4, 1024, A, 0, 0, A, None, None) == 2     # rv_ld below 16
    assert g(A, A, 2048, A, A, 4, 1024, A, 0, 0, A, None, None) == 2  # rv_ld above k
    assert g(A, A, ld, A, A, 4, 1024, A, 2, 0, A, None, None) == 4    # x dtype
    assert g(U, A, ld, A, A, 4, 1024, A, 0, 0, A, None, None) == 3
    assert g(A, U, ld, A, A, 4, 1024, A, 0, 0, A, None, None) == 3
    assert g(A, A, ld, A, A, 4, 1024, U, 1, 0, A, None, None) == 3
    h = l.qg_qgemv_sep_grouped

    def M(cls=A, rv=A, rv_ld=ld, n=4, y=A):
        return qg.CSepMatrix(cls, rv, rv_ld, A, A, n, y, None)

    def grp(*ms):
        return (qg.CSepMatrix * len(ms))(*ms)
    # (m, count, k, x, xt, skip, stream)
    assert h(None, 1, 1024, A, 0, 0, None) == 1
    assert h(grp(M()), 0, 1024, A, 0, 0, None) == 4                 # count below 1
    assert h(grp(*[M()] * 9), 9, 1024, A, 0, 0, None) == 4          # count above QG_MAX_GROUP
    assert h(grp(M(), M(y=None)), 2, 1024, A, 0, 0, None) == 1      # a later matrix fails: nothing launched
    assert h(grp(M(), M(n=0)), 2, 1024, A, 0, 0, None) == 2
    assert h(grp(M(), M(rv_ld=8)), 2, 1024, A, 0, 0, None) == 2
    assert h(grp(M(), M(cls=U)), 2, 1024, A, 0, 0, None) == 3
    assert h(grp(M(), M()), 2, 1000, A, 0, 0, None) == 2            # shared k not a multiple of 128
    assert h(grp(M(), M()), 2, 1024, U, 1, 0, None) == 3            # shared x misaligned
    assert h(grp(M(), M()), 2, 1024, A, 2, 0, None) == 4            # x dtype


@needs_no_gpu
def test_validation_qgemv_batch(qg):
    l = qg.lib()

    def W(fmt=0, n=64, k=256, codes=A, scale=A):
        return qg.CWeight(fmt, 0, n, k, codes, None, scale, None)
    f = l.qg_qgemv_batch
    # (w, m, x, xt, y, yt, stream)
    assert f(None, 4, A, 1, A, 0, None) == 1
    assert f(ctypes.byref(W(codes=None)), 4, A, 1, A, 0, None) == 1
    assert f(ctypes.byref(W(scale=None)), 4, A, 1, A, 0, None) == 1
    assert f(ctypes.byref(W()), 4, None, 1, A, 0, None) == 1
    assert f(ctypes.byref(W()), 4, A, 0, A, 0, None) == 4          # x must be bf16
    assert f(ctypes.byref(W()), 4, A, 1, A, 2, None) == 4          # y dtype
    assert f(ctypes.byref(W(fmt=1)), 4, A, 1, A, 0, None) == 4     # int8 weights only
    assert f(ctypes.byref(W()), 0, A, 1, A, 0, None) == 2          # m >= 1
    assert f(ctypes.byref(W()), 17, A, 1, A, 0, None) == 2         # m <= QG_BATCH_MAX_M
    assert f(ctypes.byref(W(k=192)), 4, A, 1, A, 0, None) == 2     # k % 128
    assert f(ctypes.byref(W(k=262144 + 128)), 4, A, 1, A, 0, None) == 2
    assert f(ctypes.byref(W(n=0)), 4, A, 1, A, 0, None) == 2
    assert f(ctypes.byref(W(codes=U)), 4, A, 1, A, 0, None) == 3
    assert f(ctypes.byref(W()), 4, U, 1, A, 0, None) == 3
    g = l.qg_qgemv_batch_grouped
    arr = (qg.CWeight * 2)(W(), W(k=512))
    ys = (ctypes.c_void_p * 2)(A, A)
    assert g(arr, 2, 4, A, 1, ys, 0, None) == 2                    # k must agree
    assert g(arr, 0, 4, A, 1, ys, 0, None) == 4
    assert g(arr, 9, 4, A, 1, ys, 0, None) == 4
    ys0 = (ctypes.c_void_p * 2)(A, None)
    arr2 = (qg.CWeight * 2)(W(), W())
    assert g(arr2, 2, 4, A, 1, ys0, 0, None) == 1


def test_batch_workspace_bytes(qg):
    # sizes on the 256-CU part (the library's count when no device answers):
    # 4 splits x 256 tiles x 64 lanes x 16 B of partial tiles, then 64 row
    # blocks of 4 tiles, one 4-B counter each, rounded up to 256 B
    l = qg.lib()
    if torch.cuda.device_count() > 0:
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        if cus != 256:
            pytest.skip("sizes below are for 256 CUs")
    f = l.qg_qgemv_batch_workspace_bytes
    assert f(4096, 11008, 16) == 4 * 256 * 64 * 16 + 256
    assert f(4096, 8192, 4) == 4 * 256 * 64 * 16 + 256
    assert f(777, 8192, 7) == 4 * 49 * 64 * 16 + 256     # 49 tiles, one per row block
    assert f(4096, 16384, 16) > 0                        # 64 units per split: 8 per wave
    assert f(4096, 16384 + 128, 16) == 0                 # 9 per wave: no split
    assert f(4096, 8192 - 128, 16) == 0                  # below the split's smallest k
    assert f(4096, 4096, 16) == 0
    assert f(4097, 11008, 16) == 0                       # more tiles than CUs
    assert f(4096, 11008, 1) == 0                        # one token: batch-1 kernel
    assert f(4096, 11008, 17) == 0
    assert f(4096, 192, 4) == 0                          # invalid k
    assert f(0, 11008, 4) == 0


@needs_no_gpu
def test_validation_qgemv_batch_ws(qg):
    l = qg.lib()
    f = l.qg_qgemv_batch_ws
    need = l.qg_qgemv_batch_workspace_bytes(4096, 11008, 16)
    w = qg.CWeight(0, 0, 4096, 11008, A, None, A, None)
    # (w, m, x, xt, y, yt, ws, ws_bytes, stream)
    assert f(None, 16, A, 1, A, 0, A, need, None) == 1
    assert f(ctypes.byref(w), 16, A, 1, A, 0, None, need, None) == 5       # no workspace
    assert f(ctypes.byref(w), 16, A, 1, A, 0, A, need - 1, None) == 5      # too small
    assert f(ctypes.byref(w), 16, A, 1, A, 0, U, need, None) == 3          # misaligned workspace
    assert f(ctypes.byref(w), 16, U, 1, A, 0, A, need, None) == 3
    assert f(ctypes.byref(w), 16, A, 0, A, 0, A, need, None) == 4          # x must be bf16
    assert f(ctypes.byref(w), 16, A, 1, A, 2, A, need, None) == 4
    assert f(ctypes.byref(w), 16, None, 1, A, 0, A, need, None) == 1
    wt = qg.CWeight(1, 0, 4096, 11008, A, None, A, None)
    assert f(ctypes.byref(wt), 16, A, 1, A, 0, A, need, None) == 4         # int8 weights only
    # shapes without a split fall through to qg_qgemv_batch's checks
    assert f(ctypes.byref(w), 17, A, 1, A, 0, None, 0, None) == 2
    wk = qg.CWeight(0, 0, 4096, 192, A, None, A, None)
    assert f(ctypes.byref(wk), 4, A, 1, A, 0, None, 0, None) == 2


def test_tiles16_bytes(qg):
    f = qg.lib().qg_tiles16_bytes
    assert f(16, 128) == 16 * 128
    assert f(17, 128) == 32 * 128          # the last tile padded to 16 rows
    assert f(4096, 4096) == 4096 * 4096
    assert f(777, 1152) == 784 * 1152
    assert f(0, 128) == 0 and f(16, 192) == 0 and f(16, 64) == 0 and f(16, 262144 + 128) == 0


@needs_no_gpu
def test_validation_tiled16(qg):
    l = qg.lib()
    p = l.qg_pack_tiles16
    # (codes, n, k, out, stream)
    assert p(None, 16, 128, A, None) == 1
    assert p(A, 16, 128, None, None) == 1
    assert p(A, 0, 128, A, None) == 2
    assert p(A, 16, 192, A, None) == 2
    assert p(U, 16, 128, A, None) == 3
    assert p(A, 16, 128, U, None) == 3
    # a grouped batch launch takes one layout
    g = l.qg_qgemv_batch_grouped
    arr = (qg.CWeight * 2)(qg.CWeight(0, 0, 64, 256, A, None, A, None), qg.CWeight(6, 0, 64, 256, A, None, A, None))
    ys = (ctypes.c_void_p * 2)(A, A)
    assert g(arr, 2, 4, A, 1, ys, 0, None) == 4
    # the batch-1 product does not read the tiled layout
    q = l.qg_qgemv
    wt = qg.CWeight(6, 0, 64, 256, A, None, A, None)
    assert q(ctypes.byref(wt), 1, A, 1, A, 0, None, None) == 4


@needs_no_gpu
def test_validation_mxfp4(qg):
    l = qg.lib()
    q = l.qg_quantize_mxfp4
    # (x, xt, rows, cols, codes, scales, stream)
    assert q(None, 1, 4, 256, A, A, None) == 1
    assert q(A, 1, 4, 256, A, None, None) == 1
    assert q(A, 2, 4, 256, A, A, None) == 4
    assert q(A, 1, 0, 256, A, A, None) == 2
    assert q(A, 1, 4, 48, A, A, None) == 2      # cols % 256
    assert q(A, 1, 4, 288, A, A, None) == 2
    assert q(U, 1, 4, 256, A, A, None) == 3
    assert q(A, 1, 4, 256, U, A, None) == 3
    g = l.qg_gemm_mxfp4
    # (a, as, m, k, b, bs, n, y, stream)
    assert g(None, A, 4, 256, A, A, 4, A, None) == 1
    assert g(A, A, 4, 256, A, A, 4, None, None) == 1
    assert g(A, A, 0, 256, A, A, 4, A, None) == 2
    assert g(A, A, 4, 128, A, A, 4, A, None) == 2  # k % 256
    assert g(A, A, 4, 256 + 128, A, A, 4, A, None) == 2
    assert g(A, A, 4, 256, A, A, 0, A, None) == 2
    assert g(A, U, 4, 256, A, A, 4, A, None) == 3
    assert g(A, A, 4, 256, U, A, 4, A, None) == 3
    need = l.qg_prefill_mxfp4_workspace_bytes(64, 512)
    assert need >= 64 * 256 + 64 * 16 and need % 256 == 0
    assert l.qg_prefill_mxfp4_workspace_bytes(64, 100) == 0
    p = l.qg_prefill_mxfp4
    # (x, m, k, w, ws_scales, n, y, ws, ws_bytes, stream)
    assert p(None, 64, 512, A, A, 8, A, A, need, None) == 1
    assert p(A, 64, 512, A, A, 8, A, None, need, None) == 5
    assert p(A, 64, 512, A, A, 8, A, A, need - 1, None) == 5
    assert p(A, 64, 512, A, A, 8, A, U, need, None) == 3
    assert p(A, 64, 500, A, A, 8, A, A, need, None) == 2
