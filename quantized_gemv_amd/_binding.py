"""ctypes binding over libqgemv.so (the C ABI declared in include/qgemv.h).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, their data pointers and the current HIP stream are passed to the
library, and a non-zero status raises ``QgError``.  Every computation runs in
the library's HIP kernels; there is no fallback of any kind.  PyTorch is used
for device memory (output and workspace allocation) and streams.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqgemv.so")

QG_OK = 0
QG_ERR_DEVICE_CHECK = 7  # QG_DEBUG=1 (or 2) only: a device-side check of the outlier path failed
QG_F32, QG_BF16 = 0, 1
QG_PER_TENSOR, QG_PER_ROW = 0, 1
QG_WFMT_INT8, QG_WFMT_TERNARY2, QG_WFMT_SIGN1_RES8, QG_WFMT_Q4K, QG_WFMT_SIGN1_RES8Z, QG_WFMT_TERNARY3 = 0, 1, 2, 3, 4, 5
QG_WFMT_INT8_T16 = 6
QG_ACT_INT8, QG_ACT_FLOAT = 0, 1
QG_MAX_OUTLIERS = 256
QG_QGEMV_MAX_K = 32768
QG_MAX_GROUP = 8
QG_OUT_LD_ALIGN = 8
QG_MAX_OUT_LD = 65536
QG_SEP_MAX_K = 65536
QG_BATCH_MAX_M = 16
QG_BATCH_MAX_K = 262144
QG_MX_BLOCK = 32
QG_QGEMM_MAX_K = 133120
QG_ABSMAX_SCRATCH_PARTS = 1024
QG_CHAIN_MAX_STAGES = 4096
QG_CHAIN_MIN_K = 128
QG_CHAIN_MAX_K = 16384
QG_CHAIN_ERROR_OFFSET = 64
QG_CHAIN_TIMEOUT_TICKS = 200000000

_c_i32, _c_i64, _c_sz, _c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p


class QgError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__("%s failed: %s (status %d)" % (what, status_str(status), status))
        self.status = status


class CWeight(ctypes.Structure):
    _fields_ = [("fmt", _c_i32), ("reserved", _c_i32), ("n", _c_i64), ("k", _c_i64),
                ("codes", _c_vp), ("resid", _c_vp), ("scale", _c_vp), ("scale2", _c_vp), ("zero", _c_vp)]


class CSepMatrix(ctypes.Structure):
    _fields_ = [("cls", _c_vp), ("rv", _c_vp), ("rv_ld", _c_i64), ("alpha", _c_vp), ("s_r", _c_vp), ("n", _c_i64),
                ("y", _c_vp), ("acc_out", _c_vp)]


class CChainStage(ctypes.Structure):
    _fields_ = [("count", _c_i32), ("dep", _c_i32), ("x", _c_vp), ("w", ctypes.POINTER(CWeight)),
                ("y", ctypes.POINTER(_c_vp))]


_SIGS = {
    "qg_status_str": (ctypes.c_char_p, [_c_i32]),
    "qg_abi_version": (_c_i32, []),
    "qg_quantize_absmax_workspace_bytes": (_c_sz, [_c_i64, _c_i64, _c_i32]),
    "qg_quantize_absmax": (_c_i32, [_c_vp, _c_i32, _c_i64, _c_i64, _c_i32, _c_vp, _c_vp, _c_vp, _c_sz, _c_vp]),
    "qg_quantize_absmax_noalloc": (_c_i32, [_c_vp, _c_i32, _c_i64, _c_i64, _c_i32, _c_vp, _c_vp, _c_vp]),
    "qg_probe_stream_read_bytes": (_c_sz, [_c_i64, _c_i32]),
    "qg_probe_stream_read": (_c_i32, [_c_vp, _c_i64, _c_i32, _c_vp, _c_vp]),
    "qg_chain_plan_bytes": (_c_sz, [ctypes.POINTER(CChainStage), _c_i32, _c_i32]),
    "qg_chain_plan": (_c_i32, [ctypes.POINTER(CChainStage), _c_i32, _c_i32, _c_vp, _c_sz]),
    "qg_qgemv_chain": (_c_i32, [_c_vp, _c_vp, _c_vp]),
    "qg_quantize_absmax_split": (_c_i32, [_c_vp, _c_i64, _c_i64, _c_vp, _c_i32, _c_vp, _c_vp, _c_vp, _c_i32,
                                          _c_vp]),
    "qg_detect_outliers_workspace_bytes": (_c_sz, [_c_i64]),
    "qg_detect_outliers": (_c_i32, [_c_vp, _c_i64, _c_i64, _c_i32, _c_vp, _c_vp, _c_sz, _c_vp]),
    "qg_gather_columns_bf16": (_c_i32, [_c_vp, _c_i64, _c_i64, _c_vp, _c_i32, _c_vp, _c_i32, _c_vp]),
    "qg_ternary_workspace_bytes": (_c_sz, [_c_i64, _c_i64]),
    "qg_quantize_ternary": (_c_i32, [_c_vp, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp, _c_sz, _c_vp]),
    "qg_split_sign_residual": (_c_i32, [_c_vp, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp]),
    "qg_split_sign_residual_zp": (_c_i32, [_c_vp, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp]),
    "qg_quantize_asym": (_c_i32, [_c_vp, _c_i32, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp, _c_vp]),
    "qg_quantize_q4k": (_c_i32, [_c_vp, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp]),
    "qg_qgemv_batch": (_c_i32, [ctypes.POINTER(CWeight), _c_i32, _c_vp, _c_i32, _c_vp, _c_i32, _c_vp]),
    "qg_qgemv_batch_workspace_bytes": (_c_sz, [_c_i64, _c_i64, _c_i32]),
    "qg_qgemv_batch_ws": (_c_i32, [ctypes.POINTER(CWeight), _c_i32, _c_vp, _c_i32, _c_vp, _c_i32, _c_vp, _c_sz, _c_vp]),
    "qg_qgemv_batch_grouped": (_c_i32, [ctypes.POINTER(CWeight), _c_i32, _c_i32, _c_vp, _c_i32,
                                        ctypes.POINTER(_c_vp), _c_i32, _c_vp]),
    "qg_quantize_mxfp4": (_c_i32, [_c_vp, _c_i32, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp]),
    "qg_gemm_mxfp4": (_c_i32, [_c_vp, _c_vp, _c_i64, _c_i64, _c_vp, _c_vp, _c_i64, _c_vp, _c_vp]),
    "qg_prefill_mxfp4_workspace_bytes": (_c_sz, [_c_i64, _c_i64]),
    "qg_prefill_mxfp4": (_c_i32, [_c_vp, _c_i64, _c_i64, _c_vp, _c_vp, _c_i64, _c_vp, _c_vp, _c_sz, _c_vp]),
    "qg_sep_resid_ld": (_c_i64, [_c_i64, _c_i32]),
    "qg_split_sep_threshold": (_c_i32, [_c_vp, _c_i64, _c_i64, _c_i32, _c_i32, _c_vp, _c_vp, _c_i64, _c_vp, _c_vp,
                                        _c_vp]),
    "qg_qgemv_sep": (_c_i32, [_c_vp, _c_vp, _c_i64, _c_vp, _c_vp, _c_i64, _c_i64, _c_vp, _c_i32, _c_i32, _c_vp,
                              _c_vp, _c_vp]),
    "qg_qgemv_sep_grouped": (_c_i32, [ctypes.POINTER(CSepMatrix), _c_i32, _c_i64, _c_vp, _c_i32, _c_i32, _c_vp]),
    "qg_pack": (_c_i32, [_c_vp, _c_i64, _c_i64, _c_i32, _c_vp, _c_vp]),
    "qg_base3_row_bytes": (_c_i64, [_c_i64]),
    "qg_pack_base3": (_c_i32, [_c_vp, _c_i64, _c_i64, _c_vp, _c_vp]),
    "qg_tiles16_bytes": (_c_i64, [_c_i64, _c_i64]),
    "qg_pack_tiles16": (_c_i32, [_c_vp, _c_i64, _c_i64, _c_vp, _c_vp]),
    "qg_unpack_base3": (_c_i32, [_c_vp, _c_i64, _c_i64, _c_vp, _c_vp]),
    "qg_unpack": (_c_i32, [_c_vp, _c_i64, _c_i64, _c_i32, _c_vp, _c_vp]),
    "qg_qgemv": (_c_i32, [ctypes.POINTER(CWeight), _c_i32, _c_vp, _c_i32, _c_vp, _c_i32, _c_vp, _c_vp]),
    "qg_qgemv_grouped": (_c_i32, [ctypes.POINTER(CWeight), _c_i32, _c_i32, _c_vp, _c_i32, ctypes.POINTER(_c_vp),
                                  _c_i32, ctypes.POINTER(_c_vp), _c_vp]),
    "qg_qgemm_workspace_bytes": (_c_sz, [_c_i64, _c_i64, _c_i32]),
    "qg_qgemm_w8a8_outlier": (_c_i32, [_c_vp, _c_i64, _c_i64, _c_vp, _c_i32, _c_vp, _c_vp, _c_vp, _c_i32, _c_i64,
                                       _c_vp, _c_vp, _c_vp, _c_sz, _c_vp]),
    "qg_qgemm_w8a8": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_i32, _c_i64, _c_i64, _c_i32, _c_vp, _c_vp, _c_vp, _c_i32,
                               _c_i64, _c_vp, _c_vp, _c_vp]),
}
EXPORTED = tuple(_SIGS)

_lib = None


def lib() -> ctypes.CDLL:
    """Load libqgemv.so (built in-tree by quantized_gemv_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libqgemv.so is not built (%s); run quantized_gemv_amd.build.build()" % LIB_PATH)
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def status_str(st: int) -> str:
    return lib().qg_status_str(st).decode()


def _check(st: int, what: str):
    if st != QG_OK:
        raise QgError(st, what)


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    return t


def _xt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return QG_F32
    if t.dtype == torch.bfloat16:
        return QG_BF16
    raise ValueError("activation dtype must be float32 or bfloat16")


def _idx_host(idx: Optional[Sequence[int]]):
    if idx is None:
        return None, 0
    arr = (ctypes.c_int32 * max(len(idx), 1))(*[int(v) for v in idx])
    return arr, len(idx)


# ------------------------------------------------------------------ quantizers

def quantize_absmax(x: torch.Tensor, per_row: bool = True, q: torch.Tensor = None, s: torch.Tensor = None):
    """Symmetric absmax int8 quantization (qg_quantize_absmax). Returns (q, s)."""
    _dev(x, "x", (torch.float32, torch.bfloat16))
    rows, cols = (1, x.shape[0]) if x.dim() == 1 else tuple(x.shape)
    q = torch.empty(x.shape, dtype=torch.int8, device=x.device) if q is None else _dev(q, "q", torch.int8)
    s = torch.empty(rows if per_row else 1, dtype=torch.float32, device=x.device) if s is None else _dev(s, "s", torch.float32)
    gran = QG_PER_ROW if per_row else QG_PER_TENSOR
    nws = lib().qg_quantize_absmax_workspace_bytes(rows, cols, gran)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=x.device) if nws else None
    _check(lib().qg_quantize_absmax(_p(x), _xt(x), rows, cols, gran, _p(q), _p(s), _p(ws), nws, _stream(x)),
           "qg_quantize_absmax")
    return q, s


def out_ld(n_out: int) -> int:
    """Row stride of an outlier operand the prefill GEMMs read: n_out rounded
    up to QG_OUT_LD_ALIGN elements."""
    return -(-n_out // QG_OUT_LD_ALIGN) * QG_OUT_LD_ALIGN


def quantize_absmax_split(x: torch.Tensor, idx: Sequence[int], ld: Optional[int] = None):
    """Per-token int8 quantization with outlier channels split out
    (qg_quantize_absmax_split). Returns (q, s, x_out) with x_out [rows][ld]
    (ld defaults to out_ld(n_out); columns >= n_out are zero)."""
    _dev(x, "x", torch.bfloat16)
    rows, cols = x.shape
    cidx, n_out = _idx_host(idx)
    ld = out_ld(n_out) if ld is None else ld
    q = torch.empty((rows, cols), dtype=torch.int8, device=x.device)
    s = torch.empty(rows, dtype=torch.float32, device=x.device)
    xo = torch.empty((rows, ld), dtype=torch.bfloat16, device=x.device)
    _check(lib().qg_quantize_absmax_split(_p(x), rows, cols, cidx, n_out, _p(q), _p(s), _p(xo) if n_out else None,
                                          ld, _stream(x)), "qg_quantize_absmax_split")
    return q, s, xo


def detect_outliers(x: torch.Tensor, n_out: int, ws: torch.Tensor = None) -> torch.Tensor:
    """The n_out channels of calibration activations x [rows][cols] (bf16)
    with the largest max |x| (qg_detect_outliers). Returns int32 [n_out] on
    the device, ascending."""
    _dev(x, "x", torch.bfloat16)
    rows, cols = x.shape
    idx = torch.empty(n_out, dtype=torch.int32, device=x.device)
    if ws is None:
        ws = torch.empty(max(1, lib().qg_detect_outliers_workspace_bytes(cols)), dtype=torch.uint8, device=x.device)
    _check(lib().qg_detect_outliers(_p(x), rows, cols, n_out, _p(idx) if n_out else None, _p(ws), ws.numel(),
                                    _stream(x)), "qg_detect_outliers")
    return idx


def gather_columns_bf16(w: torch.Tensor, idx: Sequence[int], ld: Optional[int] = None):
    """W_out[n][j] = bf16(W[n][idx[j]]) (qg_gather_columns_bf16), as [n][ld]
    (ld defaults to out_ld(n_out); columns >= n_out are zero)."""
    _dev(w, "w", torch.float32)
    n, k = w.shape
    cidx, n_out = _idx_host(idx)
    ld = out_ld(n_out) if ld is None else ld
    wo = torch.empty((n, ld), dtype=torch.bfloat16, device=w.device)
    _check(lib().qg_gather_columns_bf16(_p(w), n, k, cidx, n_out, _p(wo) if n_out else None, ld, _stream(w)),
           "qg_gather_columns_bf16")
    return wo


def quantize_ternary(w: torch.Tensor):
    """Ternary absmean quantization (qg_quantize_ternary). Returns (codes, gamma[1])."""
    _dev(w, "w", torch.float32)
    n, k = (1, w.shape[0]) if w.dim() == 1 else tuple(w.shape)
    q = torch.empty(w.shape, dtype=torch.int8, device=w.device)
    g = torch.empty(1, dtype=torch.float32, device=w.device)
    nws = lib().qg_ternary_workspace_bytes(n, k)
    ws = torch.empty(nws, dtype=torch.uint8, device=w.device)
    _check(lib().qg_quantize_ternary(_p(w), n, k, _p(q), _p(g), _p(ws), nws, _stream(w)), "qg_quantize_ternary")
    return q, g


def split_sign_residual(w: torch.Tensor):
    """Sign backbone + int8 residual split (qg_split_sign_residual).
    Returns (sign int8, alpha, rq int8, s_r)."""
    _dev(w, "w", torch.float32)
    n, k = w.shape
    sign = torch.empty((n, k), dtype=torch.int8, device=w.device)
    rq = torch.empty((n, k), dtype=torch.int8, device=w.device)
    alpha = torch.empty(n, dtype=torch.float32, device=w.device)
    s_r = torch.empty(n, dtype=torch.float32, device=w.device)
    _check(lib().qg_split_sign_residual(_p(w), n, k, _p(sign), _p(alpha), _p(rq), _p(s_r), _stream(w)),
           "qg_split_sign_residual")
    return sign, alpha, rq, s_r


def split_sign_residual_zp(w: torch.Tensor):
    """Sign backbone + asymmetric int8 residual (qg_split_sign_residual_zp).
    Returns (sign int8, alpha, rq int8, s_r, z_r int8)."""
    _dev(w, "w", torch.float32)
    n, k = w.shape
    sign = torch.empty((n, k), dtype=torch.int8, device=w.device)
    rq = torch.empty((n, k), dtype=torch.int8, device=w.device)
    alpha = torch.empty(n, dtype=torch.float32, device=w.device)
    s_r = torch.empty(n, dtype=torch.float32, device=w.device)
    z_r = torch.empty(n, dtype=torch.int8, device=w.device)
    _check(lib().qg_split_sign_residual_zp(_p(w), n, k, _p(sign), _p(alpha), _p(rq), _p(s_r), _p(z_r), _stream(w)),
           "qg_split_sign_residual_zp")
    return sign, alpha, rq, s_r, z_r


def quantize_asym(x: torch.Tensor):
    """Asymmetric int8 quantization per row (qg_quantize_asym): x [rows][cols]
    fp32 or bf16. Returns (q int8, s fp32 [rows], z int8 [rows])."""
    _dev(x, "x", (torch.float32, torch.bfloat16))
    if x.dim() != 2:
        raise ValueError("x must be [rows][cols]")
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.int8, device=x.device)
    s = torch.empty(rows, dtype=torch.float32, device=x.device)
    z = torch.empty(rows, dtype=torch.int8, device=x.device)
    _check(lib().qg_quantize_asym(_p(x), _xt(x), rows, cols, _p(q), _p(s), _p(z), _stream(x)), "qg_quantize_asym")
    return q, s, z


def pack(codes: torch.Tensor, bits: int, out: torch.Tensor = None):
    """Bit packing (qg_pack): bits=2 ternary, bits=1 sign."""
    _dev(codes, "codes", torch.int8)
    n, k = (1, codes.shape[0]) if codes.dim() == 1 else tuple(codes.shape)
    if bits not in (1, 2) or k % (8 // bits):
        raise ValueError("bad bits or row length")
    out = torch.empty((n, k * bits // 8), dtype=torch.uint8, device=codes.device) if out is None else out
    _check(lib().qg_pack(_p(codes), n, k, bits, _p(out), _stream(codes)), "qg_pack")
    return out


def unpack(packed: torch.Tensor, bits: int, k: int):
    """Inverse of pack (qg_unpack)."""
    _dev(packed, "packed", torch.uint8)
    n = packed.shape[0] if packed.dim() == 2 else 1
    out = torch.empty((n, k), dtype=torch.int8, device=packed.device)
    _check(lib().qg_unpack(_p(packed), n, k, bits, _p(out), _stream(packed)), "qg_unpack")
    return out


def base3_row_bytes(k: int) -> int:
    """Bytes of one base-3 packed row (qg_base3_row_bytes): 16 per 80 weights."""
    return int(lib().qg_base3_row_bytes(k))


def pack_base3(codes: torch.Tensor, out: torch.Tensor = None):
    """Ternary codes, five per byte (qg_pack_base3): [n][k] int8 -> [n][base3_row_bytes(k)] uint8."""
    _dev(codes, "codes", torch.int8)
    n, k = (1, codes.shape[0]) if codes.dim() == 1 else tuple(codes.shape)
    rb = base3_row_bytes(k)
    out = torch.empty((n, rb), dtype=torch.uint8, device=codes.device) if out is None else out
    _check(lib().qg_pack_base3(_p(codes), n, k, _p(out), _stream(codes)), "qg_pack_base3")
    return out


def pack_tiles16(codes: torch.Tensor, out: torch.Tensor = None):
    """Int8 codes [n][k] in 16-row tiles for the batch products
    (qg_pack_tiles16): returns a flat int8 tensor of qg_tiles16_bytes(n, k)."""
    _dev(codes, "codes", torch.int8)
    if codes.dim() != 2:
        raise ValueError("codes must be [n][k]")
    n, k = codes.shape
    nb = int(lib().qg_tiles16_bytes(n, k))
    if nb == 0:
        raise ValueError("shape (%d, %d) has no 16-row tiled layout" % (n, k))
    out = torch.empty(nb, dtype=torch.int8, device=codes.device) if out is None else out
    if out.numel() < nb:
        raise ValueError("out holds %d bytes, %d needed" % (out.numel(), nb))
    _check(lib().qg_pack_tiles16(_p(codes), n, k, _p(out), _stream(codes)), "qg_pack_tiles16")
    return out


def tiled16(w: "QWeight") -> "QWeight":
    """The QG_WFMT_INT8 matrix w with its codes in 16-row tiles."""
    if w.fmt != QG_WFMT_INT8:
        raise ValueError("tiled16 takes QG_WFMT_INT8 weights")
    return QWeight(QG_WFMT_INT8_T16, w.n, w.k, pack_tiles16(w.codes.view(w.n, w.k)), w.scale)


def unpack_base3(packed: torch.Tensor, k: int):
    """Inverse of pack_base3 (qg_unpack_base3)."""
    _dev(packed, "packed", torch.uint8)
    n = packed.shape[0] if packed.dim() == 2 else 1
    out = torch.empty((n, k), dtype=torch.int8, device=packed.device)
    _check(lib().qg_unpack_base3(_p(packed), n, k, _p(out), _stream(packed)), "qg_unpack_base3")
    return out


# ------------------------------------------------------------------ products

@dataclass
class QWeight:
    """A quantized weight matrix as the library stores it."""
    fmt: int
    n: int
    k: int
    codes: torch.Tensor
    scale: Optional[torch.Tensor]
    resid: Optional[torch.Tensor] = None
    scale2: Optional[torch.Tensor] = None
    zero: Optional[torch.Tensor] = None

    def c_struct(self) -> CWeight:
        return CWeight(self.fmt, 0, self.n, self.k, self.codes.data_ptr(),
                       self.resid.data_ptr() if self.resid is not None else None,
                       self.scale.data_ptr() if self.scale is not None else None,
                       self.scale2.data_ptr() if self.scale2 is not None else None,
                       self.zero.data_ptr() if self.zero is not None else None)


def quantize_q4k(w: torch.Tensor):
    """Group-wise 4-bit codes with two-level scales (qg_quantize_q4k).
    Returns (codes plane uint8 [n][k/2], meta plane uint8 [n][k/256][16]);
    QWeight(QG_WFMT_Q4K, n, k, codes, None, resid=meta) describes them."""
    _dev(w, "w", torch.float32)
    n, k = w.shape
    codes = torch.empty((n, k // 2), dtype=torch.uint8, device=w.device)
    meta = torch.empty((n, k // 256, 16), dtype=torch.uint8, device=w.device)
    _check(lib().qg_quantize_q4k(_p(w), n, k, _p(codes), _p(meta), _stream(w)), "qg_quantize_q4k")
    return codes, meta


def qgemv_batch(w: QWeight, x: torch.Tensor, y_dtype=torch.float32, y: torch.Tensor = None,
                ws: Optional[torch.Tensor] = None):
    """Weight-only int8 product of a batch of tokens (qg_qgemv_batch): x bf16
    [m][k] -> y [m][n]. Returns y.  With ws (a uint8 device tensor of at least
    batch_workspace_bytes(w.n, w.k, m) bytes, zero-filled when allocated) the
    call is qg_qgemv_batch_ws (K split over workgroups)."""
    _dev(x, "x", torch.bfloat16)
    if x.dim() != 2:
        raise ValueError("x must be [m][k]")
    m = x.shape[0]
    if y is None:
        y = torch.empty((m, w.n), dtype=y_dtype, device=x.device)
    _dev(y, "y", (torch.float32, torch.bfloat16))
    cw = w.c_struct()
    if ws is None:
        _check(lib().qg_qgemv_batch(ctypes.byref(cw), m, _p(x), QG_BF16, _p(y), _xt(y), _stream(x)), "qg_qgemv_batch")
    else:
        _dev(ws, "ws", torch.uint8)
        _check(lib().qg_qgemv_batch_ws(ctypes.byref(cw), m, _p(x), QG_BF16, _p(y), _xt(y), _p(ws), ws.numel(),
                                       _stream(x)), "qg_qgemv_batch_ws")
    return y


def batch_workspace_bytes(n: int, k: int, m: int) -> int:
    """Workspace of qg_qgemv_batch_ws (0: the split path does not apply)."""
    return int(lib().qg_qgemv_batch_workspace_bytes(n, k, m))


def qgemv_batch_grouped(weights: Sequence[QWeight], x: torch.Tensor, y_dtype=torch.float32, ys=None):
    """qg_qgemv_batch_grouped: several int8 matrices sharing x [m][k] in one
    launch. Returns the list of y [m][n_j]."""
    _dev(x, "x", torch.bfloat16)
    m = x.shape[0]
    cnt = len(weights)
    if not 1 <= cnt <= QG_MAX_GROUP:
        raise ValueError("need 1..%d weights" % QG_MAX_GROUP)
    if ys is None:
        ys = [torch.empty((m, W.n), dtype=y_dtype, device=x.device) for W in weights]
    arr = (CWeight * cnt)(*[W.c_struct() for W in weights])
    yp = (_c_vp * cnt)(*[y.data_ptr() for y in ys])
    _check(lib().qg_qgemv_batch_grouped(arr, cnt, m, _p(x), QG_BF16, yp, _xt(ys[0]), _stream(x)),
           "qg_qgemv_batch_grouped")
    return ys


def quantize_mxfp4(x: torch.Tensor):
    """MXFP4 quantization of the rows of x [rows][cols] (fp32 or bf16)
    (qg_quantize_mxfp4). Returns (codes uint8 [rows][cols/2], scales uint8
    [cols/256][rows][8])."""
    _dev(x, "x", (torch.float32, torch.bfloat16))
    r, c = x.shape
    codes = torch.empty((r, c // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((c // 256, r, 8), dtype=torch.uint8, device=x.device)
    _check(lib().qg_quantize_mxfp4(_p(x), _xt(x), r, c, _p(codes), _p(scales), _stream(x)), "qg_quantize_mxfp4")
    return codes, scales


def gemm_mxfp4(a, a_scales, b, b_scales, y: torch.Tensor = None):
    """Y = A B^T of two MXFP4 operands (qg_gemm_mxfp4). Returns y fp32 [m][n]."""
    for t, nm in ((a, "a"), (a_scales, "a_scales"), (b, "b"), (b_scales, "b_scales")):
        _dev(t, nm, torch.uint8)
    m, n, k = a.shape[0], b.shape[0], 2 * a.shape[1]
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=a.device)
    _dev(y, "y", torch.float32)
    _check(lib().qg_gemm_mxfp4(_p(a), _p(a_scales), m, k, _p(b), _p(b_scales), n, _p(y), _stream(a)),
           "qg_gemm_mxfp4")
    return y


def prefill_mxfp4(x: torch.Tensor, w, w_scales, y: torch.Tensor = None, ws: torch.Tensor = None):
    """Format-separated prefill (qg_prefill_mxfp4): x bf16 [m][k] quantized to
    MXFP4 in the workspace, times the MXFP4 weights. Returns y fp32 [m][n]."""
    _dev(x, "x", torch.bfloat16)
    m, k = x.shape
    n = w.shape[0]
    need = int(lib().qg_prefill_mxfp4_workspace_bytes(m, k))
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=x.device)
    _check(lib().qg_prefill_mxfp4(_p(x), m, k, _p(w), _p(w_scales), n, _p(y), _p(ws), ws.numel(), _stream(x)),
           "qg_prefill_mxfp4")
    return y


class SepWeight:
    """Thresholded separated weights as qg_split_sep_threshold writes them:
    cls [n][k/4] uint8 (2-bit classes), rv [n][ld] int8 (residual codes in
    increasing k, then zeros), alpha [n] and s_r [n] fp32."""

    def __init__(self, cls: torch.Tensor, rv: torch.Tensor, alpha: torch.Tensor, s_r: torch.Tensor, k: int):
        self.cls, self.rv, self.alpha, self.s_r = cls, rv, alpha, s_r
        self.n, self.k = cls.shape[0], k
        self.ld = rv.shape[1]


def sep_resid_ld(k: int, pct_zero: int) -> int:
    """Smallest valid row stride of the residual stream (qg_sep_resid_ld)."""
    return int(lib().qg_sep_resid_ld(k, pct_zero))


def split_sep_threshold(w: torch.Tensor, pct_backbone: int = 80, pct_zero: int = 50, ld: Optional[int] = None):
    """Thresholded separated split (qg_split_sep_threshold). Returns SepWeight."""
    _dev(w, "w", torch.float32)
    n, k = w.shape
    if ld is None:
        ld = sep_resid_ld(k, pct_zero)
    cls = torch.empty((n, k // 4), dtype=torch.uint8, device=w.device)
    rv = torch.empty((n, max(int(ld), 1)), dtype=torch.int8, device=w.device)
    alpha = torch.empty(n, dtype=torch.float32, device=w.device)
    s_r = torch.empty(n, dtype=torch.float32, device=w.device)
    _check(lib().qg_split_sep_threshold(_p(w), n, k, pct_backbone, pct_zero, _p(cls), _p(rv), int(ld), _p(alpha),
                                        _p(s_r), _stream(w)), "qg_split_sep_threshold")
    return SepWeight(cls, rv, alpha, s_r, k)


def qgemv_sep(sw: SepWeight, x: torch.Tensor, skip_residual: bool = False, y: torch.Tensor = None,
              acc_out: torch.Tensor = None):
    """Batch-1 product on thresholded separated weights (qg_qgemv_sep);
    acc_out, if given, is int32 [2][n] (backbone, residual). Returns y (fp32)."""
    _dev(x, "x", (torch.float32, torch.bfloat16))
    if y is None:
        y = torch.empty(sw.n, dtype=torch.float32, device=x.device)
    _dev(y, "y", torch.float32)
    if acc_out is not None:
        _dev(acc_out, "acc_out", torch.int32)
    _check(lib().qg_qgemv_sep(_p(sw.cls), _p(sw.rv), sw.ld, _p(sw.alpha), _p(sw.s_r), sw.n, sw.k, _p(x), _xt(x),
                              1 if skip_residual else 0, _p(y), _p(acc_out), _stream(x)), "qg_qgemv_sep")
    return y


class SepGroupLaunch:
    """Pre-marshalled arguments of one qg_qgemv_sep_grouped call: products of
    1..QG_MAX_GROUP thresholded separated matrices on the same x (kept alive
    by this object); launch() enqueues it on x's current stream."""

    def __init__(self, weights: Sequence[SepWeight], x: torch.Tensor, ys: Sequence[torch.Tensor],
                 skip_residual: bool = False, accs: Optional[Sequence[torch.Tensor]] = None):
        _dev(x, "x", (torch.float32, torch.bfloat16))
        n = len(weights)
        if not 1 <= n <= QG_MAX_GROUP or len(ys) != n or (accs is not None and len(accs) != n):
            raise ValueError("need 1..%d weights and as many outputs" % QG_MAX_GROUP)
        for y in ys:
            _dev(y, "y", torch.float32)
        if accs is not None:
            for a in accs:
                if a is not None:
                    _dev(a, "acc_out", torch.int32)
        self.keep = (list(weights), x, list(ys), accs)
        self.m = (CSepMatrix * n)(*[
            CSepMatrix(_p(w.cls), _p(w.rv), w.ld, _p(w.alpha), _p(w.s_r), w.n, _p(y),
                       None if accs is None or accs[i] is None else _p(accs[i]))
            for i, (w, y) in enumerate(zip(weights, ys))])
        self.n, self.k, self.x, self.xt = n, weights[0].k, x, _xt(x)
        self.skip = 1 if skip_residual else 0

    def launch(self):
        _check(lib().qg_qgemv_sep_grouped(self.m, self.n, self.k, _p(self.x), self.xt, self.skip, _stream(self.x)),
               "qg_qgemv_sep_grouped")


def qgemv_sep_grouped(weights: Sequence[SepWeight], x: torch.Tensor, skip_residual: bool = False,
                      accs: Optional[Sequence[torch.Tensor]] = None):
    """Thresholded separated products on the same x in one launch
    (qg_qgemv_sep_grouped). Returns [y] (fp32)."""
    ys = [torch.empty(w.n, dtype=torch.float32, device=x.device) for w in weights]
    SepGroupLaunch(weights, x, ys, skip_residual, accs).launch()
    return ys


def qgemv(w: QWeight, x: torch.Tensor, act_int8: bool, y_dtype=torch.float32, y: torch.Tensor = None,
          acc_out: torch.Tensor = None):
    """Batch-1 quantized GEMV (qg_qgemv). Returns y."""
    _dev(x, "x", (torch.float32, torch.bfloat16))
    if y is None:
        y = torch.empty(w.n, dtype=y_dtype, device=x.device)
    _dev(y, "y", (torch.float32, torch.bfloat16))
    if acc_out is not None:
        _dev(acc_out, "acc_out", torch.int32)
    cw = w.c_struct()
    _check(lib().qg_qgemv(ctypes.byref(cw), QG_ACT_INT8 if act_int8 else QG_ACT_FLOAT, _p(x), _xt(x), _p(y), _xt(y),
                          _p(acc_out), _stream(x)), "qg_qgemv")
    return y


class GroupLaunch:
    """Pre-marshalled arguments of one qg_qgemv_grouped call (kept alive by
    this object); launch() enqueues it on the current stream."""

    def __init__(self, weights: Sequence[QWeight], x: torch.Tensor, ys: Sequence[torch.Tensor], act_int8: bool,
                 accs: Optional[Sequence[torch.Tensor]] = None):
        _dev(x, "x", (torch.float32, torch.bfloat16))
        n = len(weights)
        if not 1 <= n <= QG_MAX_GROUP or len(ys) != n:
            raise ValueError("need 1..%d weights and as many outputs" % QG_MAX_GROUP)
        for y in ys:
            _dev(y, "y", (torch.float32, torch.bfloat16))
        self.x, self.ys, self.accs = x, list(ys), accs
        self.cw = (CWeight * n)(*[w.c_struct() for w in weights])
        self.yp = (_c_vp * n)(*[y.data_ptr() for y in ys])
        self.ap = None if accs is None else (_c_vp * n)(*[None if a is None else a.data_ptr() for a in accs])
        self.n = n
        self.amode = QG_ACT_INT8 if act_int8 else QG_ACT_FLOAT
        self.xt = _xt(x)
        self.yt = _xt(ys[0])

    def launch(self):
        _check(lib().qg_qgemv_grouped(self.cw, self.n, self.amode, _p(self.x), self.xt, self.yp, self.yt, self.ap,
                                      _stream(self.x)), "qg_qgemv_grouped")


def qgemv_grouped(weights: Sequence[QWeight], x: torch.Tensor, act_int8: bool, y_dtype=torch.float32,
                  accs: Optional[Sequence[torch.Tensor]] = None):
    """Several GEMVs on the same x in one launch (qg_qgemv_grouped). Returns [y]."""
    ys = [torch.empty(w.n, dtype=y_dtype, device=x.device) for w in weights]
    GroupLaunch(weights, x, ys, act_int8, accs).launch()
    return ys


def qgemv_launch_raw(cw: CWeight, amode: int, x_ptr: int, xt: int, y_ptr: int, yt: int, stream_ptr: int) -> int:
    """Pre-marshalled launch for tight timing loops (returns the status)."""
    return lib().qg_qgemv(ctypes.byref(cw), amode, ctypes.c_void_p(x_ptr), xt, ctypes.c_void_p(y_ptr), yt, None,
                          ctypes.c_void_p(stream_ptr))


def qgemm_w8a8_outlier(x: torch.Tensor, idx: Sequence[int], wq: torch.Tensor, s_w: torch.Tensor,
                       w_out: Optional[torch.Tensor], y: torch.Tensor = None, acc_out: torch.Tensor = None,
                       ws: torch.Tensor = None):
    """W8A8 prefill GEMM with the outlier split (qg_qgemm_w8a8_outlier). Returns y."""
    _dev(x, "x", torch.bfloat16)
    _dev(wq, "wq", torch.int8)
    _dev(s_w, "s_w", torch.float32)
    m, k = x.shape
    n = wq.shape[0]
    cidx, n_out = _idx_host(idx)
    w_ld = 0
    if n_out:
        _dev(w_out, "w_out", torch.bfloat16)
        w_ld = w_out.shape[1]
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=x.device)
    nws = lib().qg_qgemm_workspace_bytes(m, k, n_out)
    if ws is None:
        ws = torch.empty(nws, dtype=torch.uint8, device=x.device)
    _check(lib().qg_qgemm_w8a8_outlier(_p(x), m, k, cidx, n_out, _p(wq), _p(s_w), _p(w_out) if n_out else None, w_ld,
                                       n, _p(y), _p(acc_out), _p(ws), ws.numel(), _stream(x)), "qg_qgemm_w8a8_outlier")
    return y


def qgemm_w8a8(xq: torch.Tensor, s_x: torch.Tensor, x_out: Optional[torch.Tensor], wq: torch.Tensor,
               s_w: torch.Tensor, w_out: Optional[torch.Tensor], n_out: int, y: torch.Tensor = None,
               acc_out: torch.Tensor = None):
    """The GEMM half of the prefill on already split activations (qg_qgemm_w8a8):
    xq [m][k] int8, s_x [m], x_out [m][x_ld] bf16 and w_out [n][w_ld] bf16 (as
    quantize_absmax_split / gather_columns_bf16 return them), n_out outlier
    channels. Returns y [m][n] fp32."""
    _dev(xq, "xq", torch.int8)
    _dev(s_x, "s_x", torch.float32)
    _dev(wq, "wq", torch.int8)
    _dev(s_w, "s_w", torch.float32)
    m, k = xq.shape
    n = wq.shape[0]
    x_ld = w_ld = 0
    if n_out:
        _dev(x_out, "x_out", torch.bfloat16)
        _dev(w_out, "w_out", torch.bfloat16)
        x_ld, w_ld = x_out.shape[1], w_out.shape[1]
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=xq.device)
    _check(lib().qg_qgemm_w8a8(_p(xq), _p(s_x), _p(x_out) if n_out else None, x_ld, m, k, n_out, _p(wq), _p(s_w),
                               _p(w_out) if n_out else None, w_ld, n, _p(y), _p(acc_out), _stream(xq)),
           "qg_qgemm_w8a8")
    return y


def chain_plan_image(stages, workgroups: int):
    """qg_chain_plan on the host: `stages` is a list of (CWeight array, count,
    x pointer, y pointer array, dep).  Returns the 16-B aligned uint8 image
    (a numpy view) and the status; nothing is sent to a device."""
    import numpy as np
    n = len(stages)
    cs = (CChainStage * n)()
    for i, (cw, count, x_ptr, yp, dep) in enumerate(stages):
        cs[i].count, cs[i].dep, cs[i].x = count, dep, x_ptr
        cs[i].w = ctypes.cast(cw, ctypes.POINTER(CWeight))
        cs[i].y = ctypes.cast(yp, ctypes.POINTER(_c_vp))
    nbytes = lib().qg_chain_plan_bytes(cs, n, workgroups)
    raw = np.zeros(max(int(nbytes), 64) + 16, np.uint8)
    off = (-raw.ctypes.data) % 16
    img = raw[off:off + max(int(nbytes), 64)]
    st = lib().qg_chain_plan(cs, n, workgroups, ctypes.c_void_p(img.ctypes.data), nbytes)
    return img, st


class ChainStep:
    """The weight-only int8 products of a decode step with their data
    dependencies, run as one launch (qg_chain_plan once, then qg_qgemv_chain
    per call).

    stages: list of (weights, x, ys, dep): weights a list of QG_WFMT_INT8
    QWeights sharing k, x a bf16 tensor [k], ys bf16 tensors [n] (one per
    weight), dep the index of the stage whose outputs x holds (-1: none)."""

    def __init__(self, stages, workgroups: Optional[int] = None):
        self.keep = []
        plan = []
        dev = None
        for weights, x, ys, dep in stages:
            _dev(x, "x", torch.bfloat16)
            dev = x.device
            for y in ys:
                _dev(y, "y", torch.bfloat16)
            cw = (CWeight * len(weights))(*[w.c_struct() for w in weights])
            yp = (_c_vp * len(ys))(*[y.data_ptr() for y in ys])
            self.keep += [cw, yp, x, list(ys), list(weights)]
            plan.append((cw, len(weights), x.data_ptr(), yp, dep))
        if workgroups is None:
            workgroups = torch.cuda.get_device_properties(dev).multi_processor_count
        self.image, st = chain_plan_image(plan, workgroups)
        _check(st, "qg_chain_plan")
        self.plan = torch.from_numpy(self.image.copy()).to(dev)
        self.device = dev

    def launch(self):
        _check(lib().qg_qgemv_chain(ctypes.c_void_p(self.image.ctypes.data), _p(self.plan), _stream(self.plan)),
               "qg_qgemv_chain")

    def error(self) -> int:
        """The plan's error word (nonzero: a wait ran past its time bound)."""
        return int(self.plan[QG_CHAIN_ERROR_OFFSET:QG_CHAIN_ERROR_OFFSET + 4].view(torch.int32).item())

    def restore(self):
        """Copy the plan image to the device again (after an error)."""
        self.plan.copy_(torch.from_numpy(self.image))
