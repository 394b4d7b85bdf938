"""CPU oracle for the outlier-separated dual-path GEMM.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this package.  It is a thin numpy
wrapper over ``sqf_oracle.c`` (plain scalar loops, see that file for the
method steps and the page each one follows); it shares no code with the GPU
library and never calls it.

All arrays are numpy arrays in host memory.  Functions mirror the steps of
the method:

* :func:`select_channels`  -- static outlier-channel choice from calibration
  data (SQ-format article, sections 二/五; OSC abstract).
* :func:`pack_weights`     -- int4 low part + high-precision branch rows.
* :func:`pack_weights_sq`  -- weight-side SQ-format (int4 with a reserved
  mark + int8 sparse values) (SQ-format article, section 九).
* :func:`quantize_split_act` -- per-token int4/int8 quantisation plus the
  outlier sub-tensor gather (OSC abstract).
* :func:`dual_gemm`        -- low path + masked path + branch + fused output.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "sqf_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-std=c11"]

F32, BF16, FP8, I8, I4 = 0, 1, 2, 3, 4
_FMT = {"f32": F32, "bf16": BF16, "fp8": FP8, "i8": I8, "i4": I4}

K_ALIGN_LOW = 256  # low slots are padded to a multiple of this
K_ALIGN_OUT_BYTES = 128  # branch rows are padded to a multiple of 128 bytes


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (scalar C, no fast-math, no contraction)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"])
        os.replace(tmp, LIB)
    return LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build(force=True)
        _lib = ctypes.CDLL(LIB)
        _declare(_lib)
    return _lib


P = ctypes.c_void_p
I64 = ctypes.c_int64
INT = ctypes.c_int


def _declare(lib):
    lib.orc_select_channels.argtypes = [P, I64, I64, P, I64, I64, P, P, P, P]
    lib.orc_select_channels.restype = None
    lib.orc_quantize_vec.argtypes = [P, I64, INT, P]
    lib.orc_quantize_vec.restype = ctypes.c_float
    lib.orc_pack_weights.argtypes = [P, I64, I64, P, I64, I64, I64, I64, INT, P, P, P, P]
    lib.orc_pack_weights.restype = None
    lib.orc_sq_row.argtypes = [P, P, I64, I64, INT, P, P, P, P]
    lib.orc_sq_row.restype = None
    lib.orc_pack_weights_sq.argtypes = [P, I64, I64, P, P, I64, I64, I64, I64, I64, P, P, P, P, P, P]
    lib.orc_pack_weights_sq.restype = None
    lib.orc_quantize_split_act.argtypes = [P, INT, I64, I64, I64, P, I64, I64, I64, I64, INT, INT,
                                           P, P, P, P]
    lib.orc_quantize_split_act.restype = None
    lib.orc_dual_gemm.argtypes = [I64, I64, I64, P, I64, P, I64, INT, P, P, I64, INT, P, P, I64, P,
                                  P, P, I64, P, P, P, I64, P, P, P]
    lib.orc_dual_gemm.restype = None
    lib.orc_bf16_from_float.argtypes = [ctypes.c_float]
    lib.orc_bf16_from_float.restype = ctypes.c_uint16
    lib.orc_e4m3_from_float.argtypes = [ctypes.c_float]
    lib.orc_e4m3_from_float.restype = ctypes.c_uint8
    lib.orc_e4m3_to_double.argtypes = [ctypes.c_uint8]
    lib.orc_e4m3_to_double.restype = ctypes.c_double
    lib.orc_num_threads.argtypes = []
    lib.orc_num_threads.restype = ctypes.c_int


def _p(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return ctypes.c_void_p(a.ctypes.data)


def pad_k_low(k_low: int) -> int:
    return -(-k_low // K_ALIGN_LOW) * K_ALIGN_LOW


def pad_k_out(k_out: int, branch: str = "bf16") -> int:
    step = K_ALIGN_OUT_BYTES // (2 if branch == "bf16" else 1)
    return -(-k_out // step) * step


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().orc_num_threads())


# ---------------------------------------------------------------- formats
def bf16_from_float(v: float) -> int:
    return int(_load().orc_bf16_from_float(float(v)))


def e4m3_from_float(v: float) -> int:
    return int(_load().orc_e4m3_from_float(float(v)))


def e4m3_to_float(c: int) -> float:
    return float(_load().orc_e4m3_to_double(int(c) & 0xFF))


def quantize_vec(v: np.ndarray, fmt: str):
    """Symmetric per-vector quantisation; returns (codes int32, scale float32)."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    codes = np.zeros(max(len(v), 1), dtype=np.int32)
    s = _load().orc_quantize_vec(_p(v), len(v), _FMT[fmt], _p(codes))
    return codes[: len(v)], np.float32(s)


# ---------------------------------------------------------------- steps
def select_channels(x_cal: np.ndarray, w: np.ndarray, k_out: int):
    """Return (idx[k_out] int32 ascending, map[k] int32, score[k] f64, hdiag[k] f32)."""
    x_cal = np.ascontiguousarray(x_cal, dtype=np.float32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    m_cal, k = x_cal.shape
    k2, n = w.shape
    assert k == k2 and 0 <= k_out <= k
    idx = np.zeros(max(k_out, 1), dtype=np.int32)
    mp = np.zeros(k, dtype=np.int32)
    score = np.zeros(k, dtype=np.float64)
    hdiag = np.zeros(k, dtype=np.float32)
    _load().orc_select_channels(_p(x_cal), m_cal, k, _p(w), n, k_out, _p(idx), _p(mp), _p(score),
                                _p(hdiag))
    return idx[:k_out].copy(), mp, score, hdiag


def _branch_dtype(fmt: str):
    return np.uint16 if fmt == "bf16" else np.uint8


def pack_weights(w: np.ndarray, mp: np.ndarray, branch: str = "bf16"):
    """Weights [k][n] -> dict(w_low u8 [n][ldk], s_w f32 [n], w_out [n][ldo], s_wo f32 [n])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    mp = np.ascontiguousarray(mp, dtype=np.int32)
    k, n = w.shape
    k_out = int((mp < 0).sum())
    k_low = k - k_out
    ldk = pad_k_low(k_low) // 2
    ldo = pad_k_out(k_out, branch)
    w_low = np.zeros((n, max(ldk, 1)), dtype=np.uint8)[:, :ldk].copy()
    s_w = np.zeros(n, dtype=np.float32)
    w_out = np.zeros((n, ldo), dtype=_branch_dtype(branch))
    s_wo = np.zeros(n, dtype=np.float32)
    _load().orc_pack_weights(_p(w), k, n, _p(mp), k_low, k_out, ldk, ldo, _FMT[branch],
                             _p(w_low) if ldk else None, _p(s_w), _p(w_out) if ldo else None,
                             _p(s_wo))
    return dict(w_low=w_low, s_w=s_w, w_out=w_out, s_wo=s_wo, k_low=k_low, k_out=k_out, ldk=ldk,
                ldo=ldo, branch=branch, sq_nnz=0)


def sq_row(wrow: np.ndarray, hdiag: np.ndarray, nnz: int, bits: int = 4):
    """One weight-side SQ-format row -> (fields u8 [k_low], v8 i8 [nnz], s8, s_low)."""
    wrow = np.ascontiguousarray(wrow, dtype=np.float32)
    hdiag = np.ascontiguousarray(hdiag, dtype=np.float32)
    k_low = len(wrow)
    fields = np.zeros(max(k_low, 1), dtype=np.uint8)
    v8 = np.zeros(max(nnz, 1), dtype=np.int8)
    s8 = np.zeros(1, dtype=np.float32)
    sl = np.zeros(1, dtype=np.float32)
    _load().orc_sq_row(_p(wrow), _p(hdiag), k_low, nnz, bits, _p(fields), _p(v8), _p(s8), _p(sl))
    return fields[:k_low], v8[:nnz], s8[0], sl[0]


def pack_weights_sq(w: np.ndarray, mp: np.ndarray, hdiag: np.ndarray, nnz: int):
    """Weight-side SQ-format with an int8 branch over the outlier channels."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    mp = np.ascontiguousarray(mp, dtype=np.int32)
    hdiag = np.ascontiguousarray(hdiag, dtype=np.float32)
    k, n = w.shape
    k_out = int((mp < 0).sum())
    k_low = k - k_out
    ldk = pad_k_low(k_low) // 2
    ldo = pad_k_out(k_out, "i8")
    w_low = np.zeros((n, ldk), dtype=np.uint8)
    s_w4 = np.zeros(n, dtype=np.float32)
    sq_val = np.zeros((n, max(nnz, 1)), dtype=np.int8)
    s_w8 = np.zeros(n, dtype=np.float32)
    w_out = np.zeros((n, ldo), dtype=np.int8)
    s_wo = np.zeros(n, dtype=np.float32)
    _load().orc_pack_weights_sq(_p(w), k, n, _p(mp), _p(hdiag), k_low, k_out, ldk, ldo, nnz,
                                _p(w_low), _p(s_w4), _p(sq_val), _p(s_w8),
                                _p(w_out) if ldo else None, _p(s_wo))
    return dict(w_low=w_low, s_w=s_w4, sq_val=sq_val[:, :nnz].copy(), s_w8=s_w8, w_out=w_out,
                s_wo=s_wo, k_low=k_low, k_out=k_out, ldk=ldk, ldo=ldo, branch="i8", sq_nnz=nnz)


def quantize_split_act(x: np.ndarray, mp: np.ndarray, low: str = "i4", branch: str = "bf16",
                       x_fmt: str = "f32"):
    """Activations [m][k] (fp32 array, or uint16 bf16 patterns with x_fmt='bf16')."""
    x = np.ascontiguousarray(x)
    mp = np.ascontiguousarray(mp, dtype=np.int32)
    m, k = x.shape
    if x_fmt == "bf16":
        assert x.dtype == np.uint16
    else:
        assert x.dtype == np.float32
    k_out = int((mp < 0).sum())
    k_low = k - k_out
    ldk = pad_k_low(k_low) // (2 if low == "i4" else 1)
    ldo = pad_k_out(k_out, branch)
    x_low = np.zeros((m, ldk), dtype=np.uint8)
    s_x = np.zeros(m, dtype=np.float32)
    x_out = np.zeros((m, ldo), dtype=_branch_dtype(branch))
    s_xo = np.zeros(m, dtype=np.float32)
    _load().orc_quantize_split_act(_p(x), _FMT[x_fmt], m, k, k, _p(mp), k_low, k_out, ldk, ldo,
                                   _FMT[low], _FMT[branch], _p(x_low) if ldk else None, _p(s_x),
                                   _p(x_out) if ldo else None, _p(s_xo))
    return dict(x_low=x_low, s_x=s_x, x_out=x_out, s_xo=s_xo, k_low=k_low, k_out=k_out, ldk=ldk,
                ldo=ldo, low=low, branch=branch)


def dual_gemm(a: dict, w: dict, rows=None, debug: bool = False):
    """Y rows for token indices ``rows`` (default: all).  Returns y [nr][n] f32 and,
    with debug, int64 accumulators (acc_low, acc_sp, acc_o)."""
    m = a["x_low"].shape[0] if a["x_low"].size else a["x_out"].shape[0]
    if rows is None:
        rows = np.arange(m, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    n = w["s_w"].shape[0]
    nr = len(rows)
    y = np.zeros((nr, n), dtype=np.float32)
    dbg = [np.zeros((nr, n), dtype=np.int64) for _ in range(3)] if debug else [None] * 3
    assert a["k_low"] == w["k_low"] and a["k_out"] == w["k_out"] and a["branch"] == w["branch"]
    sq = w.get("sq_nnz", 0)
    _load().orc_dual_gemm(
        n, a["k_low"], a["k_out"], _p(rows), nr,
        _p(a["x_low"]) if a["x_low"].size else None, a["ldk"], _FMT[a["low"]], _p(a["s_x"]),
        _p(a["x_out"]) if a["x_out"].size else None, a["ldo"], _FMT[a["branch"]], _p(a["s_xo"]),
        _p(w["w_low"]) if w["w_low"].size else None, w["ldk"], _p(w["s_w"]),
        _p(w["w_out"]) if w["w_out"].size else None, _p(w["s_wo"]),
        sq, _p(w["sq_val"]) if sq else None, _p(w["s_w8"]) if sq else None,
        _p(y), n, _p(dbg[0]), _p(dbg[1]), _p(dbg[2]))
    if debug:
        return y, dbg[0], dbg[1], dbg[2]
    return y
