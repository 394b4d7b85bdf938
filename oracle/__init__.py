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
* :func:`i4x2_to_e2m3`     -- the same int4 codes stored in 6-bit E2M3 fields,
  K-blocked (the storage a 6-bit matrix unit reads).
* :func:`sqf_row`, :func:`pack_weights_sqf`, :func:`dual_gemm_sqf` -- the
  floating-point weight-side SQ-format (FP4 E2M1 low part with the 0x8 mark,
  FP8 E4M3 sparse values; SQ-format article, section 八).
* :func:`rmsnorm`, :func:`rmsnorm_quantize_split_act` -- the norm in front
  of the split, and the two composed; :func:`slot_order` -- the channel
  order that turns the split into a slice (SQ-format article, section 九).
* :func:`pack_weights_mx`, :func:`quantize_split_act_mx`, :func:`dual_gemm_mx`
  -- the MXFP4 low path (OCP Microscaling: E2M1 elements, one E8M0 scale
  per 32 slots; OSC abstract, 4-bit micro-scaling hardware), and
  :func:`mx_storage`, the K-blocked storage of those rows.
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


# AddressSanitizer + UndefinedBehaviorSanitizer build of the same source
# (tests/test_sanitizers.py runs the oracle's pins against it, with gcc's
# libasan preloaded into the interpreter)
SAN_LIB = os.path.join(HERE, "liboracle_san.so")
SAN_CFLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
              "-fno-sanitize-recover=undefined", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
              "-fPIC", "-shared", "-std=c11"]


def build(force: bool = True, sanitize: bool = False) -> str:
    """Compile liboracle.so with gcc (scalar C, no fast-math, no contraction);
    ``sanitize`` builds liboracle_san.so with ASan and UBSan instead."""
    lib, flags = (SAN_LIB, SAN_CFLAGS) if sanitize else (LIB, CFLAGS)
    if force or not os.path.exists(lib) or os.path.getmtime(lib) < os.path.getmtime(SRC):
        tmp = lib + ".tmp"
        subprocess.check_call(["gcc", *flags, SRC, "-o", tmp, "-lm"])
        os.replace(tmp, lib)
    return lib


_lib = None


def _load():
    global _lib
    if _lib is None:
        # SQF_ORACLE_LIBRARY (read once, at the first call) names another
        # build of this source, e.g. the sanitizer build
        path = os.environ.get("SQF_ORACLE_LIBRARY") or LIB
        if path == LIB and not os.path.exists(LIB):
            build(force=True)
        _lib = ctypes.CDLL(path)
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
    lib.orc_sq_row.argtypes = [P, P, I64, I64, I64, INT, P, P, P, P]
    lib.orc_sq_row.restype = None
    lib.orc_pack_weights_sq.argtypes = [P, I64, I64, P, P, I64, I64, I64, I64, I64, I64, P, P, P, P,
                                        P, P]
    lib.orc_pack_weights_sq.restype = None
    lib.orc_e2m3_field_of_code.argtypes = [INT]
    lib.orc_e2m3_field_of_code.restype = ctypes.c_uint8
    lib.orc_i4x2_to_e2m3.argtypes = [P, I64, I64, I64, P]
    lib.orc_i4x2_to_e2m3.restype = None
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
    lib.orc_e2m1_to_double.argtypes = [ctypes.c_uint8]
    lib.orc_e2m1_to_double.restype = ctypes.c_double
    lib.orc_e2m1_from_double.argtypes = [ctypes.c_double]
    lib.orc_e2m1_from_double.restype = ctypes.c_uint8
    lib.orc_mx_block.argtypes = [P, I64, P]
    lib.orc_mx_block.restype = ctypes.c_uint8
    lib.orc_pack_weights_mx.argtypes = [P, I64, I64, P, I64, I64, I64, I64, P, P, P]
    lib.orc_pack_weights_mx.restype = None
    lib.orc_quantize_split_act_mx.argtypes = [P, INT, I64, I64, I64, P, I64, I64, I64, I64, P, P, P]
    lib.orc_quantize_split_act_mx.restype = None
    lib.orc_mx_storage.argtypes = [P, P, I64, I64, I64, P, P]
    lib.orc_mx_storage.restype = None
    lib.orc_dual_gemm_mx.argtypes = [I64, I64, I64, I64, P, I64, P, P, P, I64, P, P, P, P, I64]
    lib.orc_dual_gemm_mx.restype = None
    lib.orc_rmsnorm.argtypes = [P, INT, I64, I64, I64, P, ctypes.c_float, P]
    lib.orc_rmsnorm.restype = None
    lib.orc_slot_order.argtypes = [P, I64, P, P]
    lib.orc_slot_order.restype = None
    lib.orc_sqf_row.argtypes = [P, P, I64, I64, I64, P, P, P, P]
    lib.orc_sqf_row.restype = None
    lib.orc_pack_weights_sqf.argtypes = [P, I64, I64, P, P, I64, I64, I64, I64, I64, I64, P, P, P, P,
                                         P, P]
    lib.orc_pack_weights_sqf.restype = None
    lib.orc_dual_gemm_sqf.argtypes = [I64, I64, I64, P, I64, P, I64, P, P, I64, P, P, I64, P, I64, P,
                                      P, P, P, P, I64]
    lib.orc_dual_gemm_sqf.restype = None
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


def e2m3_field_of_code(code: int) -> int:
    return int(_load().orc_e2m3_field_of_code(int(code)))


def pad_rows(rows: int) -> int:
    """Row count of the K-blocked 6-bit layout: rows rounded up to 256."""
    return -(-rows // 256) * 256


def i4x2_to_e2m3(packed: np.ndarray, rows_pad: int | None = None) -> np.ndarray:
    """Packed int4 rows [rows][ldk] -> the K-blocked E2M3 storage holding the
    same codes, shaped [2*ldk/128][rows_pad/32][3072] (K block, pair of
    16-row groups, the pair's two head KiB and tail KiB; see orc_i4x2_to_e2m3)."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    rows, ldk = packed.shape
    rp = pad_rows(rows) if rows_pad is None else rows_pad
    out = np.zeros((2 * ldk // 128, rp // 32, 3072), dtype=np.uint8)
    if rows and ldk:
        _load().orc_i4x2_to_e2m3(_p(packed), rows, ldk, rp, _p(out))
    return out


def e2m3_group(storage: np.ndarray, r: int, kb: int, g: int) -> np.ndarray:
    """The 24 bytes (32 six-bit fields) of slot group g of K block kb of row r
    in the K-blocked E2M3 storage (the layout's position formula)."""
    lane, h = g * 16 + r % 16, (r // 16) % 2
    blk = storage[kb, r // 32]
    return np.concatenate([blk[h * 1024 + lane * 16: h * 1024 + lane * 16 + 16],
                           blk[2048 + lane * 16 + 8 * h: 2048 + lane * 16 + 8 * h + 8]])


def e2m3_row_of_byte(nkb: int, rows_pad: int) -> np.ndarray:
    """For every byte of the K-blocked E2M3 storage, the row it belongs to."""
    o = np.arange(3072)
    row = np.empty(3072, np.int64)
    head = o < 2048
    h_head = o // 1024
    lane_head = (o % 1024) // 16
    row[head] = h_head[head] * 16 + lane_head[head] % 16
    lane_tail = (o - 2048) // 16
    h_tail = ((o - 2048) % 16) // 8
    row[~head] = h_tail[~head] * 16 + lane_tail[~head] % 16
    rows = (np.arange(rows_pad // 32) * 32)[:, None] + row[None, :]
    return np.broadcast_to(rows, (nkb, rows_pad // 32, 3072))


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


def _check_bank(k_low: int, nnz: int, bank: int) -> int:
    if bank <= 0 or bank >= k_low:
        return 0
    if k_low % bank or nnz % (k_low // bank):
        raise ValueError(f"bank {bank} must divide k_low {k_low} and the bank count nnz {nnz}")
    return bank


def sq_row(wrow: np.ndarray, hdiag: np.ndarray, nnz: int, bits: int = 4, bank: int = 0):
    """One weight-side SQ-format row -> (fields u8 [k_low], v8 i8 [nnz], s8, s_low).
    ``bank`` > 0: banks of that many slots, nnz / banks marks in each."""
    wrow = np.ascontiguousarray(wrow, dtype=np.float32)
    hdiag = np.ascontiguousarray(hdiag, dtype=np.float32)
    k_low = len(wrow)
    fields = np.zeros(max(k_low, 1), dtype=np.uint8)
    v8 = np.zeros(max(nnz, 1), dtype=np.int8)
    s8 = np.zeros(1, dtype=np.float32)
    sl = np.zeros(1, dtype=np.float32)
    bank = _check_bank(k_low, nnz, bank)
    _load().orc_sq_row(_p(wrow), _p(hdiag), k_low, nnz, bank, bits, _p(fields), _p(v8), _p(s8),
                       _p(sl))
    return fields[:k_low], v8[:nnz], s8[0], sl[0]


def pack_weights_sq(w: np.ndarray, mp: np.ndarray, hdiag: np.ndarray, nnz: int, bank: int = 0):
    """Weight-side SQ-format with an int8 branch over the outlier channels
    (``bank`` > 0: banks of that many slots with an equal count of marks)."""
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
    bank = _check_bank(k_low, nnz, bank)
    _load().orc_pack_weights_sq(_p(w), k, n, _p(mp), _p(hdiag), k_low, k_out, ldk, ldo, nnz, bank,
                                _p(w_low), _p(s_w4), _p(sq_val), _p(s_w8),
                                _p(w_out) if ldo else None, _p(s_wo))
    return dict(w_low=w_low, s_w=s_w4, sq_val=sq_val[:, :nnz].copy(), s_w8=s_w8, w_out=w_out,
                s_wo=s_wo, k_low=k_low, k_out=k_out, ldk=ldk, ldo=ldo, branch="i8", sq_nnz=nnz,
                sq_bank=bank)


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
    # The integer sums are exact in int64 here; the GPU keeps them in int32.
    # Their worst case |acc| is the code range product times the length.
    qx = 7 if a["low"] == "i4" else 127
    worst = max(qx * 7 * a["k_low"], qx * 127 * sq,
                127 * 127 * a["k_out"] if a["branch"] == "i8" else 0)
    if worst >= 2 ** 31:
        raise ValueError(f"integer accumulators may exceed int32 (worst case {worst})")
    _load().orc_dual_gemm(
        n, a["k_low"], a["k_out"], _p(rows), nr,
        _p(a["x_low"]) if a["x_low"].size else None, a["ldk"], _FMT[a["low"]], _p(a["s_x"]),
        _p(a["x_out"]) if a["x_out"].size else None, a["ldo"], _FMT[a["branch"]], _p(a["s_xo"]),
        _p(w["w_low"]) if w["w_low"].size else None, w["ldk"], _p(w["s_w"]),
        _p(w["w_out"]) if w["w_out"].size else None, _p(w["s_wo"]),
        sq, _p(w["sq_val"]) if sq else None, _p(w["s_w8"]) if sq else None,
        _p(y), n, _p(dbg[0]), _p(dbg[1]), _p(dbg[2]))
    if debug:
        for d in dbg:
            assert np.abs(d).max(initial=0) < 2 ** 31
        return y, dbg[0], dbg[1], dbg[2]
    return y


# ---------------------------------------------------------------- MXFP4 low path
def e2m1_to_float(c: int) -> float:
    """Value of a 4-bit OCP E2M1 code."""
    return float(_load().orc_e2m1_to_double(int(c) & 0xF))


def e2m1_from_float(t: float) -> int:
    """Nearest E2M1 code (ties to mantissa bit 0, saturating at +-6)."""
    return int(_load().orc_e2m1_from_double(float(t)))


def mx_block(v: np.ndarray):
    """One MX block (<= 32 values) -> (E8M0 scale byte, E2M1 codes u8)."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    codes = np.zeros(max(len(v), 1), dtype=np.uint8)
    b = _load().orc_mx_block(_p(v), len(v), _p(codes))
    return int(b), codes[: len(v)]


def pack_weights_mx(w: np.ndarray, mp: np.ndarray):
    """Weights [k][n] -> dict(w_low u8 [n][pad/2] E2M1 pairs, s_wb u8 [n][pad/32]
    E8M0, w_out u16 [n][ldo] bf16) for the MXFP4 low path."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    mp = np.ascontiguousarray(mp, dtype=np.int32)
    k, n = w.shape
    k_out = int((mp < 0).sum())
    k_low = k - k_out
    pad = pad_k_low(k_low)
    ldo = pad_k_out(k_out, "bf16")
    w_low = np.zeros((n, pad // 2), dtype=np.uint8)
    s_wb = np.zeros((n, pad // 32), dtype=np.uint8)
    w_out = np.zeros((n, ldo), dtype=np.uint16)
    _load().orc_pack_weights_mx(_p(w), k, n, _p(mp), k_low, k_out, pad, ldo,
                                _p(w_low) if pad else None, _p(s_wb) if pad else None,
                                _p(w_out) if ldo else None)
    return dict(w_low=w_low, s_wb=s_wb, w_out=w_out, k_low=k_low, k_out=k_out, pad=pad, ldo=ldo,
                low="mxfp4", branch="bf16")


def quantize_split_act_mx(x: np.ndarray, mp: np.ndarray, x_fmt: str = "f32"):
    """Activations [m][k] -> dict(x_low u8 [m][pad/2], s_xb u8 [m][pad/32],
    x_out u16 [m][ldo] bf16) for the MXFP4 low path."""
    x = np.ascontiguousarray(x)
    mp = np.ascontiguousarray(mp, dtype=np.int32)
    m, k = x.shape
    assert x.dtype == (np.uint16 if x_fmt == "bf16" else np.float32)
    k_out = int((mp < 0).sum())
    k_low = k - k_out
    pad = pad_k_low(k_low)
    ldo = pad_k_out(k_out, "bf16")
    x_low = np.zeros((m, pad // 2), dtype=np.uint8)
    s_xb = np.zeros((m, pad // 32), dtype=np.uint8)
    x_out = np.zeros((m, ldo), dtype=np.uint16)
    _load().orc_quantize_split_act_mx(_p(x), _FMT[x_fmt], m, k, k, _p(mp), k_low, k_out, pad, ldo,
                                      _p(x_low) if pad else None, _p(s_xb) if pad else None,
                                      _p(x_out) if ldo else None)
    return dict(x_low=x_low, s_xb=s_xb, x_out=x_out, k_low=k_low, k_out=k_out, pad=pad, ldo=ldo,
                low="mxfp4", branch="bf16")


def mx_storage(codes: np.ndarray, scales: np.ndarray, rows_pad: int | None = None):
    """MXFP4 rows (codes [rows][pad/2], scales [rows][pad/32]) -> the K-blocked
    storage: codes [pad/128][rows_pad/16][4][16][16], scales
    [pad/128][rows_pad/64][4][16][4] (see orc_mx_storage)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    rows, half = codes.shape
    pad = 2 * half
    assert scales.shape == (rows, pad // 32)
    rp = pad_rows(rows) if rows_pad is None else rows_pad
    c = np.zeros((pad // 128, rp // 16, 4, 16, 16), dtype=np.uint8)
    sc = np.zeros((pad // 128, rp // 64, 4, 16, 4), dtype=np.uint8)
    if rows and pad:
        _load().orc_mx_storage(_p(codes), _p(scales), rows, pad, rp, _p(c), _p(sc))
    return c, sc


def dual_gemm_mx(a: dict, w: dict, rows=None):
    """Y rows of the MXFP4 dual GEMM for token indices ``rows`` (default all)."""
    m = a["x_low"].shape[0] if a["x_low"].size else a["x_out"].shape[0]
    if rows is None:
        rows = np.arange(m, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    n = w["w_low"].shape[0] if w["w_low"].size else w["w_out"].shape[0]
    assert a["k_low"] == w["k_low"] and a["k_out"] == w["k_out"] and a["pad"] == w["pad"]
    y = np.zeros((len(rows), n), dtype=np.float32)
    _load().orc_dual_gemm_mx(n, a["k_low"], a["k_out"], a["pad"], _p(rows), len(rows),
                             _p(a["x_low"]) if a["x_low"].size else None,
                             _p(a["s_xb"]) if a["s_xb"].size else None,
                             _p(a["x_out"]) if a["x_out"].size else None, a["ldo"],
                             _p(w["w_low"]) if w["w_low"].size else None,
                             _p(w["s_wb"]) if w["s_wb"].size else None,
                             _p(w["w_out"]) if w["w_out"].size else None, _p(y), n)
    return y


# ---------------------------------------------------------------- producer side
def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float, x_fmt: str = "f32") -> np.ndarray:
    """RMS normalisation of each row -> fp32 [m][k] (see orc_rmsnorm)."""
    x = np.ascontiguousarray(x)
    assert x.dtype == (np.uint16 if x_fmt == "bf16" else np.float32)
    gamma = np.ascontiguousarray(gamma, dtype=np.float32)
    m, k = x.shape
    out = np.zeros((m, k), np.float32)
    if m:
        _load().orc_rmsnorm(_p(x), _FMT[x_fmt], m, k, k, _p(gamma), float(eps), _p(out))
    return out


def rmsnorm_quantize_split_act(x, gamma, eps, mp, low="i4", branch="bf16", x_fmt="f32"):
    """The split of the normalised rows: quantize_split_act(rmsnorm(x))."""
    return quantize_split_act(rmsnorm(x, gamma, eps, x_fmt), mp, low=low, branch=branch, x_fmt="f32")


def slot_order(mp: np.ndarray):
    """(perm, slice_map): position p of the reordered channel axis holds
    channel perm[p] (low channels in slot order, then the outliers); the
    consumer's map on that axis is slice_map."""
    mp = np.ascontiguousarray(mp, dtype=np.int32)
    perm = np.zeros(len(mp), np.int32)
    sm = np.zeros(len(mp), np.int32)
    _load().orc_slot_order(_p(mp), len(mp), _p(perm), _p(sm))
    return perm, sm


# ---------------------------------------------------------------- FP8/FP4 SQ-format
def sqf_row(wrow: np.ndarray, hdiag: np.ndarray, nnz: int, bank: int = 0):
    """One floating-point SQ-format row -> (fields u8 [k_low] (E2M1, 0x8 =
    mark), v8 u8 [nnz] (E4M3), s8, s4)."""
    wrow = np.ascontiguousarray(wrow, dtype=np.float32)
    hdiag = np.ascontiguousarray(hdiag, dtype=np.float32)
    k_low = len(wrow)
    bank = _check_bank(k_low, nnz, bank)
    fields = np.zeros(max(k_low, 1), np.uint8)
    v8 = np.zeros(max(nnz, 1), np.uint8)
    s8 = np.zeros(1, np.float32)
    s4 = np.zeros(1, np.float32)
    _load().orc_sqf_row(_p(wrow), _p(hdiag), k_low, nnz, bank, _p(fields), _p(v8), _p(s8), _p(s4))
    return fields[:k_low], v8[:nnz], s8[0], s4[0]


def pack_weights_sqf(w: np.ndarray, mp: np.ndarray, hdiag: np.ndarray, nnz: int, bank: int = 0):
    """Floating-point SQ-format weights with an E4M3 branch over the outlier channels."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    mp = np.ascontiguousarray(mp, dtype=np.int32)
    hdiag = np.ascontiguousarray(hdiag, dtype=np.float32)
    k, n = w.shape
    k_out = int((mp < 0).sum())
    k_low = k - k_out
    bank = _check_bank(k_low, nnz, bank)
    ldk = pad_k_low(k_low) // 2
    ldo = pad_k_out(k_out, "fp8")
    w_low = np.zeros((n, ldk), np.uint8)
    s_w4 = np.zeros(n, np.float32)
    sq_val = np.zeros((n, max(nnz, 1)), np.uint8)
    s_w8 = np.zeros(n, np.float32)
    w_out = np.zeros((n, ldo), np.uint8)
    s_wo = np.zeros(n, np.float32)
    _load().orc_pack_weights_sqf(_p(w), k, n, _p(mp), _p(hdiag), k_low, k_out, ldk, ldo, nnz, bank,
                                 _p(w_low), _p(s_w4), _p(sq_val), _p(s_w8),
                                 _p(w_out) if ldo else None, _p(s_wo))
    return dict(w_low=w_low, s_w=s_w4, sq_val=sq_val[:, :nnz].copy(), s_w8=s_w8, w_out=w_out,
                s_wo=s_wo, k_low=k_low, k_out=k_out, ldk=ldk, ldo=ldo, branch="fp8", sq_nnz=nnz,
                sq_bank=bank, low="fp4")


def dual_gemm_sqf(a: dict, w: dict, rows=None):
    """Y of the floating-point SQ-format (activations from
    quantize_split_act(..., low="fp8", branch="fp8"))."""
    assert a["low"] == "fp8" and a["branch"] == "fp8" and w["branch"] == "fp8"
    m = a["x_low"].shape[0] if a["x_low"].size else a["x_out"].shape[0]
    if rows is None:
        rows = np.arange(m, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    n = w["s_w"].shape[0]
    assert a["k_low"] == w["k_low"] and a["k_out"] == w["k_out"]
    y = np.zeros((len(rows), n), np.float32)
    nnz = w["sq_nnz"]
    _load().orc_dual_gemm_sqf(n, a["k_low"], a["k_out"], _p(rows), len(rows),
                              _p(a["x_low"]) if a["x_low"].size else None, a["ldk"], _p(a["s_x"]),
                              _p(a["x_out"]) if a["x_out"].size else None, a["ldo"], _p(a["s_xo"]),
                              _p(w["w_low"]) if w["w_low"].size else None, w["ldk"], _p(w["s_w"]),
                              nnz, _p(w["sq_val"]) if nnz else None, _p(w["s_w8"]),
                              _p(w["w_out"]) if w["w_out"].size else None, _p(w["s_wo"]), _p(y), n)
    return y
