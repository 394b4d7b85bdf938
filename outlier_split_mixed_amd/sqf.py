"""Python binding of libsqf (include/sqf.h) over torch device tensors.

Argument marshalling only: each ``sqf_*`` function here has the same name as
the C entry point it calls, takes torch tensors on the GPU, passes their
``data_ptr()`` and the current HIP stream, and raises :class:`SqfError` on a
non-OK status.  All computation happens in the HIP kernels of libsqf.so.
Importing this module loads the library and fails loudly if it is missing.

Helpers ``alloc_weights`` / ``alloc_acts`` create caller-owned buffers with
the layouts the header documents.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# SQF_LIBRARY (read once, at import) names another build of libsqf, e.g. the
# one whose host code carries AddressSanitizer (build.build_host_sanitized)
LIB_PATH = os.environ.get("SQF_LIBRARY") or os.path.join(_HERE, "libsqf.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"libsqf not found at {LIB_PATH}; build it with `python -m outlier_split_mixed_amd.build`")
_lib = ctypes.CDLL(LIB_PATH)

SQF_OK, SQF_ERR_INVALID_ARG, SQF_ERR_SHAPE, SQF_ERR_UNSUPPORTED, SQF_ERR_HIP, SQF_ERR_ALIGN = range(6)
SQF_F32, SQF_BF16, SQF_FP8_E4M3, SQF_I8, SQF_I4X2, SQF_I4_E2M3, SQF_MXFP4, SQF_FP4_E2M1 = range(8)
DTYPES = {"f32": SQF_F32, "bf16": SQF_BF16, "fp8": SQF_FP8_E4M3, "i8": SQF_I8, "i4": SQF_I4X2,
          "i4e2m3": SQF_I4_E2M3, "mxfp4": SQF_MXFP4, "fp4": SQF_FP4_E2M1}
TILES = {"auto": -1, "256": 0, "128": 1, "64": 2}
ABI_VERSION = 6

P = ctypes.c_void_p
I64 = ctypes.c_int64
I32 = ctypes.c_int32


class sqf_weights(ctypes.Structure):
    _fields_ = [("k", I64), ("n", I64), ("k_low", I64), ("k_out", I64), ("ldk", I64),
                ("ldo", I64), ("branch", I32), ("groups", I32), ("low", I32), ("reserved0", I32),
                ("w_low", P), ("s_w", P), ("s_wb", P), ("w_out", P), ("s_wo", P), ("sq_nnz", I64),
                ("sq_bank", I64), ("sq_val", P), ("s_w8", P)]


class sqf_acts(ctypes.Structure):
    _fields_ = [("m", I64), ("k_low", I64), ("k_out", I64), ("ldk", I64), ("ldo", I64),
                ("low", I32), ("branch", I32), ("x_low", P), ("s_x", P), ("s_xb", P), ("x_out", P),
                ("s_xo", P)]


def _decl(name, args, res=ctypes.c_int):
    f = getattr(_lib, name)
    f.argtypes = args
    f.restype = res
    return f


_decl("sqf_abi_version", [], ctypes.c_int)
_decl("sqf_last_error", [], ctypes.c_char_p)
_decl("sqf_pad_k_low", [I64], I64)
_decl("sqf_pad_k_out", [I64, I32], I64)
_decl("sqf_pad_rows", [I64], I64)
_decl("sqf_select_channels", [P, I64, I64, P, I64, I64, P, P, P, P, P])
_decl("sqf_select_channels_noalloc", [P, I64, I64, P, I64, I64, P, P, P, P])
_decl("sqf_pack_weights", [P, P, P, ctypes.POINTER(sqf_weights), P])
_decl("sqf_quantize_split_act", [P, I32, I64, P, ctypes.POINTER(sqf_acts), P])
_decl("sqf_quantize_split_act_grouped", [P, I32, I64, I64, P, P, ctypes.POINTER(sqf_acts), P])
_decl("sqf_rmsnorm_quantize_split_act", [P, I32, I64, P, ctypes.c_float, P, ctypes.POINTER(sqf_acts), P])
_decl("sqf_slot_order", [P, I64, P, P, P])
_decl("sqf_permute_channels", [P, I64, I64, I64, P, I32, P, I64, P])
_decl("sqf_dual_gemm", [ctypes.POINTER(sqf_acts), ctypes.POINTER(sqf_weights), P, I64, P, P, P, P])
_decl("sqf_sq_workspace_bytes", [ctypes.POINTER(sqf_weights)], I64)
_decl("sqf_dual_gemm_sq_ws", [ctypes.POINTER(sqf_acts), ctypes.POINTER(sqf_weights), P, I64, P, I64,
                              P, P, P, P])
_decl("sqf_dual_gemm_grouped", [ctypes.POINTER(sqf_acts), ctypes.POINTER(sqf_weights), I64, P, P,
                                I64, P, P])
_decl("sqf_dual_gemm_y", [ctypes.POINTER(sqf_acts), ctypes.POINTER(sqf_weights), P, I32, I64, P])
_decl("sqf_dual_gemm_grouped_y", [ctypes.POINTER(sqf_acts), ctypes.POINTER(sqf_weights), I64, P, P,
                                  I32, I64, P])
_decl("sqf_dual_gemm_ex", [ctypes.POINTER(sqf_acts), ctypes.POINTER(sqf_weights), P, I32, I64, I32,
                           P, P, P, P])
_decl("sqf_dual_gemm_grouped_ex", [ctypes.POINTER(sqf_acts), ctypes.POINTER(sqf_weights), I64, P,
                                   P, I32, I64, I32, P, P])

if _lib.sqf_abi_version() != ABI_VERSION:
    raise ImportError(f"libsqf ABI {_lib.sqf_abi_version()} != binding ABI {ABI_VERSION}")


class SqfError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"sqf status {status}: {msg}")
        self.status = status


def _check(st: int):
    if st != SQF_OK:
        raise SqfError(st, _lib.sqf_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr()) if t.numel() else None


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def sqf_abi_version() -> int:
    return _lib.sqf_abi_version()


def sqf_last_error() -> str:
    return _lib.sqf_last_error().decode()


def sqf_pad_k_low(k_low: int) -> int:
    return _lib.sqf_pad_k_low(k_low)


def sqf_pad_k_out(k_out: int, branch: str = "bf16") -> int:
    return _lib.sqf_pad_k_out(k_out, DTYPES[branch])


def sqf_pad_rows(rows: int) -> int:
    return _lib.sqf_pad_rows(rows)


def low_ldk(k_low: int, low: str) -> int:
    """Bytes per row of the low operand (see the layouts in sqf.h)."""
    p = sqf_pad_k_low(k_low)
    return {"i4": p // 2, "mxfp4": p // 2, "fp4": p // 2, "i8": p, "fp8": p, "i4e2m3": p * 3 // 4}[low]


def _low_tensor(rows: int, k_low: int, low: str, device, zero: bool):
    """The low operand in its layout: [rows][ldk], or K-blocked with
    P = sqf_pad_rows(rows): 6-bit E2M3 [pad/128][P/32][3072] (pairs of 16-row
    groups), MXFP4 E2M1 pairs [pad/128][P/16][4][16][16]."""
    mk = torch.zeros if zero else torch.empty
    p = sqf_pad_k_low(k_low)
    if low == "i4e2m3":
        return mk((p // 128, sqf_pad_rows(rows) // 32, 3072), dtype=torch.uint8, device=device)
    if low == "mxfp4":
        return mk((p // 128, sqf_pad_rows(rows) // 16, 4, 16, 16), dtype=torch.uint8, device=device)
    return mk((rows, low_ldk(k_low, low)), dtype=torch.uint8, device=device)


def _mx_scales(rows: int, k_low: int, device):
    """MXFP4 E8M0 block scales, K-blocked [pad/128][P/64][4][16][4]."""
    p = sqf_pad_k_low(k_low)
    return torch.zeros((p // 128, sqf_pad_rows(rows) // 64, 4, 16, 4), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------ buffers
_BR_TORCH = {"bf16": torch.int16, "fp8": torch.uint8, "i8": torch.uint8}


@dataclass
class Weights:
    k: int
    n: int
    k_low: int
    k_out: int
    branch: str
    groups: int = 1
    sq_nnz: int = 0
    sq_bank: int = 0
    low: str = "i4"
    t: dict = field(default_factory=dict)

    @property
    def ldk(self):
        return low_ldk(self.k_low, self.low)

    @property
    def ldo(self):
        return sqf_pad_k_out(self.k_out, self.branch) if self.k_out else 0

    def desc(self) -> sqf_weights:
        t = self.t
        return sqf_weights(self.k, self.n, self.k_low, self.k_out, self.ldk, self.ldo,
                           DTYPES[self.branch], self.groups, DTYPES[self.low], 0, _ptr(t["w_low"]),
                           _ptr(t.get("s_w")), _ptr(t.get("s_wb")), _ptr(t["w_out"]),
                           _ptr(t.get("s_wo")), self.sq_nnz, self.sq_bank,
                           _ptr(t.get("sq_val")), _ptr(t.get("s_w8")))


@dataclass
class Acts:
    m: int
    k_low: int
    k_out: int
    low: str
    branch: str
    t: dict = field(default_factory=dict)

    @property
    def ldk(self):
        return low_ldk(self.k_low, self.low)

    @property
    def ldo(self):
        return sqf_pad_k_out(self.k_out, self.branch) if self.k_out else 0

    def desc(self) -> sqf_acts:
        t = self.t
        return sqf_acts(self.m, self.k_low, self.k_out, self.ldk, self.ldo, DTYPES[self.low],
                        DTYPES[self.branch], _ptr(t["x_low"]), _ptr(t.get("s_x")),
                        _ptr(t.get("s_xb")), _ptr(t["x_out"]), _ptr(t.get("s_xo")))


def alloc_weights(k, n, k_out, branch="bf16", groups=1, sq_nnz=0, sq_bank=0, low="i4",
                  device="cuda") -> Weights:
    w = Weights(k=k, n=n, k_low=k - k_out, k_out=k_out, branch=branch, groups=groups, sq_nnz=sq_nnz,
                sq_bank=sq_bank, low=low)
    g = groups
    t = w.t
    if low in ("i4e2m3", "mxfp4"):
        assert g == 1, "the K-blocked layouts are built for one weight set"
        t["w_low"] = _low_tensor(n, w.k_low, low, device, zero=True)
    else:
        t["w_low"] = torch.zeros((g, n, w.ldk), dtype=torch.uint8, device=device)
    if low == "mxfp4":
        t["s_wb"] = _mx_scales(n, w.k_low, device)
    else:
        t["s_w"] = torch.zeros((g, n), dtype=torch.float32, device=device)
    t["w_out"] = torch.zeros((g, n, w.ldo), dtype=_BR_TORCH[branch], device=device)
    t["s_wo"] = torch.zeros((g, n), dtype=torch.float32, device=device) if branch != "bf16" else None
    if sq_nnz:
        t["sq_val"] = torch.zeros((n, sq_nnz), dtype=torch.int8, device=device)
        t["s_w8"] = torch.zeros(n, dtype=torch.float32, device=device)
    return w


def alloc_acts(m, k_low, k_out, low="i4", branch="bf16", device="cuda") -> Acts:
    a = Acts(m=m, k_low=k_low, k_out=k_out, low=low, branch=branch)
    a.t["x_low"] = _low_tensor(m, k_low, low, device, zero=False)
    if low == "mxfp4":
        a.t["s_xb"] = _mx_scales(m, k_low, device)
    else:
        a.t["s_x"] = torch.empty(m, dtype=torch.float32, device=device)
    a.t["x_out"] = torch.empty((m, a.ldo), dtype=_BR_TORCH[branch], device=device)
    a.t["s_xo"] = torch.empty(m, dtype=torch.float32, device=device) if branch != "bf16" else None
    return a


# ------------------------------------------------------------------ entry points
def sqf_select_channels(x_cal: torch.Tensor, w: torch.Tensor, k_out: int, stream=None,
                        want_score: bool = True):
    """a0: returns (idx int32 [k_out], map int32 [k], score f64 [k] or None,
    hdiag f32 [k]).  Without ``want_score`` the library borrows its own
    workspace for the scores."""
    assert x_cal.is_cuda and w.is_cuda and x_cal.dtype == torch.float32 and w.dtype == torch.float32
    x_cal, w = x_cal.contiguous(), w.contiguous()
    m_cal, k = x_cal.shape
    n = w.shape[1]
    dev = x_cal.device
    idx = torch.empty(max(k_out, 1), dtype=torch.int32, device=dev)
    mp = torch.empty(k, dtype=torch.int32, device=dev)
    score = torch.empty(k, dtype=torch.float64, device=dev) if want_score else None
    hdiag = torch.empty(k, dtype=torch.float32, device=dev)
    _check(_lib.sqf_select_channels(_ptr(x_cal), m_cal, k, _ptr(w), n, k_out, _ptr(idx), _ptr(mp),
                                    _ptr(score), _ptr(hdiag), _stream(stream)))
    return idx[:k_out], mp, score, hdiag


def sqf_select_channels_noalloc(x_cal: torch.Tensor, w: torch.Tensor, k_out: int, idx=None,
                                mp=None, hdiag=None, stream=None):
    """a0 through the allocation-free entry point: the scores live in the
    library's static per-GPU array.  Output tensors may be passed in (the
    call itself allocates nothing); returns (idx, map, hdiag)."""
    assert x_cal.is_cuda and w.is_cuda and x_cal.dtype == torch.float32 and w.dtype == torch.float32
    assert x_cal.is_contiguous() and w.is_contiguous()
    m_cal, k = x_cal.shape
    n = w.shape[1]
    dev = x_cal.device
    if idx is None:
        idx = torch.empty(max(k_out, 1), dtype=torch.int32, device=dev)
    if mp is None:
        mp = torch.empty(k, dtype=torch.int32, device=dev)
    if hdiag is None:
        hdiag = torch.empty(k, dtype=torch.float32, device=dev)
    _check(_lib.sqf_select_channels_noalloc(_ptr(x_cal), m_cal, k, _ptr(w), n, k_out, _ptr(idx),
                                            _ptr(mp), _ptr(hdiag), _stream(stream)))
    return idx[:k_out], mp, hdiag


def sqf_pack_weights(w: torch.Tensor, mp: torch.Tensor, branch="bf16", hdiag=None, sq_nnz=0,
                     out: Weights | None = None, stream=None, sq_bank=0, low="i4") -> Weights:
    """a1: w [k][n] (or [groups][k][n] with mp [groups][k]) fp32 -> Weights."""
    groups = w.shape[0] if w.dim() == 3 else 1
    k, n = w.shape[-2], w.shape[-1]
    mpc = mp.reshape(groups, k)
    k_out = int((mpc[0] < 0).sum().item())
    if out is None:
        out = alloc_weights(k, n, k_out, branch=branch, groups=groups, sq_nnz=sq_nnz,
                            sq_bank=sq_bank, low=low, device=w.device)
    d = out.desc()
    _check(_lib.sqf_pack_weights(_ptr(w.contiguous()), _ptr(mp.contiguous()), _ptr(hdiag),
                                 ctypes.byref(d), _stream(stream)))
    return out


def sqf_quantize_split_act(x: torch.Tensor, mp: torch.Tensor, out: Acts, stream=None) -> Acts:
    """a2: x [m][k] (fp32 or bf16) -> fills ``out``."""
    xd = SQF_BF16 if x.dtype == torch.bfloat16 else SQF_F32
    d = out.desc()
    _check(_lib.sqf_quantize_split_act(_ptr(x), xd, x.stride(0), _ptr(mp), ctypes.byref(d),
                                       _stream(stream)))
    return out


def sqf_rmsnorm_quantize_split_act(x: torch.Tensor, gamma: torch.Tensor, eps: float,
                                   mp: torch.Tensor, out: Acts, stream=None) -> Acts:
    """a2 with the RMS norm in front of it fused in: x [m][k] (fp32 or
    bf16), gamma [k] fp32 -> fills ``out``."""
    xd = SQF_BF16 if x.dtype == torch.bfloat16 else SQF_F32
    assert gamma.dtype == torch.float32 and gamma.is_contiguous()
    d = out.desc()
    _check(_lib.sqf_rmsnorm_quantize_split_act(_ptr(x), xd, x.stride(0), _ptr(gamma), float(eps),
                                               _ptr(mp), ctypes.byref(d), _stream(stream)))
    return out


def sqf_slot_order(mp: torch.Tensor, stream=None):
    """(perm, slice_map) of a channel map: the slot order and the map of the
    reordered axis."""
    k = mp.numel()
    perm = torch.empty(k, dtype=torch.int32, device=mp.device)
    sm = torch.empty(k, dtype=torch.int32, device=mp.device)
    _check(_lib.sqf_slot_order(_ptr(mp), k, _ptr(perm), _ptr(sm), _stream(stream)))
    return perm, sm


def sqf_permute_channels(src: torch.Tensor, perm: torch.Tensor, axis: int, stream=None):
    """src [rows][cols] fp32 gathered along ``axis`` by perm (a new tensor)."""
    assert src.dtype == torch.float32 and src.dim() == 2 and src.stride(1) == 1
    dst = torch.empty(src.shape, dtype=torch.float32, device=src.device)
    _check(_lib.sqf_permute_channels(_ptr(src), src.shape[0], src.shape[1], src.stride(0),
                                     _ptr(perm), axis, _ptr(dst), dst.stride(0), _stream(stream)))
    return dst


def sqf_quantize_split_act_grouped(x: torch.Tensor, row_off: torch.Tensor, maps: torch.Tensor,
                                   out: Acts, stream=None) -> Acts:
    xd = SQF_BF16 if x.dtype == torch.bfloat16 else SQF_F32
    d = out.desc()
    groups = row_off.numel() - 1
    _check(_lib.sqf_quantize_split_act_grouped(_ptr(x), xd, x.stride(0), groups, _ptr(row_off),
                                               _ptr(maps), ctypes.byref(d), _stream(stream)))
    return out


def _y_out(a, w, y, y_dtype):
    dt = {"f32": torch.float32, "bf16": torch.bfloat16}[y_dtype]
    if y is None:
        y = torch.empty((a.m, w.n), dtype=dt, device=a.t["x_out"].device)
    if y.dtype != dt:
        raise ValueError(f"y is {y.dtype}, y_dtype {y_dtype}")
    return y


def sqf_dual_gemm(a: Acts, w: Weights, y: torch.Tensor | None = None, debug: bool = False,
                  stream=None, y_dtype: str = "f32", tile: str = "auto"):
    """a3-a5: returns y [m][n] (fp32, or bf16 with ``y_dtype="bf16"``), and the
    int32 accumulators with ``debug`` (fp32 y only).  ``tile`` forces a tile
    shape ("256", "128", "64") through sqf_dual_gemm_ex; the default calls
    sqf_dual_gemm (fp32) or sqf_dual_gemm_y (bf16)."""
    dev = a.t["x_out"].device
    y = _y_out(a, w, y, y_dtype)
    if debug and y_dtype != "f32":
        raise ValueError("the accumulator dump comes with fp32 y")
    dbg = [None, None, None]
    if debug:
        dbg[0] = torch.empty((a.m, w.n), dtype=torch.int32, device=dev)
        if w.sq_nnz:
            dbg[1] = torch.empty((a.m, w.n), dtype=torch.int32, device=dev)
            dbg[2] = torch.empty((a.m, w.n), dtype=torch.int32, device=dev)
    da, dw = a.desc(), w.desc()
    if tile != "auto":
        _check(_lib.sqf_dual_gemm_ex(ctypes.byref(da), ctypes.byref(dw), _ptr(y), DTYPES[y_dtype],
                                     y.stride(0), TILES[tile], _ptr(dbg[0]), _ptr(dbg[1]),
                                     _ptr(dbg[2]), _stream(stream)))
    elif y_dtype != "f32":
        _check(_lib.sqf_dual_gemm_y(ctypes.byref(da), ctypes.byref(dw), _ptr(y), DTYPES[y_dtype],
                                    y.stride(0), _stream(stream)))
    else:
        _check(_lib.sqf_dual_gemm(ctypes.byref(da), ctypes.byref(dw), _ptr(y), y.stride(0),
                                  _ptr(dbg[0]), _ptr(dbg[1]), _ptr(dbg[2]), _stream(stream)))
    return (y, *dbg) if debug else y


def sqf_sq_workspace_bytes(w: Weights) -> int:
    dw = w.desc()
    return _lib.sqf_sq_workspace_bytes(ctypes.byref(dw))


def sqf_dual_gemm_sq_ws(a: Acts, w: Weights, y: torch.Tensor | None = None,
                        workspace: torch.Tensor | None = None, debug: bool = False, stream=None):
    """a7 with the gather done once per call into ``workspace`` (a uint8
    device tensor of at least sqf_sq_workspace_bytes(w) bytes; allocated here
    when None).  Returns y [m][n] fp32, and the three int32 accumulators with
    ``debug``."""
    dev = a.t["x_out"].device
    y = _y_out(a, w, y, "f32")
    if workspace is None:
        workspace = torch.empty(max(sqf_sq_workspace_bytes(w), 1), dtype=torch.uint8, device=dev)
    dbg = [None, None, None]
    if debug:
        dbg = [torch.full((a.m, w.n), -1, dtype=torch.int32, device=dev) for _ in range(3)]
    da, dw = a.desc(), w.desc()
    _check(_lib.sqf_dual_gemm_sq_ws(ctypes.byref(da), ctypes.byref(dw), _ptr(y), y.stride(0),
                                    _ptr(workspace), workspace.numel(), _ptr(dbg[0]), _ptr(dbg[1]),
                                    _ptr(dbg[2]), _stream(stream)))
    return (y, *dbg) if debug else y


def sqf_dual_gemm_grouped(a: Acts, w: Weights, row_off: torch.Tensor, y=None, debug=False,
                          stream=None, y_dtype: str = "f32", tile: str = "auto"):
    dev = a.t["x_out"].device
    y = _y_out(a, w, y, y_dtype)
    if debug and y_dtype != "f32":
        raise ValueError("the accumulator dump comes with fp32 y")
    dbg = torch.empty((a.m, w.n), dtype=torch.int32, device=dev) if debug else None
    da, dw = a.desc(), w.desc()
    g = row_off.numel() - 1
    if tile != "auto":
        _check(_lib.sqf_dual_gemm_grouped_ex(ctypes.byref(da), ctypes.byref(dw), g, _ptr(row_off),
                                             _ptr(y), DTYPES[y_dtype], y.stride(0), TILES[tile],
                                             _ptr(dbg), _stream(stream)))
    elif y_dtype != "f32":
        _check(_lib.sqf_dual_gemm_grouped_y(ctypes.byref(da), ctypes.byref(dw), g, _ptr(row_off),
                                            _ptr(y), DTYPES[y_dtype], y.stride(0), _stream(stream)))
    else:
        _check(_lib.sqf_dual_gemm_grouped(ctypes.byref(da), ctypes.byref(dw), g, _ptr(row_off),
                                          _ptr(y), y.stride(0), _ptr(dbg), _stream(stream)))
    return (y, dbg) if debug else y
