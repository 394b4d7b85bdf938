"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, its pure host helpers are right, and every invalid argument
returns its status (and a message) before anything is launched."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sqf.h")


@pytest.fixture(scope="module")
def sqf():
    from outlier_split_mixed_amd import sqf as mod

    return mod


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sqf_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(sqf):
    names = _declared_functions()
    assert len(names) == 12
    for name in names:
        assert hasattr(sqf._lib, name), name


def test_abi_version_and_padding(sqf):
    assert sqf.sqf_abi_version() == 1
    assert sqf.sqf_pad_k_low(0) == 0 and sqf.sqf_pad_k_low(1) == 256
    assert sqf.sqf_pad_k_low(7680) == 7680 and sqf.sqf_pad_k_low(13440) == 13568
    assert sqf._lib.sqf_pad_k_low(-1) == -1
    assert sqf.sqf_pad_k_out(0, "bf16") == 0 and sqf.sqf_pad_k_out(16, "bf16") == 64
    assert sqf.sqf_pad_k_out(48, "fp8") == 128 and sqf.sqf_pad_k_out(512, "bf16") == 512
    assert sqf._lib.sqf_pad_k_out(16, 99) == -1


class FakeMem:
    """Host buffers whose addresses stand in for device pointers: every call
    below fails validation before any pointer is dereferenced or launched."""

    def __init__(self):
        self.bufs = []

    def __call__(self, nbytes=4096, misalign=0):
        b = ctypes.create_string_buffer(nbytes + 64)
        self.bufs.append(b)
        addr = (ctypes.addressof(b) + 15) // 16 * 16 + misalign
        return ctypes.c_void_p(addr)


def _weights(sqf, mem, k=512, n=256, k_out=32, branch="bf16", **kw):
    k_low = k - k_out
    br = sqf.DTYPES[branch]
    d = sqf.sqf_weights(k, n, k_low, k_out, sqf.sqf_pad_k_low(k_low) // 2,
                        sqf.sqf_pad_k_out(k_out, branch), br, 1, mem(), mem(), mem(),
                        mem() if branch != "bf16" else None, 0, None, None, None)
    for f, v in kw.items():
        setattr(d, f, v)
    return d


def _acts(sqf, mem, m=64, k=512, k_out=32, branch="bf16", low="i4", **kw):
    k_low = k - k_out
    pad = sqf.sqf_pad_k_low(k_low)
    d = sqf.sqf_acts(m, k_low, k_out, pad // 2 if low == "i4" else pad,
                     sqf.sqf_pad_k_out(k_out, branch), sqf.DTYPES[low], sqf.DTYPES[branch],
                     mem(), mem(), mem(), mem() if branch != "bf16" else None)
    for f, v in kw.items():
        setattr(d, f, v)
    return d


def _gemm(sqf, a, w, y, ldy, dbg=(None, None, None)):
    return sqf._lib.sqf_dual_gemm(ctypes.byref(a), ctypes.byref(w), y, ldy, *dbg, None)


CASES = [
    ("null y", dict(), dict(), "y_null", 1),
    ("ldy < n", dict(), dict(), "ldy_small", 2),
    ("k_out mismatch", dict(k_out=16), dict(), None, 1),
    ("branch mismatch", dict(), dict(branch="fp8"), None, 1),
    ("bad ldk", dict(ldk=100), dict(), None, 2),
    ("bad ldo", dict(ldo=10), dict(), None, 2),
    ("bad low dtype", dict(low=7), dict(), None, 1),
    ("misaligned x_low", dict(x_low="mis"), dict(), None, 5),
    ("null s_x", dict(s_x=None), dict(), None, 1),
    ("negative m", dict(m=-1), dict(), None, 2),
    ("weights bad n", dict(), dict(n=0), None, 2),
    ("weights inconsistent k", dict(), dict(k=999), None, 2),
    ("weights misaligned w_out", dict(), dict(w_out="mis"), None, 5),
    ("int8 branch without weight-side format", dict(branch="i8", ldo=128), dict(branch="i8"), None, 3),
    ("int8 activations with channel split", dict(low="i8"), dict(), None, 1),
]


@pytest.mark.parametrize("name,akw,wkw,ymode,status", CASES, ids=[c[0] for c in CASES])
def test_dual_gemm_argument_errors(sqf, name, akw, wkw, ymode, status):
    mem = FakeMem()
    abr = akw.pop("branch", "bf16")
    alow = akw.pop("low", "i4") if isinstance(akw.get("low"), str) else "i4"
    wbr = wkw.pop("branch", "bf16")
    a = _acts(sqf, mem, branch=abr, low=alow)
    w = _weights(sqf, mem, branch=wbr if wbr != "i8" else "bf16")
    if wbr == "i8":
        w.branch = sqf.SQF_I8
        w.ldo = 128
        w.s_wo = mem()
    for f, v in akw.items():
        setattr(a, f, mem(misalign=4) if v == "mis" else v)
    for f, v in wkw.items():
        setattr(w, f, mem(misalign=4) if v == "mis" else v)
    y = None if ymode == "y_null" else mem()
    ldy = 10 if ymode == "ldy_small" else 256
    st = _gemm(sqf, a, w, y, ldy)
    assert st == status, (st, sqf.sqf_last_error())
    assert sqf.sqf_last_error() != ""


def test_zero_rows_is_a_no_op(sqf):
    mem = FakeMem()
    a = _acts(sqf, mem, m=0)
    w = _weights(sqf, mem)
    assert _gemm(sqf, a, w, None, 256) == 0
    assert sqf._lib.sqf_quantize_split_act(mem(), sqf.SQF_BF16, 512, mem(), ctypes.byref(a), None) == 0


def test_quantize_argument_errors(sqf):
    mem = FakeMem()
    f = sqf._lib.sqf_quantize_split_act
    a = _acts(sqf, mem, k=500, k_out=20)  # k not a multiple of 8
    assert f(mem(), sqf.SQF_BF16, 504, mem(), ctypes.byref(a), None) == 2
    a = _acts(sqf, mem)
    assert f(None, sqf.SQF_BF16, 512, mem(), ctypes.byref(a), None) == 1
    assert f(mem(), sqf.SQF_I8, 512, mem(), ctypes.byref(a), None) == 1
    assert f(mem(), sqf.SQF_BF16, 500, mem(), ctypes.byref(a), None) == 2  # ldx < k
    assert f(mem(misalign=2), sqf.SQF_BF16, 512, mem(), ctypes.byref(a), None) == 5
    assert f(mem(), sqf.SQF_BF16, 512, mem(), None, None) == 1


def test_select_argument_errors(sqf):
    mem = FakeMem()
    f = sqf._lib.sqf_select_channels
    assert f(None, 4, 8, mem(), 4, 2, mem(), mem(), mem(), None, None) == 1
    assert f(mem(), 0, 8, mem(), 4, 2, mem(), mem(), mem(), None, None) == 2
    assert f(mem(), 4, 8, mem(), 4, 9, mem(), mem(), mem(), None, None) == 2
    assert f(mem(), 4, 8, mem(), 4, 2, None, mem(), mem(), None, None) == 1
    assert f(mem(), 4, 8, mem(), 4, 2, mem(), mem(), None, None, None) == 1


def test_pack_argument_errors(sqf):
    mem = FakeMem()
    f = sqf._lib.sqf_pack_weights
    w = _weights(sqf, mem)
    assert f(None, mem(), None, ctypes.byref(w), None) == 1
    w = _weights(sqf, mem, k=512, k_out=32, branch="bf16")
    w.branch = sqf.SQF_I8
    w.ldo = 128
    w.s_wo = mem()
    w.sq_nnz = 60
    assert f(mem(), mem(), None, ctypes.byref(w), None) == 1  # sq fields missing
    w.sq_val, w.s_w8, w.sq_tile_off = mem(), mem(), mem()
    assert f(mem(), mem(), None, ctypes.byref(w), None) == 1  # hdiag missing
    w.sq_nnz = 10_000
    assert f(mem(), mem(), mem(), ctypes.byref(w), None) == 2


def test_grouped_argument_errors(sqf):
    mem = FakeMem()
    a = _acts(sqf, mem)
    w = _weights(sqf, mem)
    w.groups = 4
    f = sqf._lib.sqf_dual_gemm_grouped
    assert f(ctypes.byref(a), ctypes.byref(w), 3, mem(), mem(), 256, None, None) == 1
    assert f(ctypes.byref(a), ctypes.byref(w), 4, None, mem(), 256, None, None) == 1
    w.groups = 1
    assert sqf._lib.sqf_dual_gemm(ctypes.byref(a), ctypes.byref(_weights(sqf, mem, **{})), None,
                                  256, None, None, None, None) == 1


def test_output_type_argument_errors(sqf):
    """The bf16-output entry points: an unknown output type, the weight-side
    format (fp32 output only) and the shared checks fail before any launch."""
    mem = FakeMem()
    a = _acts(sqf, mem)
    w = _weights(sqf, mem)
    f = sqf._lib.sqf_dual_gemm_y
    assert f(ctypes.byref(a), ctypes.byref(w), mem(), sqf.SQF_FP8_E4M3, 256, None) == 1
    assert f(ctypes.byref(a), ctypes.byref(w), mem(), sqf.SQF_BF16, 10, None) == 2  # ldy < n
    assert f(ctypes.byref(a), ctypes.byref(w), None, sqf.SQF_BF16, 256, None) == 1
    assert sqf.sqf_last_error() != ""
    a8 = _acts(sqf, mem, low="i8", branch="i8")
    w8 = _weights(sqf, mem)
    w8.branch, w8.ldo, w8.s_wo = sqf.SQF_I8, 128, mem()
    w8.sq_nnz, w8.sq_val, w8.s_w8, w8.sq_tile_off = 60, mem(), mem(), mem()
    assert f(ctypes.byref(a8), ctypes.byref(w8), mem(), sqf.SQF_BF16, 256, None) == 3
    g = sqf._lib.sqf_dual_gemm_grouped_y
    w.groups = 4
    assert g(ctypes.byref(a), ctypes.byref(w), 4, mem(), mem(), 7, 256, None) == 1
    assert g(ctypes.byref(a), ctypes.byref(w), 3, mem(), mem(), sqf.SQF_BF16, 256, None) == 1
