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
    assert len(names) == 21
    for name in names:
        assert hasattr(sqf._lib, name), name


def test_abi_version_and_padding(sqf):
    assert sqf.sqf_abi_version() == 6
    assert sqf.sqf_pad_rows(0) == 0 and sqf.sqf_pad_rows(1) == 256 and sqf.sqf_pad_rows(4096) == 4096
    assert sqf.sqf_pad_rows(300) == 512 and sqf._lib.sqf_pad_rows(-1) == -1
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
                        sqf.sqf_pad_k_out(k_out, branch), br, 1, sqf.SQF_I4X2, 0, mem(), mem(),
                        None, mem(), mem() if branch != "bf16" else None, 0, 0, None, None)
    for f, v in kw.items():
        setattr(d, f, v)
    return d


def _acts(sqf, mem, m=64, k=512, k_out=32, branch="bf16", low="i4", **kw):
    k_low = k - k_out
    pad = sqf.sqf_pad_k_low(k_low)
    d = sqf.sqf_acts(m, k_low, k_out, pad // 2 if low == "i4" else pad,
                     sqf.sqf_pad_k_out(k_out, branch), sqf.DTYPES[low], sqf.DTYPES[branch],
                     mem(), mem(), None, mem(), mem() if branch != "bf16" else None)
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
    a = _acts(sqf, mem, k=70000, k_out=20)  # k beyond 65536
    assert f(mem(), sqf.SQF_BF16, 70000, mem(), ctypes.byref(a), None) == 2
    a = _acts(sqf, mem)
    assert f(None, sqf.SQF_BF16, 512, mem(), ctypes.byref(a), None) == 1
    assert f(mem(), sqf.SQF_I8, 512, mem(), ctypes.byref(a), None) == 1
    assert f(mem(), sqf.SQF_BF16, 500, mem(), ctypes.byref(a), None) == 2  # ldx < k
    assert f(mem(misalign=1), sqf.SQF_BF16, 512, mem(), ctypes.byref(a), None) == 5  # odd bf16
    assert f(mem(misalign=2), sqf.SQF_F32, 512, mem(), ctypes.byref(a), None) == 5  # fp32 at 2 B
    g = sqf._lib.sqf_quantize_split_act_grouped
    # a grouped call takes the 16-byte chunk loads only
    assert g(mem(misalign=2), sqf.SQF_BF16, 512, 2, mem(), mem(), ctypes.byref(a), None) == 3
    assert f(mem(), sqf.SQF_BF16, 512, mem(), None, None) == 1


def test_select_argument_errors(sqf):
    mem = FakeMem()
    f = sqf._lib.sqf_select_channels
    assert f(None, 4, 8, mem(), 4, 2, mem(), mem(), mem(), None, None) == 1
    assert f(mem(), 0, 8, mem(), 4, 2, mem(), mem(), mem(), None, None) == 2
    assert f(mem(), 4, 8, mem(), 4, 9, mem(), mem(), mem(), None, None) == 2
    assert f(mem(), 4, 8, mem(), 4, 2, None, mem(), mem(), None, None) == 1
    assert f(mem(), 4, 8, mem(), 4, 2, mem(), None, mem(), None, None) == 1  # map_out required


def test_noalloc_select_argument_errors(sqf):
    """The allocation-free channel choice: the shared checks, and k beyond
    its static score array, fail before any device call."""
    mem = FakeMem()
    f = sqf._lib.sqf_select_channels_noalloc
    assert f(None, 4, 8, mem(), 4, 2, mem(), mem(), None, None) == 1
    assert f(mem(), 4, 8, mem(), 4, 9, mem(), mem(), None, None) == 2
    assert f(mem(), 4, 8, mem(), 4, 2, mem(), None, None, None) == 1
    assert f(mem(), 4, 65537, mem(), 4, 2, mem(), mem(), None, None) == 2
    assert "65536" in sqf.sqf_last_error()


def test_producer_side_argument_errors(sqf):
    """The fused norm + split, the slot order and the channel permutation
    refuse bad arguments before any launch."""
    mem = FakeMem()
    f = sqf._lib.sqf_rmsnorm_quantize_split_act
    a = _acts(sqf, mem)
    assert f(mem(), sqf.SQF_BF16, 512, None, 1e-5, mem(), ctypes.byref(a), None) == 1  # no gamma
    assert f(mem(), sqf.SQF_BF16, 512, mem(), -1.0, mem(), ctypes.byref(a), None) == 1  # eps
    assert f(mem(), sqf.SQF_BF16, 512, mem(misalign=2), 1e-5, mem(), ctypes.byref(a), None) == 5
    a8 = _acts(sqf, mem, branch="fp8")
    assert f(mem(), sqf.SQF_BF16, 512, mem(), 1e-5, mem(), ctypes.byref(a8), None) == 3
    am, _ = _mx_pair(sqf, mem)
    assert f(mem(), sqf.SQF_BF16, 512, mem(), 1e-5, mem(), ctypes.byref(am), None) == 3
    big = _acts(sqf, mem, k=60000, k_out=64)  # gamma does not fit next to the images
    assert f(mem(), sqf.SQF_BF16, 60000, mem(), 1e-5, mem(), ctypes.byref(big), None) == 2
    so = sqf._lib.sqf_slot_order
    assert so(None, 8, mem(), mem(), None) == 1
    assert so(mem(), 0, mem(), mem(), None) == 2
    pc = sqf._lib.sqf_permute_channels
    assert pc(mem(), 4, 8, 8, mem(), 2, mem(), 8, None) == 1  # axis
    assert pc(mem(), 4, 8, 4, mem(), 1, mem(), 8, None) == 2  # ld_src < cols
    b = mem()
    assert pc(b, 4, 8, 8, mem(), 1, b, 8, None) == 1  # in place
    assert sqf.sqf_last_error() != ""


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
    w.sq_val, w.s_w8 = mem(), mem()
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
    w8.sq_nnz, w8.sq_val, w8.s_w8 = 60, mem(), mem()
    assert f(ctypes.byref(a8), ctypes.byref(w8), mem(), sqf.SQF_BF16, 256, None) == 3
    g = sqf._lib.sqf_dual_gemm_grouped_y
    w.groups = 4
    assert g(ctypes.byref(a), ctypes.byref(w), 4, mem(), mem(), 7, 256, None) == 1
    assert g(ctypes.byref(a), ctypes.byref(w), 3, mem(), mem(), sqf.SQF_BF16, 256, None) == 1


def test_explicit_options_argument_errors(sqf):
    """sqf_dual_gemm_ex / _grouped_ex: a bad tile or output type, a tile the
    branch does not have, and debug outputs with bf16 Y are refused before any
    launch."""
    mem = FakeMem()
    a = _acts(sqf, mem)
    w = _weights(sqf, mem)
    f = sqf._lib.sqf_dual_gemm_ex
    st = lambda *args: f(ctypes.byref(args[0]), ctypes.byref(args[1]), *args[2:])
    assert st(a, w, mem(), sqf.SQF_F32, 256, 7, None, None, None, None) == 1  # no such tile
    assert st(a, w, mem(), sqf.SQF_I8, 256, -1, None, None, None, None) == 1  # output type
    assert st(a, w, mem(), sqf.SQF_BF16, 256, -1, mem(), None, None, None) == 1  # dbg + bf16 Y
    a8 = _acts(sqf, mem, branch="fp8")
    w8 = _weights(sqf, mem, branch="fp8")
    assert st(a8, w8, mem(), sqf.SQF_F32, 256, sqf.TILES["256"], None, None, None, None) == 3
    g = sqf._lib.sqf_dual_gemm_grouped_ex
    w.groups = 4
    assert g(ctypes.byref(a), ctypes.byref(w), 4, mem(), mem(), sqf.SQF_F32, 256,
             sqf.TILES["64"], None, None) == 3  # grouped tiles are 256 or 128
    assert g(ctypes.byref(a), ctypes.byref(w), 4, mem(), mem(), sqf.SQF_F32, 256, 9, None,
             None) == 1
    assert sqf.sqf_last_error() != ""


def _mx_pair(sqf, mem, m=64, k=512, k_out=32, n=256):
    k_low = k - k_out
    a = _acts(sqf, mem, m=m, k=k, k_out=k_out)
    a.low, a.s_x, a.s_xb = sqf.SQF_MXFP4, None, mem()
    w = _weights(sqf, mem, k=k, n=n, k_out=k_out)
    w.low, w.s_w, w.s_wb = sqf.SQF_MXFP4, None, mem()
    assert a.ldk == w.ldk == sqf.sqf_pad_k_low(k_low) // 2
    return a, w


def test_mxfp4_contract_errors(sqf):
    """The MXFP4 low path: block scales required and 16-byte aligned, one
    weight set, a bf16 branch, the 256x256 tile only, no integer debug
    accumulators, no grouped form -- all refused before any launch."""
    mem = FakeMem()
    ex = lambda a, w, y, yd, ldy, tile, dbg: sqf._lib.sqf_dual_gemm_ex(
        ctypes.byref(a), ctypes.byref(w), y, yd, ldy, tile, dbg, None, None, None)
    a, w = _mx_pair(sqf, mem)
    assert ex(a, w, mem(), sqf.SQF_F32, 256, sqf.TILES["256"], mem()) == 3  # debug accumulators
    assert ex(a, w, mem(), sqf.SQF_F32, 256, sqf.TILES["128"], None) == 3  # one tile shape
    w.s_wb = None
    assert ex(a, w, mem(), sqf.SQF_F32, 256, -1, None) == 1
    w.s_wb = mem(misalign=4)
    assert ex(a, w, mem(), sqf.SQF_F32, 256, -1, None) == 5
    a, w = _mx_pair(sqf, mem)
    a.s_xb = None
    assert ex(a, w, mem(), sqf.SQF_F32, 256, -1, None) == 1
    a, w = _mx_pair(sqf, mem)
    w.groups = 2
    assert sqf._lib.sqf_pack_weights(mem(), mem(), None, ctypes.byref(w), None) == 3
    a, w = _mx_pair(sqf, mem)
    assert sqf._lib.sqf_dual_gemm_grouped(ctypes.byref(a), ctypes.byref(w), 1, mem(), mem(), 256,
                                          None, None) == 3
    a, w = _mx_pair(sqf, mem)
    w.branch, w.ldo, w.s_wo = sqf.SQF_FP8_E4M3, 128, mem()
    assert sqf._lib.sqf_pack_weights(mem(), mem(), None, ctypes.byref(w), None) == 3
    a, w = _mx_pair(sqf, mem)
    w.low = sqf.SQF_I4X2  # storages disagree
    w.s_w = mem()
    assert ex(a, w, mem(), sqf.SQF_F32, 256, -1, None) == 1
    assert sqf.sqf_last_error() != ""


def test_fp_weight_side_contract_errors(sqf):
    """The floating-point weight-side format: E2M1 weights only with marks and
    an E4M3 branch, E4M3 activations only with an E4M3 branch, and the two
    forms never mixed -- refused before any launch."""
    mem = FakeMem()

    def wfp(**kw):
        w = _weights(sqf, mem, k=544, k_out=32, branch="fp8")
        w.low, w.sq_nnz, w.sq_val, w.s_w8, w.s_wo = sqf.SQF_FP4_E2M1, 64, mem(), mem(), mem()
        for f, v in kw.items():
            setattr(w, f, v)
        return w

    pack = lambda w: sqf._lib.sqf_pack_weights(mem(), mem(), mem(), ctypes.byref(w), None)
    assert pack(wfp(sq_nnz=0)) == 3
    w = wfp()
    w.branch, w.ldo = sqf.SQF_I8, 128
    assert pack(w) == 3
    afp = _acts(sqf, mem, k=544, k_out=32, branch="fp8")
    afp.low, afp.ldk = sqf.SQF_FP8_E4M3, 512
    g = lambda a, w, dbg=(None, None, None): _gemm(sqf, a, w, mem(), 256, dbg)
    assert g(afp, wfp(), (mem(), mem(), mem())) == 3  # no integer accumulators
    a8 = _acts(sqf, mem, k=544, k_out=32, branch="fp8", low="i8")
    assert g(a8, wfp()) == 1  # int8 activations with E2M1 weights
    abf = _acts(sqf, mem, k=544, k_out=32)
    abf.low, abf.ldk = sqf.SQF_FP8_E4M3, 512
    assert sqf._lib.sqf_quantize_split_act(mem(), sqf.SQF_BF16, 544, mem(), ctypes.byref(abf), None) == 3
    assert sqf.sqf_last_error() != ""


def test_weight_side_bank_must_be_supported(sqf):
    """Banks: a multiple of 64 slots that divides k_low, an equal count of
    marks in each bank, at most 1024 slots (or the whole row)."""
    mem = FakeMem()

    def st(k_low, nnz, bank):
        w = _weights(sqf, mem, k=k_low + 32, k_out=32)
        w.branch, w.ldo, w.s_wo = sqf.SQF_I8, 128, mem()
        w.sq_nnz, w.sq_val, w.s_w8, w.sq_bank = nnz, mem(), mem(), bank
        return sqf._lib.sqf_pack_weights(mem(), mem(), mem(), ctypes.byref(w), None)

    assert st(480, 60, 7) == 2     # not a multiple of 64
    assert st(512, 60, 64) == 2    # 60 marks over 8 banks
    assert st(512, 64, 96) == 2    # 96 is not a multiple of 64
    assert st(512, 64, 192) == 2   # does not divide 512
    assert st(4096, 64, 2048) == 3  # beyond the largest bank built
    assert "bank" in sqf.sqf_last_error()


def test_no_entry_point_reads_the_environment():
    """Every option is an argument: the library sources call no getenv."""
    csrc = os.path.join(ROOT, "outlier_split_mixed_amd", "csrc")
    for fn in os.listdir(csrc):
        text = open(os.path.join(csrc, fn)).read()
        assert "getenv" not in text, fn


def test_weight_side_workspace_contract(sqf):
    """sqf_dual_gemm_sq_ws: the workspace holds one decoded image per (128-row
    weight tile, 128-slot stage) -- 32 KiB in the integer form (int8 clean and
    sparse tiles), 24 KiB in the FP8/FP4 form (E2M1 clean tile) -- and the
    call refuses, before any launch, channel-split weights, a NULL, misaligned
    or too small workspace."""
    mem = FakeMem()

    def wsq(k_low=480, n=300, fp=False):
        w = _weights(sqf, mem, k=k_low + 32, n=n, k_out=32, branch="fp8" if fp else "bf16")
        w.branch, w.ldo, w.s_wo = (sqf.SQF_FP8_E4M3 if fp else sqf.SQF_I8), 128, mem()
        w.sq_nnz, w.sq_val, w.s_w8 = k_low // 8, mem(), mem()
        if fp:
            w.low = sqf.SQF_FP4_E2M1
        return w

    ws = lambda w: sqf._lib.sqf_sq_workspace_bytes(ctypes.byref(w))
    # k_low 480 -> 512 padded slots = 4 stages; 300 rows -> 3 tiles
    assert ws(wsq()) == 3 * 4 * 32768
    assert ws(wsq(fp=True)) == 3 * 4 * 24576
    assert ws(wsq(k_low=3840, n=14336)) == 112 * 30 * 32768
    assert ws(_weights(sqf, mem)) == -1  # channel-split weights
    assert sqf._lib.sqf_sq_workspace_bytes(None) == -1

    a = _acts(sqf, mem, k=512, k_out=32, branch="i8", low="i8")
    a.ldo = 128
    a.s_xo = mem()

    def call(w, wsp, nbytes):
        return sqf._lib.sqf_dual_gemm_sq_ws(ctypes.byref(a), ctypes.byref(w), mem(), 300, wsp,
                                            nbytes, None, None, None, None)

    w = wsq()
    need = ws(w)
    assert call(w, None, need) == 1
    assert "NULL" in sqf.sqf_last_error()
    assert call(w, mem(misalign=16), need) == 5
    big = ctypes.create_string_buffer(need + 512)
    aligned = ctypes.c_void_p((ctypes.addressof(big) + 255) // 256 * 256)
    assert call(w, aligned, need - 1) == 2
    assert "needed" in sqf.sqf_last_error()
    ab = _acts(sqf, mem, k=512, k_out=32)
    st = sqf._lib.sqf_dual_gemm_sq_ws(ctypes.byref(ab), ctypes.byref(_weights(sqf, mem)), mem(), 256,
                                      aligned, need, None, None, None, None)
    assert st == 1 and "weight-side" in sqf.sqf_last_error()
