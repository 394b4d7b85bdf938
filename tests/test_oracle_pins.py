"""Pins of the CPU oracle against things other than itself.

Each test fixes part of the oracle with an independent source: a hand-worked
case, a fact the pages state, a library routine, a closed form or a brute
force.  Each is chosen so that a plausible slip in the oracle (a dropped
term, a wrong sign or index, a transposed operand, a wrong rounding) fails.
No GPU is needed.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from outlier_split_mixed_amd import synth

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def _floats(rows):
    return np.array([[float(v) for v in r] for r in rows], dtype=np.float32)


def _hexbytes(rows):
    return np.array([[int(v, 16) for v in r] for r in rows], dtype=np.int64)


# ------------------------------------------------------------------ hand-worked
def test_hand_case_osc(golden):
    g = golden("osc_hand_case.txt")
    x_cal, w = _floats(g["x_cal"]), _floats(g["w"])
    idx, mp, score, _ = oracle.select_channels(x_cal, w, int(g["k_out"][0][0]))
    assert idx.tolist() == [int(v) for v in g["idx"][0]]
    assert mp.tolist() == [int(v) for v in g["map"][0]]
    a = oracle.quantize_split_act(_floats(g["x"]), mp)
    assert a["ldk"] == 128 and a["ldo"] == 64
    exp = _hexbytes(g["x_low_bytes"])[0]
    assert a["x_low"][0, :2].tolist() == exp.tolist()
    assert not a["x_low"][0, 2:].any()
    assert a["s_x"][0] == np.float32(g["s_x"][0][0])
    assert int(a["x_out"][0, 0]) == int(g["x_out_bf16"][0][0], 16)
    assert not a["x_out"][0, 1:].any()
    wp = oracle.pack_weights(w, mp)
    assert wp["w_low"][:, :2].tolist() == _hexbytes(g["w_low_bytes"]).tolist()
    assert not wp["w_low"][:, 2:].any()
    assert wp["s_w"].tolist() == _floats(g["s_w"])[0].tolist()
    assert wp["w_out"][:, :1].astype(np.int64).tolist() == _hexbytes(g["w_out_bf16"]).tolist()
    y, acc, _, _ = oracle.dual_gemm(a, wp, debug=True)
    assert acc[0].tolist() == [int(v) for v in g["acc"][0]]
    assert y[0].tolist() == _floats(g["y"])[0].tolist()


def test_hand_case_sq_row(golden):
    g = golden("sq_row_hand_case.txt")
    wrow, hd = _floats(g["w"])[0], _floats(g["hdiag"])[0]
    nnz = int(g["nnz"][0][0])
    fields, v8, s8, s4 = oracle.sq_row(wrow, hd, nnz, bits=4)
    assert fields.tolist() == [int(v, 16) for v in g["fields"][0]]
    assert v8.tolist() == [int(v) for v in g["v8"][0]]
    assert s8 == np.float32(g["s_w8"][0][0]) and s4 == np.float32(g["s_w4"][0][0])
    # whole-matrix path: one output channel, no outlier channels, int8 activations
    w = wrow.reshape(8, 1)
    mp = np.arange(8, dtype=np.int32)
    wp = oracle.pack_weights_sq(w, mp, hd, nnz)
    assert wp["w_low"][0, :4].tolist() == _hexbytes(g["packed"])[0].tolist()
    a = oracle.quantize_split_act(_floats(g["x"]), mp, low="i8", branch="i8")
    assert a["s_x"][0] == 1.0
    y, al, asp, _ = oracle.dual_gemm(a, wp, debug=True)
    assert al[0, 0] == int(g["acc_low"][0][0]) and asp[0, 0] == int(g["acc_sp"][0][0])
    assert y[0, 0] == np.float32(g["y"][0][0])


# ------------------------------------------------------------------ page facts
def test_int2_reserved_code_matches_page_example():
    """SQ-format article, section 九: with INT2 the used values are {-1, 0, 1}
    and the value 2 marks a high-precision position."""
    rng = np.random.default_rng(7)
    w = rng.standard_normal(64).astype(np.float32)
    fields, v8, _, s_low = oracle.sq_row(w, np.ones(64, np.float32), 8, bits=2)
    signed = np.where(fields >= 2, fields.astype(np.int64) - 4, fields.astype(np.int64))
    marked = fields == 2
    assert marked.sum() == 8
    assert set(np.unique(signed[~marked]).tolist()) <= {-1, 0, 1}
    # the 8 marked slots are the 8 largest |w| (hdiag = 1)
    assert set(np.nonzero(marked)[0].tolist()) == set(np.argsort(-np.abs(w), kind="stable")[:8].tolist())


def test_storage_is_five_bits_at_seven_eighths_low():
    """SQ-format article, section 八: FP8 high / FP4 low at 87.5% low-precision
    share is about a 5-bit format.  With the dense 4-bit tensor covering every
    slot and 8-bit values carrying no index, 4 + 8/8 = 5 bits per weight."""
    k, n = 1024, 16
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((k, n)) * 0.02).astype(np.float32)
    mp = np.arange(k, dtype=np.int32)
    nnz = k // 8
    wp = oracle.pack_weights_sq(w, mp, np.ones(k, np.float32), nnz)
    bits = (wp["w_low"].nbytes + wp["sq_val"].nbytes) * 8 / (k * n)
    assert bits == 5.0
    # every row marks exactly nnz slots and stores exactly nnz values
    nib = np.stack([wp["w_low"] & 0xF, wp["w_low"] >> 4], -1).reshape(n, -1)
    assert ((nib == 8).sum(1) == nnz).all()


# ------------------------------------------------------------------ number formats
def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(11)
    v = np.concatenate([rng.standard_normal(3000).astype(np.float32) * 37,
                        # exact ties: bf16 value + half an ulp
                        (np.arange(1, 200, dtype=np.uint32) << 16 | 0x8000).view(np.float32)])
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.bf16_from_float(t) for t in v], dtype=np.uint16)
    assert (got == ref).all()


def test_e4m3_codes_match_torch_and_definition():
    # library routine: torch's float8_e4m3fn cast (round to nearest even) in range
    grid = np.concatenate([np.linspace(-448, 448, 4001), np.linspace(-0.02, 0.02, 801),
                           [2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -10, 1.0625, 1.1875, 240.0, 232.0]])
    grid = grid.astype(np.float32)
    ref = torch.from_numpy(grid).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_from_float(t) for t in grid], dtype=np.uint8)
    # torch keeps the sign of a value that rounds to zero; the oracle emits +0
    zero = (ref & 0x7F) == 0
    assert (got[~zero] == ref[~zero]).all()
    assert (got[zero] == 0).all()
    # definition facts: largest finite 448 = 0x7E, 1.0 = 0x38, min subnormal 2^-9 = 0x01,
    # ties to even (1.0625 -> 1.0, 1.1875 -> 1.25), saturation above 448
    assert oracle.e4m3_from_float(448.0) == 0x7E and oracle.e4m3_from_float(1.0) == 0x38
    assert oracle.e4m3_from_float(2.0 ** -9) == 0x01
    assert oracle.e4m3_from_float(1.0625) == 0x38 and oracle.e4m3_from_float(1.1875) == 0x3A
    assert oracle.e4m3_from_float(1000.0) == 0x7E and oracle.e4m3_from_float(-1000.0) == 0xFE
    for c in range(0x7F):
        assert oracle.e4m3_from_float(oracle.e4m3_to_float(c)) == c


# ------------------------------------------------------------------ quantiser
def _brute_codes(v, q):
    """Nearest integer in [-q, q] to v*inv by exhaustive search (ties to even)."""
    v = np.asarray(v, np.float32)
    a = np.float32(np.abs(v).max())
    inv = np.float32(q) / a
    out = []
    for t in v:
        p = float(np.float32(t * inv))
        best = None
        for c in range(-q, q + 1):
            d = abs(p - c)
            if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
                best = (d, c)
        out.append(best[1])
    return np.array(out), np.float32(a / np.float32(q))


@pytest.mark.parametrize("fmt,q", [("i4", 7), ("i8", 127)])
def test_quantizer_brute_force(fmt, q):
    rng = np.random.default_rng(5)
    v = rng.standard_normal(300).astype(np.float32) * 3
    v[17] = 0.5 * np.abs(v).max()  # likely tie region
    codes, s = oracle.quantize_vec(v, fmt)
    ref, sref = _brute_codes(v, q)
    assert (codes == ref).all() and s == sref


def test_quantizer_pow2_equivariance_and_sign_symmetry():
    rng = np.random.default_rng(9)
    v = rng.standard_normal(500).astype(np.float32)
    c0, s0 = oracle.quantize_vec(v, "i4")
    for e in (-3, 1, 5):
        c1, s1 = oracle.quantize_vec(v * np.float32(2.0 ** e), "i4")
        assert (c1 == c0).all() and s1 == np.float32(s0 * 2.0 ** e)
    cn, sn = oracle.quantize_vec(-v, "i4")
    assert (cn == -c0).all() and sn == s0
    cz, sz = oracle.quantize_vec(np.zeros(10, np.float32), "i4")
    assert not cz.any() and sz == 0.0


# ------------------------------------------------------------------ selection
def test_selection_matches_numpy_ranking():
    lay = synth.tiny()
    idx, mp, score, hdiag = oracle.select_channels(lay.x_cal, lay.w, lay.k_out)
    x64, w64 = lay.x_cal.astype(np.float64), lay.w.astype(np.float64)
    ref = np.abs(x64).mean(0) * np.linalg.norm(w64, axis=1)
    np.testing.assert_allclose(score, ref, rtol=1e-12)
    np.testing.assert_allclose(hdiag, (x64 ** 2).sum(0).astype(np.float32), rtol=1e-6)
    order = np.lexsort((np.arange(lay.k), -ref))
    srt = np.sort(ref)[::-1]
    assert (srt[lay.k_out - 1] - srt[lay.k_out]) / srt[lay.k_out - 1] > 1e-9  # margin guard
    assert idx.tolist() == sorted(order[: lay.k_out].tolist())
    # map: ascending slots for low channels, -(t+1) for outlier t
    is_out = np.zeros(lay.k, bool)
    is_out[idx] = True
    low = np.nonzero(~is_out)[0]
    assert (mp[low] == np.arange(len(low))).all()
    assert (mp[idx] == -(np.arange(len(idx)) + 1)).all()
    # token-persistent outliers are the ones found (OSC abstract)
    assert set(lay.scaled.tolist()) <= set(idx.tolist())


def test_selection_ties_go_to_lower_index():
    x = np.ones((4, 6), np.float32)
    w = np.ones((6, 3), np.float32)
    idx, mp, _, _ = oracle.select_channels(x, w, 2)
    assert idx.tolist() == [0, 1]
    assert mp.tolist() == [-1, -2, 0, 1, 2, 3]


# ------------------------------------------------------------------ whole op
def _np_w4a4(x, w):
    """Plain W4A4 (per-token / per-output-channel int4), numpy float32 + int64."""
    def q(v, axis):
        a = np.abs(v).max(axis=axis, keepdims=True).astype(np.float32)
        inv = np.where(a > 0, np.float32(7) / np.where(a > 0, a, 1), 0).astype(np.float32)
        c = np.clip(np.rint((v * inv).astype(np.float32)), -7, 7).astype(np.int64)
        return c, (a / np.float32(7)).astype(np.float32)
    cx, sx = q(x, 1)
    cw, sw = q(w, 0)
    acc = cx @ cw
    return sx.astype(np.float64) * sw.astype(np.float64) * acc, acc


def test_zero_outliers_is_plain_w4a4():
    lay = synth.tiny()
    mp = np.arange(lay.k, dtype=np.int32)
    a = oracle.quantize_split_act(lay.x, mp)
    wp = oracle.pack_weights(lay.w, mp)
    y, acc, _, _ = oracle.dual_gemm(a, wp, debug=True)
    ref, racc = _np_w4a4(lay.x, lay.w)
    assert (acc == racc).all()
    np.testing.assert_allclose(y, ref, rtol=1e-6, atol=1e-6)


def test_all_outliers_is_bf16_gemm():
    lay = synth.tiny()
    mp = -(np.arange(lay.k, dtype=np.int32) + 1)
    a = oracle.quantize_split_act(lay.x, mp)
    wp = oracle.pack_weights(lay.w, mp)
    assert a["ldk"] == 0
    y = oracle.dual_gemm(a, wp)
    xb = synth.bf16_bits_to_f32(synth.to_bf16_bits(lay.x)).astype(np.float64)
    wb = synth.bf16_bits_to_f32(synth.to_bf16_bits(lay.w)).astype(np.float64)
    ref = xb @ wb
    np.testing.assert_allclose(y, ref, rtol=1e-6, atol=1e-5 * np.abs(ref).max())


def test_integer_grid_is_exact():
    """Inputs on the int4 grid with every row / column absmax exactly 7: the
    quantisation is the identity (inv = s = 1), so Y must equal X.W exactly;
    outlier channels carry integers exactly representable in bf16."""
    rng = np.random.default_rng(21)
    m, k, n = 24, 300, 40
    x = rng.integers(-7, 8, (m, k)).astype(np.float32)
    w = rng.integers(-7, 8, (k, n)).astype(np.float32)
    out = np.array([3, 77, 150, 299])
    low = np.setdiff1d(np.arange(k), out)
    x[:, low[0]] = 7
    w[low[1], :] = -7
    x[:, out] = rng.integers(-200, 200, (m, len(out)))
    w[out, :] = rng.integers(-100, 100, (len(out), n))
    mp = np.zeros(k, np.int32)
    mp[low] = np.arange(len(low))
    mp[out] = -(np.arange(len(out)) + 1)
    a = oracle.quantize_split_act(x, mp)
    wp = oracle.pack_weights(w, mp)
    assert (a["s_x"] == 1).all() and (wp["s_w"] == 1).all()
    y = oracle.dual_gemm(a, wp)
    assert (y.astype(np.float64) == x.astype(np.float64) @ w.astype(np.float64)).all()


def _np_unpack_i4(packed, k_low):
    lo = (packed & 0xF).astype(np.int64)
    hi = (packed >> 4).astype(np.int64)
    nib = np.stack([lo, hi], -1).reshape(packed.shape[0], -1)[:, :k_low]
    return np.where(nib == 8, 0, np.where(nib > 8, nib - 16, nib))


def test_low_accumulators_equal_int64_matmul():
    lay = synth.tiny()
    idx, mp, _, _ = oracle.select_channels(lay.x_cal, lay.w, lay.k_out)
    a = oracle.quantize_split_act(lay.x, mp)
    wp = oracle.pack_weights(lay.w, mp)
    _, acc, _, _ = oracle.dual_gemm(a, wp, debug=True)
    cx = _np_unpack_i4(a["x_low"], a["k_low"])
    cw = _np_unpack_i4(wp["w_low"], wp["k_low"])
    assert (acc == cx @ cw.T).all()


def test_error_within_quantisation_bound():
    """|Y - X.W| is bounded by the per-element rounding errors: each int4 value
    is off by at most half a step, each bf16 branch value by 2^-9 relative.
    A dropped branch, a transposed operand or a wrong scale breaks it."""
    lay = synth.tiny()
    idx, mp, _, _ = oracle.select_channels(lay.x_cal, lay.w, lay.k_out)
    a = oracle.quantize_split_act(lay.x, mp)
    wp = oracle.pack_weights(lay.w, mp)
    y = oracle.dual_gemm(a, wp).astype(np.float64)
    x, w = lay.x.astype(np.float64), lay.w.astype(np.float64)
    low = mp >= 0
    sx = a["s_x"].astype(np.float64)[:, None]
    sw = wp["s_w"].astype(np.float64)[None, :]
    xl, wl = np.abs(x[:, low]), np.abs(w[low, :])
    bound_low = 0.5 * sx * wl.sum(0)[None, :] + 0.5 * (xl @ np.ones_like(wl)) * sw \
        + 0.25 * low.sum() * sx * sw
    xh, wh = np.abs(x[:, ~low]), np.abs(w[~low, :])
    bound_hi = 2 * 2.0 ** -8 * (xh @ wh)
    err = np.abs(y - x @ w)
    assert (err <= bound_low + bound_hi + 1e-6).all()
    # and the split actually matters: without the branch the error is far larger
    assert np.abs(x[:, ~low] @ w[~low, :]).max() > 10 * err.max()


def test_token_permutation_equivariance():
    lay = synth.tiny()
    idx, mp, _, _ = oracle.select_channels(lay.x_cal, lay.w, lay.k_out)
    wp = oracle.pack_weights(lay.w, mp)
    perm = np.random.default_rng(1).permutation(lay.m)
    y0 = oracle.dual_gemm(oracle.quantize_split_act(lay.x, mp), wp)
    y1 = oracle.dual_gemm(oracle.quantize_split_act(np.ascontiguousarray(lay.x[perm]), mp), wp)
    assert (y1 == y0[perm]).all()


def test_channel_permutation_invariance():
    lay = synth.tiny()
    perm = np.random.default_rng(2).permutation(lay.k)
    ys = []
    for p in (np.arange(lay.k), perm):
        xc, x, w = lay.x_cal[:, p].copy(), lay.x[:, p].copy(), lay.w[p].copy()
        idx, mp, _, _ = oracle.select_channels(xc, w, lay.k_out)
        ys.append(oracle.dual_gemm(oracle.quantize_split_act(x, mp), oracle.pack_weights(w, mp)))
    # the low sums are exact integers in any order; only the fp64 branch sum reorders
    np.testing.assert_allclose(ys[0], ys[1], rtol=1e-6, atol=1e-6)


def test_zero_row_gives_branch_only():
    lay = synth.tiny()
    idx, mp, _, _ = oracle.select_channels(lay.x_cal, lay.w, lay.k_out)
    x = lay.x.copy()
    x[3, mp >= 0] = 0.0
    a = oracle.quantize_split_act(x, mp)
    assert a["s_x"][3] == 0 and not a["x_low"][3].any()
    wp = oracle.pack_weights(lay.w, mp)
    y = oracle.dual_gemm(a, wp)
    xb = synth.bf16_bits_to_f32(synth.to_bf16_bits(x[3, idx])).astype(np.float64)
    wb = synth.bf16_bits_to_f32(synth.to_bf16_bits(lay.w[idx])).astype(np.float64)
    np.testing.assert_allclose(y[3], xb @ wb, rtol=1e-6, atol=1e-6)


# ------------------------------------------------------------------ branch variants
def test_fp8_branch_all_channels_bound():
    """FP8 fallback (OSC abstract) applied to every channel: Y approximates X.W
    within E4M3's relative step (2^-3 at worst per operand, 2^-4 after RNE)."""
    lay = synth.tiny()
    mp = -(np.arange(lay.k, dtype=np.int32) + 1)
    a = oracle.quantize_split_act(lay.x, mp, branch="fp8")
    wp = oracle.pack_weights(lay.w, mp, branch="fp8")
    y = oracle.dual_gemm(a, wp).astype(np.float64)
    x, w = lay.x.astype(np.float64), lay.w.astype(np.float64)
    # per value: relative error <= 2^-4 for normals, plus an absolute subnormal floor
    sx = a["s_xo"].astype(np.float64)[:, None]
    sw = wp["s_wo"].astype(np.float64)[None, :]
    ex = 2.0 ** -4 * np.abs(x) + sx * 2.0 ** -10
    ew = 2.0 ** -4 * np.abs(w) + sw * 2.0 ** -10
    bound = ex @ np.abs(w) + np.abs(x) @ ew + ex @ ew
    assert (np.abs(y - x @ w) <= bound + 1e-9).all()


def test_int8_branch_accumulator_exact():
    lay = synth.tiny()
    idx, mp, _, hd = oracle.select_channels(lay.x_cal, lay.w, lay.k_out)
    a = oracle.quantize_split_act(lay.x, mp, low="i8", branch="i8")
    wp = oracle.pack_weights_sq(lay.w, mp, hd, (lay.k - lay.k_out) // 8)
    _, al, asp, ao = oracle.dual_gemm(a, wp, debug=True)
    xo = a["x_out"].view(np.int8).astype(np.int64)[:, : lay.k_out]
    wo = wp["w_out"].view(np.int8).astype(np.int64)[:, : lay.k_out]
    assert (ao == xo @ wo.T).all()
    # low and masked accumulators from an independent decode of the format
    k_low = a["k_low"]
    cx = a["x_low"].view(np.int8).astype(np.int64)[:, :k_low]
    lo = (wp["w_low"] & 0xF).astype(np.int64)
    hi = (wp["w_low"] >> 4).astype(np.int64)
    nib = np.stack([lo, hi], -1).reshape(lay.n, -1)[:, :k_low]
    marked = nib == 8
    cw = np.where(marked, 0, np.where(nib > 8, nib - 16, nib))
    assert (al == cx @ cw.T).all()
    dense_sp = np.zeros_like(cw)
    for nn in range(lay.n):
        dense_sp[nn, np.nonzero(marked[nn])[0]] = wp["sq_val"][nn]
    assert (asp == cx @ dense_sp.T).all()


def test_sq_mask_is_top_key_per_row():
    lay = synth.tiny()
    idx, mp, _, hd = oracle.select_channels(lay.x_cal, lay.w, lay.k_out)
    nnz = (lay.k - lay.k_out) // 8
    wp = oracle.pack_weights_sq(lay.w, mp, hd, nnz)
    low = np.nonzero(mp >= 0)[0]
    lo = (wp["w_low"] & 0xF)
    hi = (wp["w_low"] >> 4)
    nib = np.stack([lo, hi], -1).reshape(lay.n, -1)[:, : len(low)]
    for nn in range(0, lay.n, 17):
        key = lay.w[low, nn].astype(np.float64) ** 2 * hd[low].astype(np.float64)
        top = np.lexsort((np.arange(len(low)), -key))[:nnz]
        assert set(np.nonzero(nib[nn] == 8)[0].tolist()) == set(top.tolist())
