"""Run the GPU path (through the C ABI) and the CPU oracle on the same seeded
inputs, stage by stage, and compare.

Integer and byte stages must match bit for bit; the fp32 output must satisfy,
for every token row m:  max_n |y_gpu - y_oracle| <= 1e-3 * max_n |y_oracle|.
The oracle computes every stage from the raw inputs itself; nothing it
consumes comes from the GPU.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from outlier_split_mixed_amd import synth

Y_TOL = 1e-3


def x_inputs(lay, x_dtype):
    """(oracle array, oracle fmt, torch device tensor) for the activations."""
    if x_dtype == "bf16":
        bits = synth.to_bf16_bits(lay.x)
        xt = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
        return bits, "bf16", xt
    return lay.x, "f32", torch.from_numpy(lay.x).cuda()


def assert_rows_close(y_gpu, y_orc, what=""):
    y_gpu = np.asarray(y_gpu, np.float64)
    y_orc = np.asarray(y_orc, np.float64)
    assert y_gpu.shape == y_orc.shape
    scale = np.abs(y_orc).max(axis=1, keepdims=True)
    err = np.abs(y_gpu - y_orc)
    bad = err > Y_TOL * scale
    if bad.any():
        r, c = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: y mismatch at row {r} col {c}: gpu {y_gpu[r, c]} oracle "
                             f"{y_orc[r, c]} (row max {scale[r, 0]}), {bad.sum()} bad elements")
    return float((err / np.maximum(scale, 1e-30)).max())


def f32_bits_equal(a, b):
    a = np.ascontiguousarray(a, np.float32).view(np.uint32)
    b = np.ascontiguousarray(b, np.float32).view(np.uint32)
    return np.array_equal(a, b)


def sample_rows(m, count, seed=0):
    """Deterministic row sample that always contains the first and last row."""
    if m <= count:
        return np.arange(m, dtype=np.int64)
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, m - 1), size=count - 2, replace=False)
    return np.sort(np.concatenate([[0, m - 1], mid])).astype(np.int64)


def tile_band_rows(m, tile=256):
    """Every row of the second 256-row tile band (every row position a tile
    has) and of the last, possibly partial, tile."""
    band = np.arange(tile, min(2 * tile, m))
    last = np.arange((m - 1) // tile * tile, m)
    return np.unique(np.concatenate([band, last])).astype(np.int64)


def e2m3_rows_equal(got, want, m):
    """K-blocked E2M3 storages equal on every byte of the m real rows (the
    activation kernel never writes the padding rows)."""
    rb = oracle.e2m3_row_of_byte(got.shape[0], got.shape[1] * 32)
    keep = rb < m
    return got.shape == want.shape and np.array_equal(got[keep], want[keep])


def _decode_i4(packed, k_low):
    lo = (packed & 0xF).astype(np.int8)
    hi = (packed >> 4).astype(np.int8)
    nib = np.stack([lo, hi], -1).reshape(packed.shape[0], -1)[:, :k_low]
    return np.where(nib > 7, nib - 16, nib).astype(np.float32)


def check_band(acc_gpu, y_gpu, o_a, o_w, rows, what):
    """At full size, on whole tile bands: every GPU int32 low sum equals the
    exact dot product of the codes (decoded from the packed bytes already
    matched bit for bit against the oracle; float32 products and sums of
    integers below 2^24 are exact in any order), and every Y element is
    within tolerance of s_x*s_w*acc + bf16 branch evaluated in fp64."""
    k_low = o_a["k_low"]
    cx = _decode_i4(o_a["x_low"][rows], k_low)
    cw = _decode_i4(o_w["w_low"], k_low)
    acc = cx @ cw.T
    assert float(np.abs(acc).max(initial=0)) < 2 ** 24
    assert np.array_equal(acc_gpu[rows].astype(np.int64), acc.astype(np.int64)), f"{what}: band sums"
    y = (o_a["s_x"][rows].astype(np.float64)[:, None] * o_w["s_w"].astype(np.float64)[None, :]
         * acc.astype(np.float64))
    if o_a["k_out"]:
        xo = synth.bf16_bits_to_f32(o_a["x_out"][rows].view(np.uint16)).astype(np.float64)
        wo = synth.bf16_bits_to_f32(o_w["w_out"].view(np.uint16)).astype(np.float64)
        y += xo @ wo.T
    return assert_rows_close(y_gpu[rows], y, what + " (band)")


def run_layer(sqf, lay, k_out, branch="bf16", x_dtype="bf16", rows=None, check_select=True,
              debug=True, tile="auto", low="i4", band=None):
    """Full path for one layer on both sides.  Returns a dict of comparison stats.
    low="i4e2m3": the int4 codes in the K-blocked 6-bit layout (FP6 GEMM); its
    bytes are compared with the oracle's re-encoding of its own packed int4."""
    stats = {}
    # ---------------- GPU ----------------
    x_cal = torch.from_numpy(lay.x_cal).cuda()
    w = torch.from_numpy(lay.w).cuda()
    idx, mp, score, hdiag = sqf.sqf_select_channels(x_cal, w, k_out)
    wts = sqf.sqf_pack_weights(w, mp, branch=branch, low=low)
    ox, ofmt, xt = x_inputs(lay, x_dtype)
    acts = sqf.alloc_acts(lay.m, lay.k - k_out, k_out, branch=branch, low=low)
    sqf.sqf_quantize_split_act(xt, mp, acts)
    out = sqf.sqf_dual_gemm(acts, wts, debug=debug, tile=tile)
    y, acc = (out[0], out[1]) if debug else (out, None)
    # the launch that timing uses (no accumulator dump) is checked as well
    y_fast = sqf.sqf_dual_gemm(acts, wts, tile=tile) if debug else y
    torch.cuda.synchronize()
    del w, x_cal
    # ---------------- oracle ----------------
    o_idx, o_mp, o_score, o_hd = oracle.select_channels(lay.x_cal, lay.w, k_out)
    if check_select:
        assert np.array_equal(idx.cpu().numpy(), o_idx), "outlier channel set differs"
        assert np.array_equal(mp.cpu().numpy(), o_mp), "channel map differs"
        assert np.array_equal(score.cpu().numpy().view(np.uint64), o_score.view(np.uint64)), \
            "fp64 scores differ"
        assert f32_bits_equal(hdiag.cpu().numpy(), o_hd), "hdiag differs"
    o_w = oracle.pack_weights(lay.w, o_mp, branch=branch)
    if low == "i4e2m3":
        want = oracle.i4x2_to_e2m3(o_w["w_low"], oracle.pad_rows(lay.n))
        assert np.array_equal(wts.t["w_low"].cpu().numpy(), want), "6-bit w_low differs"
    else:
        assert np.array_equal(wts.t["w_low"][0].cpu().numpy(), o_w["w_low"]), "packed w_low differs"
    assert f32_bits_equal(wts.t["s_w"][0].cpu().numpy(), o_w["s_w"]), "s_w differs"
    if k_out:
        g = wts.t["w_out"][0].cpu().numpy().view(o_w["w_out"].dtype)
        assert np.array_equal(g, o_w["w_out"]), "branch weights differ"
        if branch != "bf16":
            assert f32_bits_equal(wts.t["s_wo"][0].cpu().numpy(), o_w["s_wo"]), "s_wo differs"
    o_a = oracle.quantize_split_act(ox, o_mp, branch=branch, x_fmt=ofmt)
    if low == "i4e2m3":
        want = oracle.i4x2_to_e2m3(o_a["x_low"], oracle.pad_rows(lay.m))
        got = acts.t["x_low"].cpu().numpy()
        assert got.shape == want.shape
        # rows past m are never written: compare the m real rows
        assert e2m3_rows_equal(got, want, lay.m), "6-bit x_low differs"
    else:
        assert np.array_equal(acts.t["x_low"].cpu().numpy(), o_a["x_low"]), "packed x_low differs"
    assert f32_bits_equal(acts.t["s_x"].cpu().numpy(), o_a["s_x"]), "s_x differs"
    if k_out:
        g = acts.t["x_out"].cpu().numpy().view(o_a["x_out"].dtype)
        assert np.array_equal(g, o_a["x_out"]), "branch activations differ"
        if branch != "bf16":
            assert f32_bits_equal(acts.t["s_xo"].cpu().numpy(), o_a["s_xo"]), "s_xo differs"
    if rows is None:
        rows = np.arange(lay.m, dtype=np.int64)
    o_y, o_acc, _, _ = oracle.dual_gemm(o_a, o_w, rows=rows, debug=True)
    yg = y.cpu().numpy()[rows]
    if debug:
        ag = acc.cpu().numpy()[rows].astype(np.int64)
        assert np.array_equal(ag, o_acc), "int32 low accumulators differ"
    stats["max_rel_err"] = assert_rows_close(yg, o_y, lay.name)
    if debug:
        assert_rows_close(y_fast.cpu().numpy()[rows], o_y, lay.name + " (no debug outputs)")
    stats["rows_checked"] = len(rows)
    if band is not None:
        assert debug and branch == "bf16"
        yf = y_fast.cpu().numpy()
        stats["band_rows"] = len(band)
        stats["band_max_rel_err"] = check_band(acc.cpu().numpy(), yf, o_a, o_w, band, lay.name)
    return stats, y


# ---------------------------------------------------------------- MXFP4 low path
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0])


def _mx_rows(codes_kb, scales_kb, rows):
    """K-blocked MXFP4 storage -> (codes [P][pad/2], scales [P][pad/32]) by row."""
    nkb = codes_kb.shape[0]
    c = codes_kb.transpose(1, 3, 0, 2, 4).reshape(-1, nkb * 64)[:rows]
    s = scales_kb.transpose(1, 4, 3, 0, 2).reshape(-1, nkb * 4)[:rows]
    return c, s


def _mx_dequant(codes, scales, k_low):
    """Packed E2M1 rows and their E8M0 scales -> float64 values [rows][k_low]."""
    nib = np.stack([codes & 0xF, codes >> 4], -1).reshape(codes.shape[0], -1)[:, :k_low]
    sc = np.repeat(scales.astype(np.int64), 32, axis=1)[:, :k_low]
    return E2M1[nib] * np.ldexp(1.0, sc - 127)


def run_layer_mx(sqf, lay, k_out, x_dtype="bf16", rows=None, band=None, check_select=True):
    """The MXFP4 low path for one layer on both sides: selection, the K-blocked
    codes and block scales of weights and activations (bit for bit, real rows),
    the bf16 branch, and Y on the sampled rows (oracle, fp64) and on the band
    rows (the plain product of the dequantised operands already matched bit
    for bit, fp64)."""
    stats = {}
    x_cal = torch.from_numpy(lay.x_cal).cuda()
    w = torch.from_numpy(lay.w).cuda()
    idx, mp, score, hdiag = sqf.sqf_select_channels(x_cal, w, k_out)
    wts = sqf.sqf_pack_weights(w, mp, low="mxfp4")
    ox, ofmt, xt = x_inputs(lay, x_dtype)
    acts = sqf.alloc_acts(lay.m, lay.k - k_out, k_out, low="mxfp4")
    sqf.sqf_quantize_split_act(xt, mp, acts)
    y = sqf.sqf_dual_gemm(acts, wts)
    torch.cuda.synchronize()
    del w, x_cal
    o_idx, o_mp, _, _ = oracle.select_channels(lay.x_cal, lay.w, k_out)
    if check_select:
        assert np.array_equal(mp.cpu().numpy(), o_mp), "channel map differs"
    o_w = oracle.pack_weights_mx(lay.w, o_mp)
    wc, ws = oracle.mx_storage(o_w["w_low"], o_w["s_wb"], oracle.pad_rows(lay.n))
    assert np.array_equal(wts.t["w_low"].cpu().numpy(), wc), "MXFP4 w_low differs"
    assert np.array_equal(wts.t["s_wb"].cpu().numpy(), ws), "MXFP4 weight scales differ"
    if k_out:
        assert np.array_equal(wts.t["w_out"][0].cpu().numpy().view(np.uint16), o_w["w_out"]), \
            "branch weights differ"
    o_a = oracle.quantize_split_act_mx(ox, o_mp, x_fmt=ofmt)
    if o_a["pad"]:
        gc, gs = _mx_rows(acts.t["x_low"].cpu().numpy(), acts.t["s_xb"].cpu().numpy(), lay.m)
        assert np.array_equal(gc, o_a["x_low"]), "MXFP4 x_low differs"
        assert np.array_equal(gs, o_a["s_xb"]), "MXFP4 activation scales differ"
    if k_out:
        assert np.array_equal(acts.t["x_out"].cpu().numpy().view(np.uint16), o_a["x_out"]), \
            "branch activations differ"
    if rows is None:
        rows = np.arange(lay.m, dtype=np.int64)
    o_y = oracle.dual_gemm_mx(o_a, o_w, rows=rows)
    yg = y.cpu().numpy()
    stats["max_rel_err"] = assert_rows_close(yg[rows], o_y, lay.name + " (mxfp4)")
    stats["rows_checked"] = len(rows)
    if band is not None:
        k_low = o_a["k_low"]
        xq = _mx_dequant(o_a["x_low"][band], o_a["s_xb"][band], k_low)
        wq = _mx_dequant(o_w["w_low"], o_w["s_wb"], k_low)
        yb = xq @ wq.T
        if k_out:
            xo = synth.bf16_bits_to_f32(o_a["x_out"][band]).astype(np.float64)
            wo = synth.bf16_bits_to_f32(o_w["w_out"]).astype(np.float64)
            yb += xo @ wo.T
        stats["band_rows"] = len(band)
        stats["band_max_rel_err"] = assert_rows_close(yg[band], yb, lay.name + " (mxfp4 band)")
    return stats, y
