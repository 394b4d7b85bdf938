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


def run_layer(sqf, lay, k_out, branch="bf16", x_dtype="bf16", rows=None, check_select=True,
              debug=True):
    """Full path for one layer on both sides.  Returns a dict of comparison stats."""
    stats = {}
    # ---------------- GPU ----------------
    x_cal = torch.from_numpy(lay.x_cal).cuda()
    w = torch.from_numpy(lay.w).cuda()
    idx, mp, score, hdiag = sqf.sqf_select_channels(x_cal, w, k_out)
    wts = sqf.sqf_pack_weights(w, mp, branch=branch)
    ox, ofmt, xt = x_inputs(lay, x_dtype)
    acts = sqf.alloc_acts(lay.m, lay.k - k_out, k_out, branch=branch)
    sqf.sqf_quantize_split_act(xt, mp, acts)
    out = sqf.sqf_dual_gemm(acts, wts, debug=debug)
    y, acc = (out[0], out[1]) if debug else (out, None)
    # the launch that timing uses (no accumulator dump) is checked as well
    y_fast = sqf.sqf_dual_gemm(acts, wts) if debug else y
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
    assert np.array_equal(wts.t["w_low"][0].cpu().numpy(), o_w["w_low"]), "packed w_low differs"
    assert f32_bits_equal(wts.t["s_w"][0].cpu().numpy(), o_w["s_w"]), "s_w differs"
    if k_out:
        g = wts.t["w_out"][0].cpu().numpy().view(o_w["w_out"].dtype)
        assert np.array_equal(g, o_w["w_out"]), "branch weights differ"
        if branch != "bf16":
            assert f32_bits_equal(wts.t["s_wo"][0].cpu().numpy(), o_w["s_wo"]), "s_wo differs"
    o_a = oracle.quantize_split_act(ox, o_mp, branch=branch, x_fmt=ofmt)
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
    return stats, y
