"""GPU parity at small and ragged sizes: every stage of the HIP path, called
through the C ABI, against the CPU oracle on the same seeded inputs.

Bit-exact: outlier set, channel map, fp64 scores, hdiag, packed int4 bytes,
fp32 scale patterns, branch codes, int32 low-path accumulators.  Tolerance:
per row, max |y_gpu - y_oracle| <= 1e-3 * max |y_oracle|.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle
from outlier_split_mixed_amd import synth

from harness import assert_rows_close, f32_bits_equal, run_layer, x_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sqf():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from outlier_split_mixed_amd import sqf as mod

    return mod


def _ragged(m=300, k=1000, n=520, n_scaled=37, seed=77, factor="loguniform"):
    return synth.draw_layer("ragged", seed, 0, m, k, n, 128, n_scaled, factor=factor)


def _print(*a):
    print(*a, flush=True)


def test_tiny_fp32_input(sqf):
    lay = synth.tiny()
    st, _ = run_layer(sqf, lay, lay.k_out, x_dtype="f32")
    _print("tiny", st)


@pytest.mark.parametrize("tile", ["0", "1", "2"])
def test_tiny_m_and_n_every_tile(sqf, tile):
    """7 tokens x 5 outputs: one partial tile on every configuration, almost
    every row and column of it past the ends."""
    lay = synth.draw_layer("tinymn", 1030, 0, 7, 512, 5, 32, 32)
    os.environ["SQF_GEMM_TILE"] = tile
    try:
        st, _ = run_layer(sqf, lay, lay.k_out)
    finally:
        del os.environ["SQF_GEMM_TILE"]
    _print("tiny m n", tile, st)


@pytest.mark.parametrize("k", [1000, 4096, 16384])
def test_fp32_input_row_widths(sqf, k):
    """fp32 activations (not only bf16) through the activation layouts for
    narrow, medium and wide rows, ragged M and N."""
    lay = synth.draw_layer("f32in", 1020 + k % 97, 0, 45, k, 136, 64, max(1, k // 16), x_dtype="f32")
    st, _ = run_layer(sqf, lay, lay.k_out, x_dtype="f32")
    _print("fp32 input", k, st)


@pytest.mark.parametrize("k", [512, 40960])
def test_row_width_extremes(sqf, k):
    """The narrowest and widest rows the activation kernel lays out differently
    (one 8-channel chunk per thread, and eight), ragged M and N."""
    lay = synth.draw_layer("wide", 1010, k, 37, k, 72, 96, k // 16)
    st, _ = run_layer(sqf, lay, lay.k_out)
    _print("row width", k, st)


@pytest.mark.parametrize("tile,branch", [("0", "bf16"), ("1", "bf16"), ("2", "bf16"),
                                         ("0", "fp8"), ("1", "fp8"), ("2", "fp8")])
def test_ragged_every_tile_config(sqf, tile, branch):
    """M, N and K_low are not multiples of any tile; K_out is not a multiple of 64."""
    lay = _ragged()
    os.environ["SQF_GEMM_TILE"] = tile
    try:
        st, _ = run_layer(sqf, lay, lay.k_out, branch=branch)
    finally:
        del os.environ["SQF_GEMM_TILE"]
    _print("ragged tile", tile, branch, st)


@pytest.mark.parametrize("tile", ["0", "1"])
def test_e4m3_every_channel_each_tile(sqf, tile):
    """Every channel in the E4M3 branch (a long branch loop, no low stage) on
    the 256x256 and 128x128 tiles."""
    lay = _ragged(m=300, k=1024, n=520, n_scaled=64, seed=83)
    os.environ["SQF_GEMM_TILE"] = tile
    try:
        st, _ = run_layer(sqf, lay, lay.k, branch="fp8")
    finally:
        del os.environ["SQF_GEMM_TILE"]
    _print("k_out=k fp8 tile", tile, st)


@pytest.mark.parametrize("branch", ["bf16", "fp8"])
def test_ragged_branch_types(sqf, branch):
    lay = _ragged(m=257, k=1536, n=384, n_scaled=96, seed=78)
    st, _ = run_layer(sqf, lay, lay.k_out, branch=branch)
    _print("branch", branch, st)


def test_no_outliers_is_w4a4(sqf):
    lay = _ragged(m=130, k=512, n=200, n_scaled=0, seed=79, factor=1.0)
    st, _ = run_layer(sqf, lay, 0)
    _print("k_out=0", st)


@pytest.mark.parametrize("branch", ["bf16", "fp8"])
def test_all_outliers_is_branch_gemm(sqf, branch):
    lay = _ragged(m=96, k=256, n=136, n_scaled=16, seed=80)
    st, _ = run_layer(sqf, lay, lay.k, branch=branch)
    _print("k_out=k", branch, st)


def test_outlier_fraction_one_half(sqf):
    lay = _ragged(m=200, k=2048, n=256, n_scaled=128, seed=81)
    st, _ = run_layer(sqf, lay, 1024)
    _print("f=1/2", st)


def test_zero_token_rows_and_single_row(sqf):
    lay = _ragged(m=65, k=512, n=96, n_scaled=32, seed=82)
    lay.x[5] = 0.0  # every channel zero: scale 0, codes 0
    lay.x[9, :] = 0.0
    lay.x[9, lay.scaled] = 3.0  # low channels zero, outliers non-zero
    st, _ = run_layer(sqf, lay, lay.k_out)
    one = synth.draw_layer("one", 83, 0, 1, 512, 64, 64, 32)
    run_layer(sqf, one, one.k_out)


@pytest.mark.parametrize("k,n", [(2500, 517), (1030, 1536)])
def test_selection_ties_and_ragged_rows(sqf, k, n):
    """Groups of channels with equal scores straddle the k_out boundary (the
    lower channel must win), K spans several rank slices with a ragged last
    one, and the weight rows are either not a multiple of 4 long (scalar
    loads) or several 512-column stages long.  The map, idx, fp64 scores and
    hdiag must match the oracle bit for bit; the packed weights too."""
    lay = synth.draw_layer("ties", 88, 0, 8, k, n, 40, k // 16, draw_x=False)
    x_cal, w = lay.x_cal.copy(), lay.w.copy()
    k_out = k // 16
    o_score = oracle.select_channels(x_cal, w, k_out)[2]
    order = np.argsort(-o_score, kind="stable")
    # copy channel order[k_out - 1] into four channels around the boundary and
    # channel order[3] into two others: equal columns of x_cal and equal rows of
    # W give equal scores
    src_a, src_b = int(order[k_out - 1]), int(order[3])
    for dst in (int(order[k_out - 3]), int(order[k_out]), int(order[k_out + 2]), int(order[-1])):
        x_cal[:, dst], w[dst] = x_cal[:, src_a], w[src_a]
    for dst in (int(order[k_out + 5]), int(order[0])):
        x_cal[:, dst], w[dst] = x_cal[:, src_b], w[src_b]
    idx, mp, score, hdiag = sqf.sqf_select_channels(torch.from_numpy(x_cal).cuda(),
                                                    torch.from_numpy(w).cuda(), k_out)
    wts = sqf.sqf_pack_weights(torch.from_numpy(w).cuda(), mp)
    torch.cuda.synchronize()
    o_idx, o_mp, o_sc, o_hd = oracle.select_channels(x_cal, w, k_out)
    sc = o_sc[o_idx]
    assert (sc == o_sc[src_a]).any() and (o_sc[np.setdiff1d(np.arange(k), o_idx)] == o_sc[src_a]).any(), \
        "the tie group must straddle the boundary"
    assert np.array_equal(score.cpu().numpy().view(np.uint64), o_sc.view(np.uint64))
    assert np.array_equal(idx.cpu().numpy(), o_idx)
    assert np.array_equal(mp.cpu().numpy(), o_mp)
    assert f32_bits_equal(hdiag.cpu().numpy(), o_hd)
    o_w = oracle.pack_weights(w, o_mp)
    assert np.array_equal(wts.t["w_low"][0].cpu().numpy(), o_w["w_low"])
    assert f32_bits_equal(wts.t["s_w"][0].cpu().numpy(), o_w["s_w"])
    assert np.array_equal(wts.t["w_out"][0].cpu().numpy().view(o_w["w_out"].dtype), o_w["w_out"])
    _print("ties", k, n, "boundary score", o_sc[src_a])


@pytest.mark.parametrize("tile,branch", [("0", "bf16"), ("1", "bf16"), ("2", "bf16"), ("1", "fp8")])
def test_bf16_output(sqf, tile, branch):
    """bf16 Y: each element is the round-to-nearest-even of the fp32 Y the
    fp32 launch writes (same accumulators, same epilogue arithmetic), within
    the fp32 tolerance plus one bf16 step of the oracle; both the 16-byte
    store path and, with an odd row stride, the element-wise one (the
    columns past n stay untouched)."""
    lay = _ragged(m=300, k=1000, n=520, n_scaled=37, seed=95)
    x_cal = torch.from_numpy(lay.x_cal).cuda()
    w = torch.from_numpy(lay.w).cuda()
    _, mp, _, _ = sqf.sqf_select_channels(x_cal, w, lay.k_out)
    wts = sqf.sqf_pack_weights(w, mp, branch=branch)
    ox, ofmt, xt = x_inputs(lay, "bf16")
    acts = sqf.alloc_acts(lay.m, lay.k - lay.k_out, lay.k_out, branch=branch)
    sqf.sqf_quantize_split_act(xt, mp, acts)
    os.environ["SQF_GEMM_TILE"] = tile
    try:
        y32 = sqf.sqf_dual_gemm(acts, wts)
        yb = sqf.sqf_dual_gemm(acts, wts, y_dtype="bf16")
        # the output-type entry point with SQF_F32 is the plain fp32 call
        y32b = torch.empty_like(y32)
        da, dw = acts.desc(), wts.desc()
        assert sqf._lib.sqf_dual_gemm_y(ctypes.byref(da), ctypes.byref(dw), ctypes.c_void_p(y32b.data_ptr()),
                                        sqf.SQF_F32, y32b.stride(0),
                                        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) == 0
        big = torch.full((lay.m, lay.n + 3), float("nan"), dtype=torch.bfloat16, device="cuda")
        sqf.sqf_dual_gemm(acts, wts, y=big[:, :lay.n], y_dtype="bf16")
    finally:
        del os.environ["SQF_GEMM_TILE"]
    torch.cuda.synchronize()
    assert torch.equal(y32b.view(torch.int32), y32.view(torch.int32))
    want = _bf16_bits(y32.to(torch.bfloat16))
    assert np.array_equal(_bf16_bits(yb), want)
    assert np.array_equal(_bf16_bits(big[:, :lay.n]), want)
    assert torch.isnan(big[:, lay.n:]).all()
    o_mp = oracle.select_channels(lay.x_cal, lay.w, lay.k_out)[1]
    o_a = oracle.quantize_split_act(ox, o_mp, branch=branch, x_fmt=ofmt)
    o_w = oracle.pack_weights(lay.w, o_mp, branch=branch)
    o_y = oracle.dual_gemm(o_a, o_w)
    _assert_bf16_close(yb.float().cpu().numpy(), o_y, f"bf16 Y tile {tile} {branch}")
    _print("bf16 Y", tile, branch)


def test_m_zero_is_a_no_op(sqf):
    acts = sqf.alloc_acts(0, 480, 32)
    w = sqf.alloc_weights(512, 64, 32)
    x = torch.zeros((0, 512), dtype=torch.bfloat16, device="cuda")
    mp = torch.zeros(512, dtype=torch.int32, device="cuda")
    sqf.sqf_quantize_split_act(x, mp, acts)
    y = sqf.sqf_dual_gemm(acts, w)
    assert y.shape == (0, 64)


def test_deterministic_and_canary(sqf):
    """Two runs are bitwise equal; bytes past every output's extent are untouched."""
    lay = _ragged(m=190, k=768, n=200, n_scaled=48, seed=84)
    x_cal = torch.from_numpy(lay.x_cal).cuda()
    w = torch.from_numpy(lay.w).cuda()
    idx, mp, _, _ = sqf.sqf_select_channels(x_cal, w, lay.k_out)
    wts = sqf.sqf_pack_weights(w, mp)
    _, _, xt = x_inputs(lay, "bf16")
    acts = sqf.alloc_acts(lay.m, lay.k - lay.k_out, lay.k_out)
    canary = 0x5A
    # y with a wider leading dimension: the columns past n must stay untouched
    ldy = lay.n + 24
    ys = []
    for _ in range(2):
        big = torch.full((lay.m + 3, ldy), float("nan"), device="cuda")
        sqf.sqf_quantize_split_act(xt, mp, acts)
        y = big[: lay.m]
        sqf.sqf_dual_gemm(acts, wts, y=y)
        torch.cuda.synchronize()
        b = big.cpu().numpy()
        assert np.isnan(b[:, lay.n:]).all() and np.isnan(b[lay.m:]).all()
        ys.append(b[: lay.m, : lay.n].copy())
    assert np.array_equal(ys[0].view(np.uint32), ys[1].view(np.uint32))
    # activation buffers carved from a larger canary-filled allocation
    ldk, ldo = acts.ldk, acts.ldo
    raw = torch.full((lay.m * ldk + 4096,), canary, dtype=torch.uint8, device="cuda")
    acts.t["x_low"] = raw[: lay.m * ldk].view(lay.m, ldk)
    sqf.sqf_quantize_split_act(xt, mp, acts)
    torch.cuda.synchronize()
    assert (raw[lay.m * ldk:].cpu().numpy() == canary).all()


def test_sq_weight_side_small(sqf):
    """Weight-side SQ-format: int8 activations, int4 weights with reserved
    marks, int8 sparse values, int8 branch; three exact accumulators."""
    lay = _ragged(m=140, k=1280, n=300, n_scaled=80, seed=85)
    _sq_check(sqf, lay, (lay.k - lay.k_out) // 8, "sq small")


@pytest.mark.parametrize("m,k,n,den", [
    (300, 1280, 260, 2),    # ~64 marks per 128-slot stage: past the value window
    (70, 640, 130, 1),      # every low slot marked
    (257, 2048, 129, 64),   # sparse marks, one row past a tile edge on both sides
    (5, 256, 3, 128),       # a few values in total (below one 16-byte block)
])
def test_sq_weight_side_mark_density(sqf, m, k, n, den):
    """Weight-side SQ-format at mark densities and sizes that exercise the
    value windows' edges and the one-by-one path."""
    lay = _ragged(m=m, k=k, n=n, n_scaled=max(1, k // 16), seed=90 + den)
    _print(f"sq density m={m} k={k} n={n} nnz=k_low/{den}")
    _sq_check(sqf, lay, max(1, (lay.k - lay.k_out) // den), f"sq m{m} k{k} n{n} 1/{den}")


@pytest.mark.parametrize("frac", [0.125, 0.9])
def test_sq_weight_side_key_ties(sqf, frac):
    """Many equal importance keys: W on a coarse grid of 5 values (a fifth of
    them zero) and calibration columns repeated in groups of 4 channels, so
    the nnz-th largest key sits inside a group of equal keys (lowest slots
    win); at 0.9 of the low slots the threshold is the zero key itself."""
    lay = _ragged(m=96, k=1024, n=136, n_scaled=64, seed=93)
    lay.w[:] = np.clip(np.rint(lay.w / 0.01), -2, 2).astype(np.float32) * np.float32(0.01)
    for c in range(0, lay.k - 3, 4):
        lay.x_cal[:, c + 1:c + 4] = lay.x_cal[:, c:c + 1]
    nnz = int((lay.k - lay.k_out) * frac)
    _print(f"sq key ties nnz={nnz}")
    _sq_check(sqf, lay, nnz, f"sq ties {frac}")


def _sq_check(sqf, lay, nnz, label):
    k_out = lay.k_out
    k_low = lay.k - k_out
    x_cal = torch.from_numpy(lay.x_cal).cuda()
    w = torch.from_numpy(lay.w).cuda()
    idx, mp, score, hdiag = sqf.sqf_select_channels(x_cal, w, k_out)
    wts = sqf.sqf_pack_weights(w, mp, branch="i8", hdiag=hdiag, sq_nnz=nnz)
    ox, ofmt, xt = x_inputs(lay, "bf16")
    acts = sqf.alloc_acts(lay.m, k_low, k_out, low="i8", branch="i8")
    sqf.sqf_quantize_split_act(xt, mp, acts)
    y, al, asp, ao = sqf.sqf_dual_gemm(acts, wts, debug=True)
    torch.cuda.synchronize()
    o_idx, o_mp, _, o_hd = oracle.select_channels(lay.x_cal, lay.w, k_out)
    assert np.array_equal(mp.cpu().numpy(), o_mp)
    o_w = oracle.pack_weights_sq(lay.w, o_mp, o_hd, nnz)
    assert np.array_equal(wts.t["w_low"][0].cpu().numpy(), o_w["w_low"])
    assert np.array_equal(wts.t["sq_val"].cpu().numpy(), o_w["sq_val"])
    assert f32_bits_equal(wts.t["s_w"][0].cpu().numpy(), o_w["s_w"])
    assert f32_bits_equal(wts.t["s_w8"].cpu().numpy(), o_w["s_w8"])
    assert np.array_equal(wts.t["w_out"][0].cpu().numpy().view(np.int8), o_w["w_out"])
    assert f32_bits_equal(wts.t["s_wo"][0].cpu().numpy(), o_w["s_wo"])
    # tile offsets: marks before each 256-slot tile, from the oracle's bytes
    nib = np.stack([o_w["w_low"] & 0xF, o_w["w_low"] >> 4], -1).reshape(lay.n, -1)
    marks = np.concatenate([np.zeros((lay.n, 1), np.int64), np.cumsum(nib == 8, 1)], 1)
    want = marks[:, ::256]
    assert np.array_equal(wts.t["sq_tile_off"].cpu().numpy(), want)
    o_a = oracle.quantize_split_act(ox, o_mp, low="i8", branch="i8", x_fmt=ofmt)
    assert np.array_equal(acts.t["x_low"].cpu().numpy(), o_a["x_low"])
    assert np.array_equal(acts.t["x_out"].cpu().numpy(), o_a["x_out"])
    assert f32_bits_equal(acts.t["s_x"].cpu().numpy(), o_a["s_x"])
    assert f32_bits_equal(acts.t["s_xo"].cpu().numpy(), o_a["s_xo"])
    o_y, o_al, o_asp, o_ao = oracle.dual_gemm(o_a, o_w, debug=True)
    assert np.array_equal(al.cpu().numpy().astype(np.int64), o_al)
    assert np.array_equal(asp.cpu().numpy().astype(np.int64), o_asp)
    assert np.array_equal(ao.cpu().numpy().astype(np.int64), o_ao)
    assert_rows_close(y.cpu().numpy(), o_y, label)
    y_fast = sqf.sqf_dual_gemm(acts, wts)
    torch.cuda.synchronize()
    assert_rows_close(y_fast.cpu().numpy(), o_y, label + " (timed launch)")


def _moe_small(experts=6, tokens=96, topk=2, hidden=512, inter=256, seed=86):
    return synth.qwen3_moe(seed=seed, experts=experts, tokens=tokens, topk=topk, hidden=hidden,
                           inter=inter, cal_rows=64)


@pytest.mark.parametrize("branch,tile", [("bf16", "1"), ("bf16", "0"), ("fp8", "1"), ("fp8", "0")])
def test_grouped_small_with_empty_group(sqf, branch, tile):
    """Ragged expert groups, one of them empty, on both grouped tile shapes."""
    moe = _moe_small()
    lays = moe.up
    # force one empty expert group
    lays[2] = synth.Layer(name="empty", m=0, k=lays[2].k, n=lays[2].n, k_out=lays[2].k_out,
                          x=lays[2].x[:0], x_cal=lays[2].x_cal, w=lays[2].w,
                          scaled=lays[2].scaled)
    os.environ["SQF_GEMM_TILE"] = tile
    try:
        _grouped_check(sqf, lays, branch, y_bf16=True)
    finally:
        del os.environ["SQF_GEMM_TILE"]


@pytest.mark.parametrize("tile", ["0", "1"])
def test_grouped_many_groups(sqf, tile):
    """600 expert groups of 0-4 rows: more groups than one block-wide pass of
    the tile lookup covers (256 or 512 per pass), many of them empty."""
    moe = synth.qwen3_moe(seed=87, experts=600, tokens=300, topk=2, hidden=256, inter=128,
                          cal_rows=32)
    assert any(l.m == 0 for l in moe.up)
    os.environ["SQF_GEMM_TILE"] = tile
    try:
        _grouped_check(sqf, moe.up, "bf16")
    finally:
        del os.environ["SQF_GEMM_TILE"]


def _bf16_bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy()


def _assert_bf16_close(yb, o_y, label):
    """bf16 Y against the oracle's fp32 Y: the fp32 tolerance plus one bf16
    step (2^-8 relative) for the final rounding."""
    yb = np.asarray(yb, dtype=np.float64)
    o_y = np.asarray(o_y, dtype=np.float64)
    tol = 1e-3 * np.abs(o_y).max(axis=1, keepdims=True) + np.abs(o_y) * 2.0 ** -8
    bad = np.abs(yb - o_y) > tol
    assert not bad.any(), f"{label}: {int(bad.sum())} bf16 outputs beyond tolerance"


def _grouped_check(sqf, lays, branch, rows_per_group=None, y_bf16=False):
    g = len(lays)
    k, n, k_out = lays[0].k, lays[0].n, lays[0].k_out
    counts = [l.m for l in lays]
    off = np.zeros(g + 1, np.int64)
    off[1:] = np.cumsum(counts)
    maps, wst = [], []
    for l in lays:
        idx, mp, _, _ = sqf.sqf_select_channels(torch.from_numpy(l.x_cal).cuda(),
                                                torch.from_numpy(l.w).cuda(), k_out)
        maps.append(mp)
    maps_t = torch.stack(maps)
    w_all = torch.from_numpy(np.stack([l.w for l in lays])).cuda()
    wts = sqf.sqf_pack_weights(w_all, maps_t, branch=branch)
    x = np.concatenate([l.x for l in lays])
    bits = synth.to_bf16_bits(x)
    xt = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    row_off = torch.from_numpy(off).cuda()
    acts = sqf.alloc_acts(int(off[-1]), k - k_out, k_out, branch=branch)
    sqf.sqf_quantize_split_act_grouped(xt, row_off, maps_t, acts)
    y, acc = sqf.sqf_dual_gemm_grouped(acts, wts, row_off, debug=True)
    y_fast = sqf.sqf_dual_gemm_grouped(acts, wts, row_off)
    yb = sqf.sqf_dual_gemm_grouped(acts, wts, row_off, y_dtype="bf16") if y_bf16 else None
    torch.cuda.synchronize()
    if y_bf16:
        # the bf16 launch rounds exactly the values the fp32 launch writes
        assert np.array_equal(_bf16_bits(yb), _bf16_bits(y_fast.to(torch.bfloat16)))
        ybf = yb.float().cpu().numpy()
    yg, ag = y.cpu().numpy(), acc.cpu().numpy().astype(np.int64)
    yf = y_fast.cpu().numpy()
    xl, xo = acts.t["x_low"].cpu().numpy(), acts.t["x_out"].cpu().numpy()
    for e, l in enumerate(lays):
        o_idx, o_mp, _, _ = oracle.select_channels(l.x_cal, l.w, k_out)
        assert np.array_equal(maps_t[e].cpu().numpy(), o_mp)
        o_w = oracle.pack_weights(l.w, o_mp, branch=branch)
        assert np.array_equal(wts.t["w_low"][e].cpu().numpy(), o_w["w_low"])
        if l.m == 0:
            continue
        r0, r1 = off[e], off[e + 1]
        o_a = oracle.quantize_split_act(bits[r0:r1], o_mp, branch=branch, x_fmt="bf16")
        assert np.array_equal(xl[r0:r1], o_a["x_low"])
        assert np.array_equal(xo[r0:r1].view(o_a["x_out"].dtype), o_a["x_out"])
        rows = None if rows_per_group is None else np.unique(
            np.linspace(0, l.m - 1, min(rows_per_group, l.m)).astype(np.int64))
        o_y, o_acc, _, _ = oracle.dual_gemm(o_a, o_w, rows=rows, debug=True)
        sel = np.arange(l.m) if rows is None else rows
        assert np.array_equal(ag[r0:r1][sel], o_acc), f"expert {e} accumulators"
        assert_rows_close(yg[r0:r1][sel], o_y, f"expert {e}")
        assert_rows_close(yf[r0:r1][sel], o_y, f"expert {e} (no debug outputs)")
        if y_bf16:
            _assert_bf16_close(ybf[r0:r1][sel], o_y, f"expert {e} (bf16 Y)")
