"""GPU parity at small and ragged sizes: every stage of the HIP path, called
through the C ABI, against the CPU oracle on the same seeded inputs.

Bit-exact: outlier set, channel map, fp64 scores, hdiag, packed int4 bytes,
fp32 scale patterns, branch codes, int32 low-path accumulators.  Tolerance:
per row, max |y_gpu - y_oracle| <= 1e-3 * max |y_oracle|.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from outlier_split_mixed_amd import synth

from harness import assert_rows_close, f32_bits_equal, run_layer, run_layer_mx, sample_rows, x_inputs

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


@pytest.mark.parametrize("tile", ["256", "128", "64"])
def test_tiny_m_and_n_every_tile(sqf, tile):
    """7 tokens x 5 outputs: one partial tile on every configuration, almost
    every row and column of it past the ends."""
    lay = synth.draw_layer("tinymn", 1030, 0, 7, 512, 5, 32, 32)
    st, _ = run_layer(sqf, lay, lay.k_out, tile=tile)
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


@pytest.mark.parametrize("tile,branch", [("256", "bf16"), ("128", "bf16"), ("64", "bf16"),
                                         ("128", "fp8"), ("64", "fp8")])
def test_ragged_every_tile_config(sqf, tile, branch):
    """M, N and K_low are not multiples of any tile; K_out is not a multiple of 64."""
    lay = _ragged()
    st, _ = run_layer(sqf, lay, lay.k_out, branch=branch, tile=tile)
    _print("ragged tile", tile, branch, st)


@pytest.mark.parametrize("tile", ["128", "64"])
def test_e4m3_every_channel_each_tile(sqf, tile):
    """Every channel in the E4M3 branch (a long branch loop, no low stage) on
    both of its tiles, 128x128 and 64x64."""
    lay = _ragged(m=300, k=1024, n=520, n_scaled=64, seed=83)
    st, _ = run_layer(sqf, lay, lay.k, branch="fp8", tile=tile)
    _print("k_out=k fp8 tile", tile, st)


def test_forced_tile_the_e4m3_branch_lacks(sqf):
    """The E4M3 branch has no 256x256 tile: forcing one is refused with
    SQF_ERR_UNSUPPORTED (nothing runs), the automatic choice runs 128x128."""
    lay = _ragged(m=64, k=512, n=128, n_scaled=32, seed=88)
    x_cal = torch.from_numpy(lay.x_cal).cuda()
    w = torch.from_numpy(lay.w).cuda()
    _, mp, _, _ = sqf.sqf_select_channels(x_cal, w, lay.k_out)
    wts = sqf.sqf_pack_weights(w, mp, branch="fp8")
    acts = sqf.alloc_acts(lay.m, lay.k - lay.k_out, lay.k_out, branch="fp8")
    sqf.sqf_quantize_split_act(x_inputs(lay, "bf16")[2], mp, acts)
    with pytest.raises(sqf.SqfError) as ei:
        sqf.sqf_dual_gemm(acts, wts, tile="256")
    assert ei.value.status == sqf.SQF_ERR_UNSUPPORTED
    y_auto = sqf.sqf_dual_gemm(acts, wts)
    y_128 = sqf.sqf_dual_gemm(acts, wts, tile="128")
    torch.cuda.synchronize()
    assert torch.equal(y_auto.view(torch.int32), y_128.view(torch.int32))


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


@pytest.mark.parametrize("tile,branch", [("256", "bf16"), ("128", "bf16"), ("64", "bf16"), ("128", "fp8")])
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
    y32 = sqf.sqf_dual_gemm(acts, wts, tile=tile)
    yb = sqf.sqf_dual_gemm(acts, wts, y_dtype="bf16", tile=tile)
    # the output-type entry point with SQF_F32 is the plain fp32 call
    y32b = torch.empty_like(y32)
    da, dw = acts.desc(), wts.desc()
    assert sqf._lib.sqf_dual_gemm_ex(ctypes.byref(da), ctypes.byref(dw), ctypes.c_void_p(y32b.data_ptr()),
                                     sqf.SQF_F32, y32b.stride(0), sqf.TILES[tile], None, None, None,
                                     ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) == 0
    big = torch.full((lay.m, lay.n + 3), float("nan"), dtype=torch.bfloat16, device="cuda")
    sqf.sqf_dual_gemm(acts, wts, y=big[:, :lay.n], y_dtype="bf16", tile=tile)
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


def _sq_check(sqf, lay, nnz, label, bank=0):
    k_out = lay.k_out
    k_low = lay.k - k_out
    x_cal = torch.from_numpy(lay.x_cal).cuda()
    w = torch.from_numpy(lay.w).cuda()
    idx, mp, score, hdiag = sqf.sqf_select_channels(x_cal, w, k_out)
    wts = sqf.sqf_pack_weights(w, mp, branch="i8", hdiag=hdiag, sq_nnz=nnz, sq_bank=bank)
    ox, ofmt, xt = x_inputs(lay, "bf16")
    acts = sqf.alloc_acts(lay.m, k_low, k_out, low="i8", branch="i8")
    sqf.sqf_quantize_split_act(xt, mp, acts)
    y, al, asp, ao = sqf.sqf_dual_gemm(acts, wts, debug=True)
    torch.cuda.synchronize()
    o_idx, o_mp, _, o_hd = oracle.select_channels(lay.x_cal, lay.w, k_out)
    assert np.array_equal(mp.cpu().numpy(), o_mp)
    o_w = oracle.pack_weights_sq(lay.w, o_mp, o_hd, nnz, bank=bank)
    assert np.array_equal(wts.t["w_low"][0].cpu().numpy(), o_w["w_low"])
    assert np.array_equal(wts.t["sq_val"].cpu().numpy(), o_w["sq_val"])
    assert f32_bits_equal(wts.t["s_w"][0].cpu().numpy(), o_w["s_w"])
    assert f32_bits_equal(wts.t["s_w8"].cpu().numpy(), o_w["s_w8"])
    assert np.array_equal(wts.t["w_out"][0].cpu().numpy().view(np.int8), o_w["w_out"])
    assert f32_bits_equal(wts.t["s_wo"][0].cpu().numpy(), o_w["s_wo"])
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
    # the gather once per call into a workspace: the oracle's accumulators,
    # and Y bit-identical to the fused decode's
    ws = _poisoned_workspace(sqf, wts)
    y_ws, al_w, asp_w, ao_w = sqf.sqf_dual_gemm_sq_ws(acts, wts, workspace=ws, debug=True)
    torch.cuda.synchronize()
    assert np.array_equal(al_w.cpu().numpy().astype(np.int64), o_al)
    assert np.array_equal(asp_w.cpu().numpy().astype(np.int64), o_asp)
    assert np.array_equal(ao_w.cpu().numpy().astype(np.int64), o_ao)
    _sq_ws_same(sqf, acts, wts, y, label, ws=ws)


def _poisoned_workspace(sqf, wts):
    """A workspace of the required size filled with 0xA5, so that any byte
    the GEMM reads and the gather did not write shows up in Y."""
    nb = sqf.sqf_sq_workspace_bytes(wts)
    assert nb > 0
    return torch.full((nb,), 0xA5, dtype=torch.uint8, device="cuda")


def _sq_ws_same(sqf, acts, wts, y_ref, label, ws=None):
    """sqf_dual_gemm_sq_ws (timed form) gives the fused call's Y bit for bit,
    on a poisoned workspace and again on the same workspace reused."""
    ws = _poisoned_workspace(sqf, wts) if ws is None else ws
    for i in range(2):
        y_ws = torch.full_like(y_ref, float("nan"))  # a tile nobody wrote shows
        y_ws = sqf.sqf_dual_gemm_sq_ws(acts, wts, y=y_ws, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(y_ws.view(torch.int32), y_ref.view(torch.int32)), f"{label}: workspace call {i}"


@pytest.mark.parametrize("m,k,n", [
    (2048, 640, 2048),   # 128 tiles
    (1000, 640, 6400),   # 200 tiles, ragged last row tile
    (300, 1152, 8300),   # 130 tiles, ragged rows and columns
])
def test_sq_workspace_many_tiles(sqf, m, k, n):
    """The workspace call over a hundred or more tiles (most of a round of
    the GPU): the oracle's three accumulators bit for bit on sampled rows,
    and every accumulator and Y bit-identical to the fused call's, on a
    poisoned workspace, with Y and the dumps prefilled so that a tile nobody
    wrote shows."""
    lay = _ragged(m=m, k=k, n=n, n_scaled=max(1, k // 16), seed=151 + m % 97)
    k_out = lay.k_out
    k_low = lay.k - k_out
    nnz = k_low // 8
    x_cal = torch.from_numpy(lay.x_cal).cuda()
    w = torch.from_numpy(lay.w).cuda()
    _, mp, _, hdiag = sqf.sqf_select_channels(x_cal, w, k_out)
    wts = sqf.sqf_pack_weights(w, mp, branch="i8", hdiag=hdiag, sq_nnz=nnz)
    ox, ofmt, xt = x_inputs(lay, "bf16")
    acts = sqf.alloc_acts(lay.m, k_low, k_out, low="i8", branch="i8")
    sqf.sqf_quantize_split_act(xt, mp, acts)
    y, al, asp, ao = sqf.sqf_dual_gemm(acts, wts, debug=True)
    ws = _poisoned_workspace(sqf, wts)
    for i in range(2):  # the second call reuses the workspace
        # Y and the accumulator dumps start as NaN / -1: a tile nobody wrote shows
        y_w = torch.full_like(y, float("nan"))
        y_w, al_w, asp_w, ao_w = sqf.sqf_dual_gemm_sq_ws(acts, wts, y=y_w, workspace=ws, debug=True)
        torch.cuda.synchronize()
        assert torch.equal(al_w, al) and torch.equal(asp_w, asp) and torch.equal(ao_w, ao), f"call {i}"
        assert torch.equal(y_w.view(torch.int32), y.view(torch.int32)), f"call {i}"
    _sq_ws_same(sqf, acts, wts, y, f"many tiles m{m} n{n}", ws=ws)
    o_mp = mp.cpu().numpy()
    o_w = oracle.pack_weights_sq(lay.w, o_mp, hdiag.cpu().numpy(), nnz)
    o_a = oracle.quantize_split_act(ox, o_mp, low="i8", branch="i8", x_fmt=ofmt)
    rows = sample_rows(lay.m, 6, seed=m)
    o_y, o_al, o_asp, o_ao = oracle.dual_gemm(o_a, o_w, rows=rows, debug=True)
    assert np.array_equal(al_w.cpu().numpy()[rows].astype(np.int64), o_al)
    assert np.array_equal(asp_w.cpu().numpy()[rows].astype(np.int64), o_asp)
    assert np.array_equal(ao_w.cpu().numpy()[rows].astype(np.int64), o_ao)
    assert_rows_close(y_w.cpu().numpy()[rows], o_y, f"many tiles m{m} n{n}")
    _print("sq workspace many tiles ok", m, k, n)


def _moe_small(experts=6, tokens=96, topk=2, hidden=512, inter=256, seed=86):
    return synth.qwen3_moe(seed=seed, experts=experts, tokens=tokens, topk=topk, hidden=hidden,
                           inter=inter, cal_rows=64)


@pytest.mark.parametrize("branch,tile", [("bf16", "128"), ("bf16", "256"), ("fp8", "128")])
def test_grouped_small_with_empty_group(sqf, branch, tile):
    """Ragged expert groups, one of them empty, on both grouped tile shapes."""
    moe = _moe_small()
    lays = moe.up
    # force one empty expert group
    lays[2] = synth.Layer(name="empty", m=0, k=lays[2].k, n=lays[2].n, k_out=lays[2].k_out,
                          x=lays[2].x[:0], x_cal=lays[2].x_cal, w=lays[2].w,
                          scaled=lays[2].scaled)
    _grouped_check(sqf, lays, branch, y_bf16=True, tile=tile)


@pytest.mark.parametrize("tile", ["256", "128"])
def test_grouped_many_groups(sqf, tile):
    """600 expert groups of 0-4 rows: more groups than one block-wide pass of
    the tile lookup covers (256 or 512 per pass), many of them empty."""
    moe = synth.qwen3_moe(seed=87, experts=600, tokens=300, topk=2, hidden=256, inter=128,
                          cal_rows=32)
    assert any(l.m == 0 for l in moe.up)
    _grouped_check(sqf, moe.up, "bf16", tile=tile)


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


def _grouped_check(sqf, lays, branch, rows_per_group=None, y_bf16=False, tile="auto"):
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
    y, acc = sqf.sqf_dual_gemm_grouped(acts, wts, row_off, debug=True, tile=tile)
    y_fast = sqf.sqf_dual_gemm_grouped(acts, wts, row_off, tile=tile)
    yb = sqf.sqf_dual_gemm_grouped(acts, wts, row_off, y_dtype="bf16", tile=tile) if y_bf16 else None
    torch.cuda.synchronize()
    if y_bf16:
        # the bf16 launch rounds exactly the values the fp32 launch writes
        assert np.array_equal(_bf16_bits(yb), _bf16_bits(y_fast.to(torch.bfloat16)))
        ybf = yb.float().cpu().numpy()
    yg, ag = y.cpu().numpy(), acc.cpu().numpy().astype(np.int64)
    yf = y_fast.cpu().numpy()
    xl, xo = acts.t["x_low"].cpu().numpy(), acts.t["x_out"].cpu().numpy()
    sx = acts.t["s_x"].cpu().numpy()
    sxo = acts.t["s_xo"].cpu().numpy() if branch != "bf16" else None
    for e, l in enumerate(lays):
        o_idx, o_mp, _, _ = oracle.select_channels(l.x_cal, l.w, k_out)
        assert np.array_equal(maps_t[e].cpu().numpy(), o_mp)
        o_w = oracle.pack_weights(l.w, o_mp, branch=branch)
        assert np.array_equal(wts.t["w_low"][e].cpu().numpy(), o_w["w_low"])
        assert f32_bits_equal(wts.t["s_w"][e].cpu().numpy(), o_w["s_w"]), f"expert {e} s_w"
        assert np.array_equal(wts.t["w_out"][e].cpu().numpy().view(o_w["w_out"].dtype), o_w["w_out"]), \
            f"expert {e} branch weights"
        if branch != "bf16":
            assert f32_bits_equal(wts.t["s_wo"][e].cpu().numpy(), o_w["s_wo"]), f"expert {e} s_wo"
        if l.m == 0:
            continue
        r0, r1 = off[e], off[e + 1]
        o_a = oracle.quantize_split_act(bits[r0:r1], o_mp, branch=branch, x_fmt="bf16")
        assert np.array_equal(xl[r0:r1], o_a["x_low"])
        assert f32_bits_equal(sx[r0:r1], o_a["s_x"]), f"expert {e} s_x"
        assert np.array_equal(xo[r0:r1].view(o_a["x_out"].dtype), o_a["x_out"])
        if branch != "bf16":
            assert f32_bits_equal(sxo[r0:r1], o_a["s_xo"]), f"expert {e} s_xo"
        rows = None if rows_per_group is None else np.unique(
            np.linspace(0, l.m - 1, min(rows_per_group, l.m)).astype(np.int64))
        o_y, o_acc, _, _ = oracle.dual_gemm(o_a, o_w, rows=rows, debug=True)
        sel = np.arange(l.m) if rows is None else rows
        assert np.array_equal(ag[r0:r1][sel], o_acc), f"expert {e} accumulators"
        assert_rows_close(yg[r0:r1][sel], o_y, f"expert {e}")
        assert_rows_close(yf[r0:r1][sel], o_y, f"expert {e} (no debug outputs)")
        if y_bf16:
            _assert_bf16_close(ybf[r0:r1][sel], o_y, f"expert {e} (bf16 Y)")


def test_hand_case_through_the_abi(sqf, golden):
    """The hand-worked case (K = 4 channels, one outlier) through every entry
    point on the GPU, against the values worked by hand: k = 4 is not a
    multiple of the 8-channel chunk, so the activation kernel takes its
    element-wise load path; the selection runs without a score buffer."""
    g = golden("osc_hand_case.txt")
    f = lambda key: np.array([[float(v) for v in r] for r in g[key]], np.float32)
    x_cal = torch.from_numpy(f("x_cal")).cuda()
    w = torch.from_numpy(f("w")).cuda()
    idx, mp, score, _ = sqf.sqf_select_channels(x_cal, w, int(g["k_out"][0][0]), want_score=False)
    assert score is None
    wts = sqf.sqf_pack_weights(w, mp)
    x = torch.from_numpy(f("x")).cuda()
    acts = sqf.alloc_acts(1, 3, 1)
    sqf.sqf_quantize_split_act(x, mp, acts)
    y, acc = sqf.sqf_dual_gemm(acts, wts, debug=True)[:2]
    torch.cuda.synchronize()
    assert idx.cpu().tolist() == [int(v) for v in g["idx"][0]]
    assert mp.cpu().tolist() == [int(v) for v in g["map"][0]]
    xl = acts.t["x_low"][0].cpu().numpy()
    assert xl[:2].tolist() == [int(v, 16) for v in g["x_low_bytes"][0]] and not xl[2:].any()
    assert acts.t["s_x"][0].item() == float(g["s_x"][0][0])
    assert int(acts.t["x_out"][0, 0].item()) & 0xFFFF == int(g["x_out_bf16"][0][0], 16)
    wl = wts.t["w_low"][0].cpu().numpy()
    assert wl[:, :2].tolist() == [[int(v, 16) for v in r] for r in g["w_low_bytes"]]
    assert wts.t["s_w"][0].cpu().numpy().tolist() == f("s_w")[0].tolist()
    assert acc[0].cpu().tolist() == [int(v) for v in g["acc"][0]]
    assert y[0].cpu().numpy().tolist() == f("y")[0].tolist()


@pytest.mark.parametrize("x_dtype", ["bf16", "f32"])
def test_k_not_a_multiple_of_8(sqf, x_dtype):
    """k = 1003 channels (k_low 940, k_out 63), rows of exactly k elements:
    neither k nor the row stride is a multiple of the 8-channel chunk, so the
    activation kernel reads element by element; every stage against the
    oracle."""
    lay = _ragged(m=37, k=1003, n=200, n_scaled=63, seed=97)
    st, _ = run_layer(sqf, lay, lay.k_out, x_dtype=x_dtype)
    _print("k=1003", x_dtype, st)


def test_selection_without_score_buffer(sqf):
    """score_out == NULL: the library borrows the workspace; idx and map are
    those of the call with a score buffer (and of the oracle)."""
    lay = _ragged(m=16, k=3000, n=300, n_scaled=100, seed=98)
    x_cal = torch.from_numpy(lay.x_cal).cuda()
    w = torch.from_numpy(lay.w).cuda()
    i0, m0, s0, h0 = sqf.sqf_select_channels(x_cal, w, 187)
    i1, m1, s1, h1 = sqf.sqf_select_channels(x_cal, w, 187, want_score=False)
    torch.cuda.synchronize()
    assert s1 is None
    assert torch.equal(i0, i1) and torch.equal(m0, m1) and torch.equal(h0, h1)
    o_idx, o_mp, _, _ = oracle.select_channels(lay.x_cal, lay.w, 187)
    assert np.array_equal(i1.cpu().numpy(), o_idx) and np.array_equal(m1.cpu().numpy(), o_mp)


# ------------------------------------------------------------------ int4 codes on the 6-bit matrix unit
@pytest.mark.parametrize("x_dtype", ["bf16", "f32"])
def test_e2m3_low_path_ragged(sqf, x_dtype):
    """The int4 codes in 6-bit E2M3 fields through the FP6 GEMM: M, N and
    K_low past any tile multiple, K_out not a multiple of the branch stage.
    Bytes, scales and the exact int32 low sums against the oracle; Y within
    tolerance."""
    lay = _ragged(m=300, k=1000, n=520, n_scaled=37, seed=101)
    st, _ = run_layer(sqf, lay, lay.k_out, x_dtype=x_dtype, low="i4e2m3")
    _print("e2m3 ragged", x_dtype, st)


@pytest.mark.parametrize("k_out_kind", ["none", "all", "half"])
def test_e2m3_extreme_fractions(sqf, k_out_kind):
    """No outlier channel (no branch stage), every channel an outlier (no low
    stage: the bf16 branch alone), and half of them (f = 1/2)."""
    lay = _ragged(m=260, k=640, n=300, n_scaled=40, seed=102)
    k_out = {"none": 0, "all": lay.k, "half": lay.k // 2}[k_out_kind]
    st, _ = run_layer(sqf, lay, k_out, low="i4e2m3", check_select=k_out not in (0, lay.k))
    _print("e2m3 k_out", k_out_kind, st)


def test_e2m3_matches_packed_int4_kernel_bit_for_bit(sqf):
    """Same codes, same scales, same bf16 branch order: the FP6 kernel's fp32 Y
    equals the packed-int4 kernel's Y to the bit (the low sums are exact on
    both, and the fused epilogue rounds identically), and its bf16 Y is the
    nearest-even rounding of that Y."""
    lay = _ragged(m=512, k=2048, n=768, n_scaled=128, seed=103)
    x_cal = torch.from_numpy(lay.x_cal).cuda()
    w = torch.from_numpy(lay.w).cuda()
    _, mp, _, _ = sqf.sqf_select_channels(x_cal, w, lay.k_out)
    xt = x_inputs(lay, "bf16")[2]
    w4 = sqf.sqf_pack_weights(w, mp)
    w6 = sqf.sqf_pack_weights(w, mp, low="i4e2m3")
    a4 = sqf.alloc_acts(lay.m, lay.k - lay.k_out, lay.k_out)
    a6 = sqf.alloc_acts(lay.m, lay.k - lay.k_out, lay.k_out, low="i4e2m3")
    sqf.sqf_quantize_split_act(xt, mp, a4)
    sqf.sqf_quantize_split_act(xt, mp, a6)
    y4 = sqf.sqf_dual_gemm(a4, w4, tile="256")
    y6, acc6 = sqf.sqf_dual_gemm(a6, w6, debug=True)[:2]
    y4d, acc4 = sqf.sqf_dual_gemm(a4, w4, debug=True, tile="256")[:2]
    y6b = sqf.sqf_dual_gemm(a6, w6, y_dtype="bf16")
    torch.cuda.synchronize()
    assert torch.equal(acc6, acc4)
    assert torch.equal(y6.view(torch.int32), y4.view(torch.int32))
    assert torch.equal(y6b.view(torch.int16), y6.to(torch.bfloat16).view(torch.int16))
    with pytest.raises(sqf.SqfError) as ei:
        sqf.sqf_dual_gemm(a6, w6, tile="128")
    assert ei.value.status == sqf.SQF_ERR_UNSUPPORTED
    with pytest.raises(sqf.SqfError):
        sqf.sqf_dual_gemm(a6, w4)  # activations and weights in different storage


# ------------------------------------------------------------------ MXFP4 low path
@pytest.mark.parametrize("x_dtype", ["bf16", "f32"])
def test_mxfp4_low_path_ragged(sqf, x_dtype):
    """MXFP4 codes and block scales (K-blocked) from the packer and the
    activation kernel against the oracle bit for bit; Y within tolerance on
    every row.  M, N and K_low past any tile multiple, K_out not a multiple
    of the branch stage."""
    lay = _ragged(m=300, k=1000, n=520, n_scaled=37, seed=111)
    st, _ = run_layer_mx(sqf, lay, lay.k_out, x_dtype=x_dtype)
    _print("mxfp4 ragged", x_dtype, st)


@pytest.mark.parametrize("k_out_kind", ["none", "all", "half"])
def test_mxfp4_extreme_fractions(sqf, k_out_kind):
    lay = _ragged(m=260, k=640, n=300, n_scaled=40, seed=112)
    k_out = {"none": 0, "all": lay.k, "half": lay.k // 2}[k_out_kind]
    st, _ = run_layer_mx(sqf, lay, k_out, check_select=k_out not in (0, lay.k))
    _print("mxfp4 k_out", k_out_kind, st)


def test_mxfp4_block_scales_over_a_wide_range(sqf):
    """Blocks whose magnitudes span 2^-140 .. 2^60 (fp32 subnormals, the
    E8M0 clamp at -127, all-zero blocks, exact ties of the E2M1 grid): every
    code and scale byte bit for bit, Y within tolerance."""
    rng = np.random.default_rng(113)
    lay = _ragged(m=520, k=1536, n=264, n_scaled=24, seed=113)
    x = lay.x.astype(np.float64) * np.exp2(rng.integers(-140, 60, (lay.m, lay.k // 32)).repeat(32, 1))
    x[rng.random(lay.m) < 0.1, :] = 0.0
    x[:, 64:96] = 0.0  # a zero block in every row (before the permutation)
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0]) * 0.5
    x[::7, :8] = ties
    w = lay.w.astype(np.float64) * np.exp2(rng.integers(-30, 30, (lay.k // 32, lay.n)).repeat(32, 0))
    lay2 = synth.Layer(name="wide", m=lay.m, k=lay.k, n=lay.n, k_out=lay.k_out,
                       x=x.astype(np.float32), x_cal=lay.x_cal, w=w.astype(np.float32), scaled=lay.scaled)
    st, _ = run_layer_mx(sqf, lay2, lay2.k_out, x_dtype="f32")
    _print("mxfp4 wide", st)


def test_mxfp4_codes_at_rounding_boundaries(sqf):
    """Every rounding boundary of the E2M1 grid (exact ties go to the even
    code, values one bf16 step either side go to the nearer one), saturation
    at 6, and negative values that round to zero -- whose code must be the
    unsigned zero: codes and scale bytes bit for bit against the oracle.
    Each row repeats a 16-value pattern whose largest magnitude is 7.5, so
    every 32-slot block has the scale exponent of its row's power of two."""
    pattern = np.array([6.0, 0.25, -0.25, 0.75, -0.75, 1.25, -1.75, 2.5, -3.5, 5.0, -0.125,
                        -0.2490234375, 0.2509765625, -6.0, 7.5, -0.0])
    lay = _ragged(m=272, k=1024, n=256, n_scaled=16, seed=211)
    r = np.arange(lay.m)[:, None]
    c = np.arange(lay.k)[None, :]
    x = pattern[(c + r) % 16] * np.exp2((r % 41) - 20.0)
    lay2 = synth.Layer(name="e2m1 boundaries", m=lay.m, k=lay.k, n=lay.n, k_out=lay.k_out,
                       x=x.astype(np.float32), x_cal=lay.x_cal, w=lay.w, scaled=lay.scaled)
    st, _ = run_layer_mx(sqf, lay2, lay2.k_out, x_dtype="f32")
    _print("mxfp4 boundaries", st)


def test_mxfp4_bf16_output_and_errors(sqf):
    """bf16 Y is the nearest-even rounding of the fp32 Y; the MXFP4 path has
    one tile shape and no integer accumulators."""
    lay = _ragged(m=512, k=2048, n=768, n_scaled=128, seed=114)
    x_cal = torch.from_numpy(lay.x_cal).cuda()
    w = torch.from_numpy(lay.w).cuda()
    _, mp, _, _ = sqf.sqf_select_channels(x_cal, w, lay.k_out)
    wm = sqf.sqf_pack_weights(w, mp, low="mxfp4")
    am = sqf.alloc_acts(lay.m, lay.k - lay.k_out, lay.k_out, low="mxfp4")
    sqf.sqf_quantize_split_act(x_inputs(lay, "bf16")[2], mp, am)
    y = sqf.sqf_dual_gemm(am, wm)
    yb = sqf.sqf_dual_gemm(am, wm, y_dtype="bf16")
    y2 = sqf.sqf_dual_gemm(am, wm, tile="256")
    torch.cuda.synchronize()
    assert torch.equal(yb.view(torch.int16), y.to(torch.bfloat16).view(torch.int16))
    assert torch.equal(y2.view(torch.int32), y.view(torch.int32))
    for kw in (dict(tile="128"), dict(debug=True)):
        with pytest.raises(sqf.SqfError) as ei:
            sqf.sqf_dual_gemm(am, wm, **kw)
        assert ei.value.status == sqf.SQF_ERR_UNSUPPORTED


# ------------------------------------------------------------------ banked SQ-format
@pytest.mark.parametrize("bank", [64, 128, 256, 512])
def test_sq_banked(sqf, bank):
    """Banked weight-side format: the same count of marks in every bank of
    `bank` slots; marks, values, scales, the three exact accumulators and Y
    against the oracle (k_low = 1024, 1/8 of the slots marked)."""
    lay = _ragged(m=200, k=1280, n=300, n_scaled=256, seed=121)
    assert lay.k - lay.k_out == 1024
    _sq_check(sqf, lay, 128, f"sq bank {bank}", bank=bank)


@pytest.mark.parametrize("bank,den", [(64, 2), (64, 64), (1024, 8)])
def test_sq_banked_densities(sqf, bank, den):
    """Half of every bank marked, one mark per bank, and a bank equal to the
    whole row (the unbanked choice)."""
    lay = _ragged(m=130, k=1280, n=260, n_scaled=256, seed=122)
    _sq_check(sqf, lay, 1024 // den, f"sq bank {bank} 1/{den}", bank=bank)


def test_sq_banked_key_ties(sqf):
    """Equal keys inside banks (W on a 5-value grid, calibration columns
    repeated in groups of 4): the lower slot wins within each bank."""
    lay = _ragged(m=96, k=1280, n=136, n_scaled=256, seed=123)
    lay.w[:] = np.clip(np.rint(lay.w / 0.01), -2, 2).astype(np.float32) * np.float32(0.01)
    for c in range(0, lay.k - 3, 4):
        lay.x_cal[:, c + 1:c + 4] = lay.x_cal[:, c:c + 1]
    _sq_check(sqf, lay, 256, "sq bank ties", bank=64)


# ------------------------------------------------------------------ floating-point SQ-format
def _sqf_fp_check(sqf, lay, nnz, label, bank=0, x_dtype="bf16", rows=None):
    """E4M3 activations, E2M1 weights with the 0x8 mark, E4M3 sparse values
    and branch: every byte and scale bit for bit, Y within tolerance."""
    k_out = lay.k_out
    k_low = lay.k - k_out
    x_cal = torch.from_numpy(lay.x_cal).cuda()
    w = torch.from_numpy(lay.w).cuda()
    _, mp, _, hdiag = sqf.sqf_select_channels(x_cal, w, k_out)
    wts = sqf.sqf_pack_weights(w, mp, branch="fp8", hdiag=hdiag, sq_nnz=nnz, sq_bank=bank, low="fp4")
    ox, ofmt, xt = x_inputs(lay, x_dtype)
    acts = sqf.alloc_acts(lay.m, k_low, k_out, low="fp8", branch="fp8")
    sqf.sqf_quantize_split_act(xt, mp, acts)
    y = sqf.sqf_dual_gemm(acts, wts)
    torch.cuda.synchronize()
    o_mp = mp.cpu().numpy()
    o_hd = hdiag.cpu().numpy()
    o_w = oracle.pack_weights_sqf(lay.w, o_mp, o_hd, nnz, bank=bank)
    assert np.array_equal(wts.t["w_low"][0].cpu().numpy(), o_w["w_low"]), "E2M1 codes differ"
    assert np.array_equal(wts.t["sq_val"].cpu().numpy().view(np.uint8), o_w["sq_val"]), "E4M3 values differ"
    assert f32_bits_equal(wts.t["s_w"][0].cpu().numpy(), o_w["s_w"])
    assert f32_bits_equal(wts.t["s_w8"].cpu().numpy(), o_w["s_w8"])
    assert np.array_equal(wts.t["w_out"][0].cpu().numpy(), o_w["w_out"])
    assert f32_bits_equal(wts.t["s_wo"][0].cpu().numpy(), o_w["s_wo"])
    o_a = oracle.quantize_split_act(ox, o_mp, low="fp8", branch="fp8", x_fmt=ofmt)
    assert np.array_equal(acts.t["x_low"].cpu().numpy(), o_a["x_low"]), "E4M3 activations differ"
    assert np.array_equal(acts.t["x_out"].cpu().numpy(), o_a["x_out"])
    assert f32_bits_equal(acts.t["s_x"].cpu().numpy(), o_a["s_x"])
    assert f32_bits_equal(acts.t["s_xo"].cpu().numpy(), o_a["s_xo"])
    if rows is None:
        rows = np.arange(lay.m, dtype=np.int64)
    o_y = oracle.dual_gemm_sqf(o_a, o_w, rows=rows)
    st = assert_rows_close(y.cpu().numpy()[rows], o_y, label)
    _sq_ws_same(sqf, acts, wts, y, label)
    return st


@pytest.mark.parametrize("x_dtype", ["bf16", "f32"])
def test_sq_fp_small(sqf, x_dtype):
    lay = _ragged(m=300, k=1280, n=260, n_scaled=64, seed=141)
    _print("sq fp small", x_dtype, _sqf_fp_check(sqf, lay, (lay.k - lay.k_out) // 8, "sq fp", x_dtype=x_dtype))


@pytest.mark.parametrize("m,k,n,den,bank", [
    (257, 1280, 129, 2, 0),     # dense marks: past the value window
    (70, 640, 130, 1, 0),       # every low slot marked
    (200, 1280, 300, 8, 64),    # banks of 64 (k_low = 1024)
    (5, 256, 3, 128, 0),        # a few values in total
])
def test_sq_fp_densities_and_banks(sqf, m, k, n, den, bank):
    n_scaled = 256 if bank else max(1, k // 16)
    lay = _ragged(m=m, k=k, n=n, n_scaled=n_scaled, seed=142 + den)
    nnz = max(1, (lay.k - lay.k_out) // den)
    _print("sq fp", m, k, n, den, bank, _sqf_fp_check(sqf, lay, nnz, f"sq fp 1/{den} bank {bank}", bank=bank))


def test_sq_fp_refuses_debug_and_mismatch(sqf):
    lay = _ragged(m=64, k=512, n=64, n_scaled=32, seed=146)
    x_cal = torch.from_numpy(lay.x_cal).cuda()
    w = torch.from_numpy(lay.w).cuda()
    _, mp, _, hd = sqf.sqf_select_channels(x_cal, w, lay.k_out)
    wts = sqf.sqf_pack_weights(w, mp, branch="fp8", hdiag=hd, sq_nnz=60, low="fp4")
    acts = sqf.alloc_acts(lay.m, lay.k - lay.k_out, lay.k_out, low="fp8", branch="fp8")
    sqf.sqf_quantize_split_act(x_inputs(lay, "bf16")[2], mp, acts)
    with pytest.raises(sqf.SqfError) as ei:
        sqf.sqf_dual_gemm(acts, wts, debug=True)
    assert ei.value.status == sqf.SQF_ERR_UNSUPPORTED
    a8 = sqf.alloc_acts(lay.m, lay.k - lay.k_out, lay.k_out, low="i8", branch="fp8")
    with pytest.raises(sqf.SqfError):
        sqf.sqf_dual_gemm(a8, wts)
