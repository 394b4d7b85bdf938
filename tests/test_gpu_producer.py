"""GPU parity of the producer-side steps: the RMS norm fused into the split,
and the slot order folded into the neighbouring layers (the split becomes a
slice).  Codes, scales and branch values bit for bit against the oracle; Y
within tolerance, or -- for the reordering, which changes no product --
bit for bit against the unreordered path."""
import numpy as np
import pytest
import torch

import oracle
from outlier_split_mixed_amd import synth

from harness import assert_rows_close, e2m3_rows_equal, f32_bits_equal, x_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sqf():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from outlier_split_mixed_amd import sqf as mod

    return mod


def _print(*a):
    print(*a, flush=True)


def _gamma(k, seed):
    return np.random.default_rng(seed).uniform(0.3, 2.5, k).astype(np.float32)


def _norm_case(sqf, lay, low, x_dtype, eps=1e-5, seed=0, rows=None):
    g = _gamma(lay.k, seed)
    x_cal = torch.from_numpy(lay.x_cal).cuda()
    w = torch.from_numpy(lay.w).cuda()
    _, mp, _, _ = sqf.sqf_select_channels(x_cal, w, lay.k_out)
    ox, ofmt, xt = x_inputs(lay, x_dtype)
    acts = sqf.alloc_acts(lay.m, lay.k - lay.k_out, lay.k_out, low=low)
    gt = torch.from_numpy(g).cuda()
    sqf.sqf_rmsnorm_quantize_split_act(xt, gt, eps, mp, acts)
    wts = sqf.sqf_pack_weights(w, mp, low=low)
    y = sqf.sqf_dual_gemm(acts, wts)
    torch.cuda.synchronize()
    o_mp = mp.cpu().numpy()
    o_a = oracle.rmsnorm_quantize_split_act(ox, g, eps, o_mp, x_fmt=ofmt)
    if low == "i4e2m3":
        want = oracle.i4x2_to_e2m3(o_a["x_low"], oracle.pad_rows(lay.m))
        got = acts.t["x_low"].cpu().numpy()
        assert e2m3_rows_equal(got, want, lay.m), "x_low differs"
    else:
        assert np.array_equal(acts.t["x_low"].cpu().numpy(), o_a["x_low"]), "x_low differs"
    assert f32_bits_equal(acts.t["s_x"].cpu().numpy(), o_a["s_x"]), "s_x differs"
    if lay.k_out:
        assert np.array_equal(acts.t["x_out"].cpu().numpy().view(np.uint16), o_a["x_out"]), \
            "branch differs"
    o_w = oracle.pack_weights(lay.w, o_mp)
    if rows is None:
        rows = np.arange(lay.m, dtype=np.int64)
    o_y = oracle.dual_gemm(o_a, o_w, rows=rows)
    return assert_rows_close(y.cpu().numpy()[rows], o_y, lay.name + " (norm)")


@pytest.mark.parametrize("low", ["i4", "i4e2m3"])
@pytest.mark.parametrize("x_dtype", ["bf16", "f32"])
def test_rmsnorm_split_small(sqf, low, x_dtype):
    lay = synth.draw_layer("norm_small", 131, 0, 300, 2048, 520, 128, 96)
    _print("norm small", low, x_dtype, _norm_case(sqf, lay, low, x_dtype, seed=1))


def test_rmsnorm_split_ragged_rows(sqf):
    """k not a multiple of 8 (the element-wise load path) and eps = 0."""
    lay = synth.draw_layer("norm_ragged", 132, 0, 77, 1001, 130, 64, 33)
    _print("norm ragged", _norm_case(sqf, lay, "i4", "f32", eps=0.0, seed=2))


@pytest.mark.parametrize("layer", [0, 2])
def test_rmsnorm_split_llama3_70b(sqf, layer):
    """Full width (8192 and 28672 channels: gamma takes most of the LDS at
    28672); every row's codes and scales, sampled rows of Y."""
    lay = synth.llama3_70b(layer, 16)
    from harness import sample_rows
    _print("norm 70b", layer, _norm_case(sqf, lay, "i4e2m3", "bf16", seed=3 + layer,
                                          rows=sample_rows(lay.m, 4, seed=layer)))


def test_slot_order_makes_the_split_a_slice(sqf):
    """perm / slice map against the oracle; x and W reordered on the GPU by
    perm give the same packed weights, activations and Y bit for bit (also
    with the fused norm, gamma reordered alike)."""
    lay = synth.draw_layer("slice", 133, 0, 260, 1536, 384, 128, 96)
    x_cal = torch.from_numpy(lay.x_cal).cuda()
    w = torch.from_numpy(lay.w).cuda()
    _, mp, _, _ = sqf.sqf_select_channels(x_cal, w, lay.k_out)
    perm, sm = sqf.sqf_slot_order(mp)
    o_perm, o_sm = oracle.slot_order(mp.cpu().numpy())
    torch.cuda.synchronize()
    assert np.array_equal(perm.cpu().numpy(), o_perm) and np.array_equal(sm.cpu().numpy(), o_sm)
    x = torch.from_numpy(lay.x).cuda()
    xp = sqf.sqf_permute_channels(x, perm, axis=1)
    wp = sqf.sqf_permute_channels(w, perm, axis=0)
    torch.cuda.synchronize()
    assert torch.equal(xp, x[:, perm.long()]) and torch.equal(wp, w[perm.long(), :])
    k_low = lay.k - lay.k_out
    for low in ("i4", "i4e2m3"):
        w0 = sqf.sqf_pack_weights(w, mp, low=low)
        w1 = sqf.sqf_pack_weights(wp, sm, low=low)
        a0 = sqf.alloc_acts(lay.m, k_low, lay.k_out, low=low)
        a1 = sqf.alloc_acts(lay.m, k_low, lay.k_out, low=low)
        sqf.sqf_quantize_split_act(x, mp, a0)
        sqf.sqf_quantize_split_act(xp, sm, a1)
        y0 = sqf.sqf_dual_gemm(a0, w0)
        y1 = sqf.sqf_dual_gemm(a1, w1)
        torch.cuda.synchronize()
        assert torch.equal(w0.t["w_low"], w1.t["w_low"]) and torch.equal(w0.t["w_out"], w1.t["w_out"])
        assert torch.equal(y0.view(torch.int32), y1.view(torch.int32)), low
        g = torch.from_numpy(_gamma(lay.k, 7)).cuda()
        gp = sqf.sqf_permute_channels(g.view(1, -1), perm, axis=1).view(-1)
        sqf.sqf_rmsnorm_quantize_split_act(x, g, 1e-5, mp, a0)
        sqf.sqf_rmsnorm_quantize_split_act(xp, gp, 1e-5, sm, a1)
        torch.cuda.synchronize()
        assert torch.equal(a0.t["s_x"].view(torch.int32), a1.t["s_x"].view(torch.int32))
        assert torch.equal(a0.t["x_out"], a1.t["x_out"])
        if low == "i4":
            assert torch.equal(a0.t["x_low"], a1.t["x_low"])
    _print("slot order ok")
