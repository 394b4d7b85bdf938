"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times.  Every stage before the GEMM is compared in full (bit-exact);
the GEMM's int32 accumulators and fp32 outputs are compared on a sample of
token rows (first, last and random rows, all output channels), which the
oracle computes one by one.

Workloads (seeded, synthetic):
* tiny: M=64, K=N=256, fp32 input, 16 outliers.
* Llama-3-8B-shaped prefill linears: M=2048; 4096->4096, 4096->14336, 14336->4096.
* Llama-3-70B-shaped prefill linears: M=4096; 8192->8192, 8192->28672,
  28672->8192 at outlier fraction 1/16; fractions 1/2, 1/4, 1/8 as well on
  the 8192->8192 shape.
* Qwen3-30B-A3B-shaped expert GEMMs: 128 experts, 8192 tokens routed top-8,
  2048->768 (up) and 768->2048 (down); bf16 branch, E4M3 branch on the down
  projection at 1/16 and with every channel in the branch.
* Weight-side SQ-format on 4096->14336, M=2048.
"""
import numpy as np
import pytest
import torch

import oracle
from outlier_split_mixed_amd import synth

from harness import (assert_rows_close, f32_bits_equal, run_layer, run_layer_mx, sample_rows,
                     tile_band_rows, x_inputs)
from test_gpu_parity import _grouped_check, _poisoned_workspace, _sq_ws_same, _sqf_fp_check

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sqf():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from outlier_split_mixed_amd import sqf as mod

    return mod


def _log(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("low", ["i4", "i4e2m3"])
@pytest.mark.parametrize("layer", [0, 1, 2])
def test_llama3_8b_layers(sqf, layer, low):
    """Sampled rows against the oracle, plus every row of a whole tile band
    and of the last tile (exact sums, Y in tolerance)."""
    lay = synth.llama3_8b(layer)
    st, _ = run_layer(sqf, lay, lay.k_out, rows=sample_rows(lay.m, 12, seed=layer), low=low,
                      band=tile_band_rows(lay.m))
    _log(lay.name, low, st)


@pytest.mark.parametrize("low", ["i4", "i4e2m3"])
@pytest.mark.parametrize("layer", [0, 1, 2])
def test_llama3_70b_layers_f16(sqf, layer, low):
    lay = synth.llama3_70b(layer, 16)
    st, _ = run_layer(sqf, lay, lay.k_out, rows=sample_rows(lay.m, 8, seed=10 + layer), low=low,
                      band=tile_band_rows(lay.m))
    _log(lay.name, "1/16", low, st)


@pytest.mark.parametrize("low", ["i4", "i4e2m3"])
@pytest.mark.parametrize("frac", [2, 4, 8])
def test_llama3_70b_fraction_sweep(sqf, frac, low):
    lay = synth.llama3_70b(0, frac)
    st, _ = run_layer(sqf, lay, lay.k_out, rows=sample_rows(lay.m, 8, seed=20 + frac), low=low)
    _log(lay.name, f"1/{frac}", low, st)


@pytest.mark.parametrize("layer", [0, 1, 2])
def test_llama3_70b_layers_mxfp4(sqf, layer):
    """The MXFP4 low path at full size: every code and block scale, sampled
    rows against the oracle, a whole tile band plus the last tile against the
    product of the dequantised operands."""
    lay = synth.llama3_70b(layer, 16)
    st, _ = run_layer_mx(sqf, lay, lay.k_out, rows=sample_rows(lay.m, 4, seed=30 + layer),
                         band=tile_band_rows(lay.m))
    _log(lay.name, "mxfp4", st)


@pytest.mark.parametrize("layer", [0, 1, 2])
def test_llama3_8b_layers_mxfp4(sqf, layer):
    lay = synth.llama3_8b(layer)
    st, _ = run_layer_mx(sqf, lay, lay.k_out, rows=sample_rows(lay.m, 6, seed=40 + layer),
                         band=tile_band_rows(lay.m))
    _log(lay.name, "mxfp4", st)


@pytest.fixture(scope="module")
def moe():
    return synth.qwen3_moe()


def test_moe_up_bf16(sqf, moe):
    _grouped_check(sqf, moe.up, "bf16", rows_per_group=3)
    _log("moe up bf16 ok")


def test_moe_down_bf16(sqf, moe):
    _grouped_check(sqf, moe.down, "bf16", rows_per_group=3)
    _log("moe down bf16 ok")


def test_moe_down_fp8(sqf, moe):
    _grouped_check(sqf, moe.down, "fp8", rows_per_group=3)
    _log("moe down fp8 ok")


def test_moe_down_fp8_every_channel(sqf, moe):
    """The literal whole-input FP8 fallback: every channel in the E4M3 branch."""
    lays = []
    for l in moe.down[:16]:
        l2 = synth.Layer(name=l.name, m=l.m, k=l.k, n=l.n, k_out=l.k, x=l.x, x_cal=l.x_cal,
                         w=l.w, scaled=l.scaled)
        lays.append(l2)
    _grouped_check(sqf, lays, "fp8", rows_per_group=3)
    _log("moe down fp8 f=1 ok")


@pytest.mark.parametrize("bank", [0, 64, 256])
def test_sq_weight_side_full(sqf, bank):
    lay = synth.sq_weight()
    k_out = lay.k_out
    k_low = lay.k - k_out
    nnz = k_low // 8
    x_cal = torch.from_numpy(lay.x_cal).cuda()
    w = torch.from_numpy(lay.w).cuda()
    idx, mp, score, hdiag = sqf.sqf_select_channels(x_cal, w, k_out)
    wts = sqf.sqf_pack_weights(w, mp, branch="i8", hdiag=hdiag, sq_nnz=nnz, sq_bank=bank)
    ox, ofmt, xt = x_inputs(lay, "bf16")
    acts = sqf.alloc_acts(lay.m, k_low, k_out, low="i8", branch="i8")
    sqf.sqf_quantize_split_act(xt, mp, acts)
    y, al, asp, ao = sqf.sqf_dual_gemm(acts, wts, debug=True)
    y_fast = sqf.sqf_dual_gemm(acts, wts)
    torch.cuda.synchronize()
    o_idx, o_mp, _, o_hd = oracle.select_channels(lay.x_cal, lay.w, k_out)
    assert np.array_equal(mp.cpu().numpy(), o_mp)
    assert f32_bits_equal(hdiag.cpu().numpy(), o_hd)
    o_w = oracle.pack_weights_sq(lay.w, o_mp, o_hd, nnz, bank=bank)
    assert np.array_equal(wts.t["w_low"][0].cpu().numpy(), o_w["w_low"])
    assert np.array_equal(wts.t["sq_val"].cpu().numpy(), o_w["sq_val"])
    assert f32_bits_equal(wts.t["s_w8"].cpu().numpy(), o_w["s_w8"])
    assert f32_bits_equal(wts.t["s_w"][0].cpu().numpy(), o_w["s_w"])
    assert np.array_equal(wts.t["w_out"][0].cpu().numpy().view(np.int8), o_w["w_out"])
    assert f32_bits_equal(wts.t["s_wo"][0].cpu().numpy(), o_w["s_wo"])
    o_a = oracle.quantize_split_act(ox, o_mp, low="i8", branch="i8", x_fmt=ofmt)
    assert np.array_equal(acts.t["x_low"].cpu().numpy(), o_a["x_low"])
    assert np.array_equal(acts.t["x_out"].cpu().numpy(), o_a["x_out"])
    assert f32_bits_equal(acts.t["s_x"].cpu().numpy(), o_a["s_x"])
    assert f32_bits_equal(acts.t["s_xo"].cpu().numpy(), o_a["s_xo"])
    rows = sample_rows(lay.m, 8, seed=40)
    o_y, o_al, o_asp, o_ao = oracle.dual_gemm(o_a, o_w, rows=rows, debug=True)
    assert np.array_equal(al.cpu().numpy()[rows].astype(np.int64), o_al)
    assert np.array_equal(asp.cpu().numpy()[rows].astype(np.int64), o_asp)
    assert np.array_equal(ao.cpu().numpy()[rows].astype(np.int64), o_ao)
    assert_rows_close(y.cpu().numpy()[rows], o_y, "sq full")
    assert_rows_close(y_fast.cpu().numpy()[rows], o_y, "sq full (no debug outputs)")
    # the gather once per call into a workspace: the sampled rows' accumulators
    # against the oracle, and the whole Y bit for bit against the fused call
    ws = _poisoned_workspace(sqf, wts)
    y_ws, al_w, asp_w, ao_w = sqf.sqf_dual_gemm_sq_ws(acts, wts, workspace=ws, debug=True)
    torch.cuda.synchronize()
    assert np.array_equal(al_w.cpu().numpy()[rows].astype(np.int64), o_al)
    assert np.array_equal(asp_w.cpu().numpy()[rows].astype(np.int64), o_asp)
    assert np.array_equal(ao_w.cpu().numpy()[rows].astype(np.int64), o_ao)
    assert torch.equal(al_w, al) and torch.equal(asp_w, asp) and torch.equal(ao_w, ao)
    _sq_ws_same(sqf, acts, wts, y_fast, "sq full", ws=ws)
    _log("sq full ok, bank", bank)


@pytest.mark.parametrize("bank", [0, 64])
def test_sq_fp_weight_side_full(sqf, bank):
    """The floating-point weight-side format (E2M1 low, E4M3 sparse values,
    E4M3 activations and branch) at full size, 1/8 of the slots kept."""
    lay = synth.sq_weight()
    st = _sqf_fp_check(sqf, lay, (lay.k - lay.k_out) // 8, f"sq fp full bank {bank}", bank=bank,
                       rows=sample_rows(lay.m, 8, seed=50 + bank))
    _log("sq fp full", bank, st)
