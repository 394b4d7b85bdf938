"""The allocation-free entry point (sqf_select_channels_noalloc) against the
allocating one (sqf_select_channels with a caller score buffer): two calls in
a row on one GPU, the second smaller, so the second reuses the static score
array the first one filled.  Channel set, map and hdiag must match bit for
bit (index and integer results; hdiag is the same fp64 sum rounded once)."""
import numpy as np
import pytest
import torch

from outlier_split_mixed_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sqf():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from outlier_split_mixed_amd import sqf as mod

    return mod


def _pair(sqf, lay, k_out):
    x_cal = torch.from_numpy(lay.x_cal).cuda()
    w = torch.from_numpy(lay.w).cuda()
    i0, m0, s0, h0 = sqf.sqf_select_channels(x_cal, w, k_out, want_score=True)
    idx = torch.full((max(k_out, 1),), -7, dtype=torch.int32, device="cuda")
    mp = torch.full((lay.k,), -7, dtype=torch.int32, device="cuda")
    hd = torch.full((lay.k,), -7.0, dtype=torch.float32, device="cuda")
    i1, m1, h1 = sqf.sqf_select_channels_noalloc(x_cal, w, k_out, idx=idx, mp=mp, hdiag=hd)
    torch.cuda.synchronize()
    assert s0 is not None
    assert torch.equal(i0, i1), "outlier channel set differs"
    assert torch.equal(m0, m1), "channel map differs"
    assert torch.equal(h0.view(torch.int32), h1.view(torch.int32)), "hdiag differs"
    assert i1.data_ptr() == idx.data_ptr() and m1.data_ptr() == mp.data_ptr()


def test_noalloc_select_matches_the_allocating_call_twice(sqf):
    big = synth.draw_layer("noalloc_big", 401, 0, 8, 12000, 3000, 96, 700)
    small = synth.draw_layer("noalloc_small", 402, 0, 8, 3000, 700, 64, 190)
    _pair(sqf, big, big.k_out)
    print("noalloc select: k=12000 ok", flush=True)
    _pair(sqf, small, small.k_out)
    print("noalloc select: k=3000 after k=12000 ok", flush=True)


def test_noalloc_select_rejects_k_beyond_its_array(sqf):
    x_cal = torch.zeros((2, 65537), dtype=torch.float32, device="cuda")
    w = torch.zeros((65537, 1), dtype=torch.float32, device="cuda")
    with pytest.raises(sqf.SqfError) as ei:
        sqf.sqf_select_channels_noalloc(x_cal, w, 4)
    assert ei.value.status == sqf.SQF_ERR_SHAPE
