"""Saved affine maps of the linear stages: the .npz written by
save_calibrations reads back bit for bit, and malformed files are refused.
Host-only (no kernel runs)."""

import numpy as np
import pytest
import torch

from linear_hybrid_attention_zebra_amd import stage


def _cal(heads, m, seed):
    g = torch.Generator().manual_seed(seed)
    a = torch.randn(heads, 64, generator=g)
    b = torch.randn(heads, 64, generator=g)
    idx = torch.randperm(10_000, generator=g)[:m].sort().values
    return stage.Calibration(a, b, seed % 3, idx)


def test_round_trip_bitwise(tmp_path):
    cals = {1: _cal(16, 40, 1), 5: _cal(16, 40, 2), 23: _cal(16, 7, 3)}
    path = tmp_path / "affine.npz"
    stage.save_calibrations(path, cals)
    back = stage.load_calibrations(path, "cpu")
    assert sorted(back) == [1, 5, 23]
    for s, c in cals.items():
        r = back[s]
        assert r.aff_scale.dtype == torch.float32 and r.aff_scale.is_contiguous()
        assert torch.equal(r.aff_scale.view(torch.int32), c.aff_scale.view(torch.int32))
        assert torch.equal(r.aff_bias.view(torch.int32), c.aff_bias.view(torch.int32))
        assert torch.equal(r.sample_index, c.sample_index.to(torch.int64))
        assert r.n_degenerate == c.n_degenerate
        assert r.x is None and r.y is None


def test_file_holds_plain_arrays_only(tmp_path):
    path = tmp_path / "affine.npz"
    stage.save_calibrations(path, {2: _cal(4, 5, 9)})
    with np.load(path, allow_pickle=False) as z:
        assert sorted(z.files) == ["s2_aff_bias", "s2_aff_scale", "s2_n_degenerate",
                                   "s2_sample_index"]
        assert all(z[k].dtype != object for k in z.files)


def test_wrong_shape_refused(tmp_path):
    path = tmp_path / "bad.npz"
    np.savez(path, s0_aff_scale=np.zeros((4, 32), np.float32),
             s0_aff_bias=np.zeros((4, 32), np.float32),
             s0_sample_index=np.arange(3), s0_n_degenerate=np.int64(0))
    with pytest.raises(ValueError, match="expected"):
        stage.load_calibrations(path, "cpu")
