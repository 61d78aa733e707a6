"""Seeded input generators: deterministic, right shapes and distributions."""
import numpy as np
import torch

from transformer_row_normalization_amd import inputs


def test_seeded_and_deterministic():
    a = inputs.layer_f32_1024x768()
    b = inputs.layer_f32_1024x768()
    for k in ("x", "w", "b"):
        assert torch.equal(a.tensors[k], b.tensors[k])
    assert a.tensors["x"].shape == (1, 1024, 768)
    assert float(a.tensors["x"].min()) >= -1.0 and float(a.tensors["x"].max()) < 1.0
    assert float(a.tensors["w"].min()) >= 0.5 and float(a.tensors["w"].max()) < 1.5


def test_iota_variant_is_exact():
    wl = inputs.rms_f32_512x1024("iota")
    x = wl.tensors["x"].reshape(-1)
    assert x.shape[0] == 524288
    # fl32(fl32(i) / 100): compare a few against numpy's float32 division
    idx = np.array([0, 1, 7, 1000, 524287])
    ref = (idx.astype(np.float32) / np.float32(100.0)).astype(np.float32)
    assert np.array_equal(x[idx].numpy(), ref)
    assert wl.rows == 512 and wl.width == 1024


def test_dual_shapes():
    wl = inputs.dual_bf16_4096tok(tokens=16)
    assert wl.tensors["q"].shape == (16, 32, 128) and wl.tensors["k"].shape == (16, 8, 128)
    assert wl.tensors["q"].dtype == torch.bfloat16
    assert wl.rows == 16 * 40 and wl.width == 128


def test_outlier_mask_rate():
    wl = inputs.layer_bf16_65536x4096(rows=512, width=4096)
    x = wl.tensors["x"].float()
    n = x.numel()
    hits = wl.tensors["outliers"]
    assert abs(hits - 0.001 * n) < 5 * np.sqrt(0.001 * n)
    assert abs(float(x[x.abs() < 50].mean()) - 3.0) < 0.05


def test_swiglu_workload_shapes():
    wl = inputs.rms_swiglu_bf16_4096tok(tokens=8)
    assert wl.tensors["x"].shape == (8, 32, 128) == wl.tensors["g"].shape
    assert wl.tensors["w"].shape == (128,) and wl.rows == 256 and wl.width == 128
    again = inputs.rms_swiglu_bf16_4096tok(tokens=8)
    assert torch.equal(wl.tensors["g"], again.tensors["g"])
