"""Seeded input generators: determinism, value sets, and the storage sizes the
pages print for an 8192 x 8192 matrix in each format (CPU only)."""
import json
import os

import numpy as np
import torch

from tensor_core_matrix_amd import inputs as inp

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")


def test_storage_bytes_match_page_table():
    fig = json.load(open(GOLDEN))["matrix_bytes_8192"]
    w = inp.WORKLOADS["bf16_8192"]
    assert round(w.M * w.K * 2 / 1e6) == fig["bf16_MB"]
    mx = inp.WORKLOADS["mxfp8_8192"]
    elems = mx.M * mx.K
    scales = mx.M * (mx.K // fig["elements_per_scale_mx"])
    assert round(elems / 1e6, 1) == fig["fp8_e4m3_per_tensor_MB"]
    assert round((elems + scales) / 1e6, 1) == fig["mxfp8_MB"]
    assert (elems + scales) * 8 / elems == fig["bits_per_value_mxfp8"]


def test_small_workloads_are_deterministic_and_in_range():
    for name in ("tile_f16", "batched"):
        x, y = inp.make(name), inp.make(name)
        assert all(torch.equal(x[k], y[k]) for k in x)
        assert float(x["A"].float().abs().max()) <= 1.0
    t = inp.make("tile_f16")
    assert t["A"].shape == (128, 64) and t["B"].shape == (64, 64) and t["A"].dtype == torch.float16
    b = inp.make("batched")
    assert b["A"].shape == (1024, 128, 64) and b["B"].shape == (1024, 256, 64)


def test_mx_generators():
    g = inp.generator(4)
    a = inp.e4m3_normal((256, 64), g)
    assert a.dtype == torch.uint8
    vals = a.view(torch.float8_e4m3fn).float()
    assert torch.isfinite(vals).all()
    s = inp.e8m0_scales((256, 2), g)
    e = s.numpy().astype(int) - 127
    assert e.min() == -4 and e.max() == 4 and set(np.unique(e)) == set(range(-4, 5))


def test_quarter_integers_value_set():
    q = inp.quarter_integers((64, 64), inp.generator(1), torch.bfloat16).float() * 4
    assert set(torch.unique(q).tolist()) <= set(range(-4, 5))
