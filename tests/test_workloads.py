"""Seeded generator: determinism (same seeds, same bytes) and the recipes' shapes."""
import numpy as np
import pytest

import workloads as W


@pytest.mark.parametrize("name", ["tiny", "bert_attn"])
def test_same_seed_same_bytes(name):
    wl = W.get_workload(name)
    a = W.make_layer_batch(wl, 0, 3, with_w=True)
    b = W.make_layer_batch(wl, 0, 3, with_w=True)
    assert W.sha256_of(a["x"], a["gy"], a["w"]) == W.sha256_of(b["x"], b["gy"], b["w"])
    c = W.make_layer_batch(wl, 0, 4)
    assert W.sha256_of(a["x"]) != W.sha256_of(c["x"])
    assert W.sha256_of(a["x"]) != W.sha256_of(a["gy"])


def test_shapes_and_dtypes():
    for wl in W.WORKLOADS.values():
        if wl.name == "llm_mlp":
            continue
        ly = wl.layers[-1]
        d = W.make_layer_batch(wl, ly.name, 0, with_w=True)
        assert d["x"].shape == (wl.B, wl.L, ly.Cx)
        assert d["gy"].shape == (wl.B, wl.L, ly.Cy)
        assert d["w"].shape == (ly.Cy, ly.Cx)
        assert d["x"].dtype == (np.float32 if wl.dtype == "fp32" else np.uint16)


def test_bf16_rounding_is_rne():
    v = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -16, -0.0, np.inf, np.nan])
    bits = W.bf16_bits_from_f64(v)
    assert list(bits[:5]) == [0x3F80, 0x3F82, 0x3F81, 0x8000, 0x7F80]
    assert np.isnan(W.bf16_bits_to_f64(bits[5:]))[0]
    # round trip of representable values is exact
    r = np.random.default_rng(0).standard_normal(1000)
    b1 = W.bf16_bits_from_f64(r)
    assert np.array_equal(W.bf16_bits_from_f64(W.bf16_bits_to_f64(b1)), b1)
    assert np.abs(W.bf16_bits_to_f64(b1) - r).max() <= np.abs(r).max() * 2.0 ** -8
