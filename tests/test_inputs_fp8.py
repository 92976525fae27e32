"""The e4m3 encoder and decoder that prepare fp8 inputs, pinned against the
format's definition (OCP 8-bit floating point, e4m3 "fn" variant) and against
PyTorch's own float8_e4m3fn conversion."""

import numpy as np
import pytest
import torch

from exact_attention_80_amd import inputs

ALL_CODES = np.arange(256, dtype=np.uint8)


def torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()


def torch_encode(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def test_decode_matches_torch_on_every_code():
    mine, ref = inputs.e4m3_decode(ALL_CODES), torch_decode(ALL_CODES)
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    assert np.sum(np.isnan(mine)) == 2            # 0x7f and 0xff only
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])


@pytest.mark.parametrize("value,code", [
    (0.0, 0x00), (-0.0, 0x80), (1.0, 0x38), (-1.0, 0xB8), (448.0, 0x7E), (-448.0, 0xFE),
    (2.0 ** -6, 0x08), (2.0 ** -9, 0x01), (7 * 2.0 ** -9, 0x07), (1.125, 0x39), (240.0, 0x77),
    # ties go to the even code
    (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02), (1.0625, 0x38), (1.1875, 0x3A), (464.0, 0x7E),
])
def test_encode_fixed_points(value, code):
    assert int(inputs.e4m3_encode([value])[0]) == code


def test_encode_matches_torch_on_random_values_and_midpoints():
    g = np.random.default_rng(5)
    fin = np.sort(np.unique(inputs.e4m3_decode(ALL_CODES)[~np.isnan(inputs.e4m3_decode(ALL_CODES))]))
    x = np.concatenate([g.standard_normal(50000) * 30, g.standard_normal(5000) * 1e-3,
                        (fin[:-1] + fin[1:]) / 2, fin])
    x = x[np.abs(x) <= 448].astype(np.float32).astype(np.float64)
    assert np.array_equal(inputs.e4m3_encode(x), torch_encode(x))


def test_encode_decode_round_trip_and_error_bound():
    codes = ALL_CODES[(ALL_CODES & 0x7F) != 0x7F]
    assert np.array_equal(inputs.e4m3_encode(inputs.e4m3_decode(codes)), codes)
    g = np.random.default_rng(6)
    x = g.uniform(2.0 ** -6, 448, 20000) * np.where(g.random(20000) < 0.5, -1, 1)
    r = inputs.e4m3_decode(inputs.e4m3_encode(x))
    assert np.all(np.abs(r - x) <= np.abs(x) * 2.0 ** -4)   # half a step of 3 mantissa bits


@pytest.mark.parametrize("bad", [464.5, 500.0, -1e6, float("inf"), float("nan")])
def test_encode_rejects_out_of_range(bad):
    with pytest.raises(ValueError):
        inputs.e4m3_encode([bad])


def test_fp8_inputs_recipe():
    x = inputs.fp8_dense_inputs(1, 64, 2, 1, 64, seed=3)
    raw = inputs.dense_inputs(1, 64, 2, 1, 64, seed=3, round_bf16=False)
    assert x["q8"].dtype == np.uint8 and x["q8"].shape == (1, 64, 2, 64)
    assert x["k8"].shape == (1, 64, 1, 64)
    assert x["q_descale"] == np.float32(np.abs(raw["q"]).max() / 448)
    # the largest magnitude maps to the top code and dequantises within rounding
    assert np.max(x["q8"] & 0x7F) == 0x7E
    assert np.allclose(x["q"], raw["q"], rtol=2.0 ** -4, atol=x["q_descale"] * 2.0 ** -9)
    assert np.array_equal(x["v"], inputs.bf16_round(raw["v"]))


def test_fp8_packed_inputs_recipe():
    lq, lk = [1, 5, 0], [40, 5, 9]
    x = inputs.fp8_varlen_qk_inputs(lq, lk, 4, 2, 64, seed=8)
    raw = inputs.varlen_qk_inputs(lq, lk, 4, 2, 64, seed=8, round_bf16=False)
    assert x["q8"].shape == (6, 4, 64) and x["k8"].shape == (54, 2, 64)
    assert np.array_equal(x["cu_seqlens_q"], [0, 1, 6, 6])
    assert np.array_equal(x["cu_seqlens_k"], [0, 40, 45, 54])
    assert x["k_descale"] == np.float32(np.abs(raw["k"]).max() / 448)
    assert np.array_equal(x["q"], x["q_descale"] * inputs.e4m3_decode(x["q8"]))
    assert np.array_equal(x["v"], inputs.bf16_round(raw["v"]))
    # the bf16-rounded draws are the same numbers rounded
    assert np.array_equal(inputs.varlen_qk_inputs(lq, lk, 4, 2, 64, seed=8)["k"],
                          inputs.bf16_round(raw["k"]))
