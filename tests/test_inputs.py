import numpy as np

from exact_attention_80_amd import inputs


def test_bf16_round_ties_to_even_and_exact_values():
    # 1 + 2^-8 is halfway between bf16 neighbours 1 and 1 + 2^-7: ties to even -> 1
    x = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -2.5, 0.0, 3.0e38], dtype=np.float32)
    r = inputs.bf16_round(x)
    assert r[0] == 1.0
    assert r[1] == 1.0
    assert r[2] == 1 + 2 ** -6
    assert r[3] == -2.5
    assert r[4] == 0.0
    assert np.all(inputs.bf16_bits(r[:5]) == np.array([0x3F80, 0x3F80, 0x3F82, 0xC020, 0], np.uint16))
    assert np.array_equal(inputs.bits_to_f32(inputs.bf16_bits(r)), r)


def test_bf16_round_is_nearest():
    x = np.random.Generator(np.random.PCG64(0)).standard_normal(10000).astype(np.float32)
    r = inputs.bf16_round(x)
    assert np.all(np.abs(r - x) <= np.abs(x) * 2.0 ** -8 * 1.0000001)
    assert np.all(inputs.bf16_bits(r) == inputs.bf16_bits(inputs.bf16_round(r)))


def test_dense_inputs_are_seeded_and_shaped():
    a = inputs.dense_inputs(1, 16, 4, 2, 8, seed=0)
    b = inputs.dense_inputs(1, 16, 4, 2, 8, seed=0)
    c = inputs.dense_inputs(1, 16, 4, 2, 8, seed=1)
    for n in ("q", "k", "v", "do"):
        assert np.array_equal(a[n], b[n])
        assert not np.array_equal(a[n], c[n])
    assert a["q"].shape == (1, 16, 4, 8) and a["k"].shape == (1, 16, 2, 8)
    assert a["do"].shape == (1, 16, 4, 8) and a["v"].shape == (1, 16, 2, 8)


def test_varlen_lengths_procedure():
    ls = inputs.varlen_lengths(65536, 128, 16384, seed=1)
    assert sum(ls) == 65536
    assert all(128 <= l <= 16384 for l in ls)
    assert ls == inputs.varlen_lengths(65536, 128, 16384, seed=1)
    for seed in range(20):
        ls = inputs.varlen_lengths(65536, 128, 16384, seed=seed)
        assert sum(ls) == 65536 and min(ls) >= 128 and max(ls) <= 16384
    cu = inputs.cu_seqlens(ls)
    assert cu[0] == 0 and cu[-1] == 65536 and np.all(np.diff(cu) > 0)
    assert cu.dtype == np.int32
