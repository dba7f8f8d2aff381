"""The seeded input generator: determinism, distribution and encodings."""
import numpy as np

import inputs
from inputs.configs import WORKLOADS, make_inputs


def test_splitmix64_reference_value():
    # first output of SplitMix64 seeded with 1234567 (published test vector)
    assert inputs.splitmix64(1234567) == 6457827717110365317


def test_deterministic_and_stream_separated():
    a = inputs.normal(99, 0, (1000,), "f32")
    b = inputs.normal(99, 0, (1000,), "f32")
    c = inputs.normal(99, 1, (1000,), "f32")
    assert np.array_equal(a, b)
    assert not np.array_equal(a, c)
    # element i depends only on i: a prefix of a longer draw is the shorter draw
    assert np.array_equal(inputs.normal(99, 0, (10_000,), "f32")[:1000], a)


def test_normal_moments():
    x = inputs.normal(3, 0, (1 << 20,), "f32").astype(np.float64)
    assert abs(x.mean()) < 5e-3
    assert abs(x.std() - 1.0) < 5e-3
    assert abs((x ** 4).mean() - 3.0) < 0.05


def test_bf16_is_round_to_nearest_even_of_f32():
    f = inputs.normal(4, 2, (4096,), "f32", 0.5)
    bits = inputs.normal(4, 2, (4096,), "bf16", 0.5)
    assert np.array_equal(bits, inputs.f32_to_bf16_bits(f))
    # ties go to even, others to nearest
    ties = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -(1.0 + 2 ** -8)],
                    dtype=np.float32)
    assert list(inputs.f32_to_bf16_bits(ties)) == [0x3F80, 0x3F82, 0x3F81, 0xBF80]
    back = inputs.bf16_bits_to_f32(bits)
    assert np.all(np.abs(back - f) <= np.abs(f) * 2 ** -8 + 1e-30)


def test_select_positions_distinct_sorted_in_range():
    pos = inputs.select_positions(7, 3, 200_000, 2000)
    assert pos.size == 2000
    assert np.all(np.diff(pos) > 0)
    assert pos[0] >= 0 and pos[-1] < 200_000
    # spread over the whole range, not bunched at the start
    assert pos[-1] > 150_000 and pos[0] < 50_000


def test_peaked_rows_scaled_exactly_by_8():
    w = WORKLOADS["ragged_s200k"]
    q, k, v, peaked = make_inputs(w, "sqa", S=3000)
    assert peaked.size == 30
    seed = w.seed("sqa")
    plain = inputs.normal(seed, 1, k.shape, "bf16", 0.5)
    kf, pf = inputs.bf16_bits_to_f32(k), inputs.bf16_bits_to_f32(plain)
    assert np.array_equal(kf[:, peaked], 8.0 * pf[:, peaked])
    mask = np.ones(3000, dtype=bool)
    mask[peaked] = False
    assert np.array_equal(k[:, mask], plain[:, mask])


def test_workload_shapes():
    w = WORKLOADS["sweep_s4096"]
    assert [(v.H_q, v.H_kv) for v in w.variants] == [(16, 16), (16, 4), (8, 4), (4, 4)]
    q, k, v, _ = make_inputs(w, "sqa", S=64)
    assert q.shape == (2, 64, 8, 64) and k.shape == (2, 64, 4, 64) and q.dtype == np.uint16


def test_decode_lengths_recipe():
    from inputs.configs import DECODE_WORKLOADS, decode_lengths, make_decode_inputs
    w = DECODE_WORKLOADS["decode_s128k"]
    lens = decode_lengths(w.seed(w.variants[0].name), w.B, w.S_max, w.min_len_frac)
    assert lens[0] == w.S_max
    assert (lens >= w.S_max // 4).all() and (lens <= w.S_max).all()
    # same lengths for every variant of the workload, deterministic
    for v in w.variants:
        q, k, vv, l2 = make_decode_inputs(w, v.name, S_max=256)
        assert q.shape == (w.B, v.H_q, w.d) and k.shape == (w.B, 256, v.H_kv, w.d) == vv.shape
        np.testing.assert_array_equal(l2, decode_lengths(w.seed(w.variants[0].name), w.B, 256, w.min_len_frac))
    # a long uniform sample spans the range
    many = decode_lengths(123, 2000, 1000, 0.25)
    assert many.min() <= 260 and many[1:].max() >= 990 and many[1:].min() >= 250
