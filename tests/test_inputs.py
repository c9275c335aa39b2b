"""Checks of the seeded input generator against its published definitions."""
import numpy as np

import synth_inputs as si


def test_splitmix64_reference_vector():
    # First outputs of the sequential splitmix64 (Vigna's splitmix64.c) for seed 1234567.
    got = si.splitmix64(1234567, np.arange(5, dtype=np.uint64))
    exp = [6457827717110365317, 3203168211198807973, 9817491932198370423,
           4593380528125082431, 16408922859458223821]
    assert [int(x) for x in got] == exp


def test_normals_moments_and_determinism():
    x = si.normal_f64(99, 1 << 20)
    assert abs(x.mean()) < 5e-3
    assert abs(x.var() - 1.0) < 5e-3
    y = si.normal_f64(99, 1 << 20)
    np.testing.assert_array_equal(x, y)
    # chunked (threaded) generation equals one-shot generation
    big = si.normal_f64(5, (1 << 21) + 37)
    np.testing.assert_array_equal(big[:1000], si.normal_f64(5, 1000))
    np.testing.assert_array_equal(big[-37:], si._normals_chunk(5, 1 << 21, 37))


def test_bf16_round_to_nearest_even():
    one = np.float32(1.0)
    eps = np.float32(2.0 ** -8)  # half an ulp of bf16 at 1.0
    xs = np.array([one, one + eps, one + 3 * eps, one + eps + np.float32(2 ** -20), -2.5,
                   np.finfo(np.float32).max, np.inf, -np.inf], dtype=np.float32)
    r = si.round_to_bf16(xs)
    assert r[0] == 1.0
    assert r[1] == 1.0                      # tie -> even
    assert r[2] == 1.0 + 4 * 2.0 ** -8      # tie -> even (upwards)
    assert r[3] == 1.0 + 2 * 2.0 ** -8      # above the tie -> up
    assert r[4] == -2.5
    assert np.isinf(r[5])                   # FLT_MAX rounds past the largest bf16
    assert r[6] == np.inf and r[7] == -np.inf
    assert np.isnan(si.round_to_bf16(np.array([np.nan], dtype=np.float32))[0])


def test_power_of_two_variants_are_exact_scalings():
    a = si.normal_tensor(3, (4, 64), 1.0, "bf16")
    b = si.normal_tensor(3, (4, 64), 0.5, "bf16")
    c = si.normal_tensor(3, (4, 64), 2.0, "bf16")
    np.testing.assert_array_equal(b, a * 0.5)
    np.testing.assert_array_equal(c, a * 2.0)


def test_attention_inputs_distinct_tensors():
    d = si.attention_inputs(1, 2, 8, 4, "f32", seed=1, workload="w", layer=0)
    assert set(d) == {"q", "k", "v", "do"}
    assert not np.array_equal(d["q"], d["k"])
    e = si.attention_inputs(1, 2, 8, 4, "f32", seed=1, workload="w", layer=1)
    assert not np.array_equal(d["q"], e["q"])


def test_f16_rounding_is_ieee_nearest_even():
    """The fp16 inputs are IEEE binary16 round-to-nearest-even: ties go to the
    even mantissa, the largest finite value is 65504, and values from 65520 on
    round to inf."""
    u = 2.0 ** -10  # spacing of binary16 in [1, 2)
    x = np.array([1 + u / 2, 1 + 3 * u / 2, 1 + u / 2 + 2.0 ** -20, -(1 + u / 2), 65504.0,
                  65519.0, 65520.0, 2.0 ** -24, 2.0 ** -26], dtype=np.float32)
    want = np.array([1.0, 1 + 2 * u, 1 + u, -1.0, 65504.0, 65504.0, np.inf, 2.0 ** -24, 0.0],
                    dtype=np.float32)
    got = si.round_to_f16(x)
    assert np.array_equal(got, want), (got, want)


def test_f16_inputs_are_representable_and_scaled():
    a = si.attention_inputs(1, 2, 33, 16, "f16", seed=9, workload="pin")
    b = si.attention_inputs(1, 2, 33, 16, "f32", seed=9, workload="pin")
    for n in a:
        assert np.array_equal(a[n], a[n].astype(np.float16).astype(np.float32))
        # the same draw, rounded: within half an fp16 ulp of the float32 value
        assert np.all(np.abs(a[n] - b[n]) <= np.abs(b[n]) * 2.0 ** -11 + 2.0 ** -25)
