"""Host checks of the seeded workload generator and the parity metric."""
import numpy as np

from ssm_workloads import (RTOL, WATCH, WORKLOADS, bf16_bits_to_f32, f32_to_bf16_bits, make_inputs,
                           parity)


def test_bf16_round_nearest_even():
    bits = np.array([0x3F808000, 0x3F818000, 0x3F808001, 0x3F80FFFF, 0x7F7FFFFF,
                     0xFF800000, 0x7FC00001, 0x00000001], dtype=np.uint32)
    got = f32_to_bf16_bits(bits.view(np.float32))
    # ties go to even, above-half rounds up, overflow rounds to inf, NaN stays NaN
    assert got.tolist() == [0x3F80, 0x3F82, 0x3F81, 0x3F81, 0x7F80, 0xFF80, 0x7FC0, 0x0000]
    x = np.random.default_rng(0).standard_normal(1000).astype(np.float32)
    w = bf16_bits_to_f32(f32_to_bf16_bits(x))
    assert np.all(np.abs(w - x) <= np.abs(x) * 2.0 ** -8)
    assert np.array_equal(f32_to_bf16_bits(w), f32_to_bf16_bits(x))


def test_generator_is_deterministic_and_shaped():
    w = WORKLOADS["tiny"]
    a, b = make_inputs(w), make_inputs(w)
    for k in ("u", "delta", "A", "B", "C", "D", "delta_bias"):
        assert np.array_equal(a[k], b[k])
    assert a["u"].shape == (1, 64, 256) and a["B"].shape == (1, 16, 256)
    assert a["A"].shape == (64, 16) and np.all(a["A"][:, 3] == -4.0)
    dt = np.log1p(np.exp(a["delta_bias"].astype(np.float64)))
    assert np.all((dt > 0.99e-3) & (dt < 0.101))
    small = WORKLOADS["widestate"].with_(batch=1, dim=8, seqlen=16)
    s = make_inputs(small)
    assert s["u"].dtype == np.uint16 and s["z"].shape == (1, 8, 16)
    ratio = -s["A"] / np.arange(1, 65)[None, :]
    assert np.all((ratio >= 0.5) & (ratio <= 1.5))


def test_algorithmic_bytes_headline():
    # 4*2048*2048*(u, delta, z, out in bf16) + B, C + A, D, bias + final state
    assert WORKLOADS["layer"].algorithmic_bytes() == 135_413_760


def test_parity_metric():
    r = np.array([1.0, -2.0, 0.0, 3.0])
    assert parity(r, r, 1e-4).ok
    rep = parity(r + np.array([0, 0, 1e-3, 0]), r, 1e-4)
    assert not rep.ok and rep.worst_index == (2,)
    assert not parity(np.array([np.nan, 1.0]), np.array([0.0, 1.0]), 1.0).ok


def test_bf16_watch_is_the_rounding_bound():
    """The bf16 regression watch against what rounding alone does.

    An exact result rounded to nearest-even bf16, and the same with a float32-sized error
    added before rounding, stay within the watch; a result whose rounding error is doubled
    (one more unit in the last place where the rounding went one way) does not, though it
    stays within the 2e-2 bar.
    """
    rng = np.random.default_rng(77)
    r = rng.standard_normal(200_000) * np.exp(rng.uniform(-6, 6, 200_000))
    rounded = bf16_bits_to_f32(f32_to_bf16_bits(r.astype(np.float32)))
    assert parity(rounded, r, RTOL["bf16"], WATCH["bf16"]).ok
    noisy = r * (1 + rng.uniform(-5e-5, 5e-5, r.size))
    rn = bf16_bits_to_f32(f32_to_bf16_bits(noisy.astype(np.float32)))
    assert parity(rn, r, RTOL["bf16"], WATCH["bf16"]).ok
    doubled = r + 2.0 * (rounded - r)
    rep = parity(doubled, r, RTOL["bf16"], WATCH["bf16"])
    assert rep.err <= RTOL["bf16"] and not rep.ok
    assert parity(doubled, r, RTOL["bf16"]).ok  # without the watch it would pass
    assert WATCH["f32"] == RTOL["f32"]
