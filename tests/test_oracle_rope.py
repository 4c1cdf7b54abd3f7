"""Pins of the YaRN rotary-embedding oracle (CPU): the textbook 2-D rotation, the
half-split pairing on a hand example, norm preservation, the relative-position property
of rotary embeddings, the standard-RoPE limit of YaRN (factor 1) and its two
interpolation limits (frequency kept / divided by the factor)."""
import math

import numpy as np

import torch

from oracle import apply_rope, bf16_round, yarn_inv_freq, yarn_mscale


def test_two_dim_rotation_is_textbook():
    # D = 2: one pair, frequency theta**0 = 1, so position p rotates by p radians
    x = np.array([[3.0, -2.0]])
    for p in (0, 1, 5, 1000):
        got = apply_rope(x, [p], theta=10000.0)
        c, s = math.cos(p), math.sin(p)
        assert np.allclose(got, [[3 * c + 2 * s, 3 * s - 2 * c]], rtol=0, atol=1e-12)


def test_half_split_pairing_hand_example():
    # D = 4, theta = 100: frequencies 1 and 0.1; dims (0, 2) and (1, 3) rotate together
    x = np.array([[1.0, 2.0, 3.0, 4.0]])
    p = 2
    got = apply_rope(x, [p], theta=100.0)[0]
    a0, a1 = 2.0, 0.2                      # p * f_i
    want = [1 * math.cos(a0) - 3 * math.sin(a0), 2 * math.cos(a1) - 4 * math.sin(a1),
            3 * math.cos(a0) + 1 * math.sin(a0), 4 * math.cos(a1) + 2 * math.sin(a1)]
    assert np.allclose(got, want, rtol=0, atol=1e-12)


def test_norm_and_relative_position():
    rng = np.random.default_rng(0)
    d = 64
    q = rng.standard_normal((5, d))
    k = rng.standard_normal((5, d))
    for factor in (1.0, 32.0):
        m = yarn_mscale(factor)
        rq = apply_rope(q, [7] * 5, theta=150000.0, factor=factor)
        assert np.allclose(np.linalg.norm(rq, axis=-1), m * np.linalg.norm(q, axis=-1))
        # q(p) . k(p') depends on p - p' only
        for p, pp, delta in ((10, 3, 100), (0, 4000, 12345)):
            d1 = np.sum(apply_rope(q, [p] * 5, 150000.0, factor) *
                        apply_rope(k, [pp] * 5, 150000.0, factor), axis=-1)
            d2 = np.sum(apply_rope(q, [p + delta] * 5, 150000.0, factor) *
                        apply_rope(k, [pp + delta] * 5, 150000.0, factor), axis=-1)
            assert np.allclose(d1, d2, rtol=1e-9, atol=1e-9)


def test_factor_one_is_standard_rope():
    f = yarn_inv_freq(128, 10000.0, 1.0, 4096, 32.0, 1.0)
    assert np.array_equal(f, 10000.0 ** (-np.arange(64) / 64.0))
    assert yarn_mscale(1.0) == 1.0 and abs(yarn_mscale(math.e ** 10) - 2.0) < 1e-15


def test_interpolation_limits():
    d, theta, s, L = 64, 150000.0, 32.0, 4096
    base = theta ** (-2.0 * np.arange(d // 2) / d)
    f = yarn_inv_freq(d, theta, s, L, 32.0, 1.0)
    turns = L * base / (2 * math.pi)
    fast, slow = turns >= 32.0, turns <= 1.0
    assert fast.any() and slow.any() and (~fast & ~slow).any()
    assert np.array_equal(f[fast], base[fast])            # high frequencies kept
    assert np.allclose(f[slow], base[slow] / s, rtol=1e-15)  # low frequencies interpolated
    mid = ~fast & ~slow
    assert np.all((f[mid] > base[mid] / s) & (f[mid] < base[mid]))
    assert np.all(np.diff(f) < 0)                          # still strictly decreasing


def test_bf16_round_is_round_to_nearest_even():
    # representable values are fixed points; halfway cases go to the even neighbour
    assert bf16_round(1.0) == 1.0 and bf16_round(-3.0) == -3.0
    ulp = 2.0 ** -7                          # spacing of bf16 in [1, 2)
    assert bf16_round(1.0 + ulp / 2) == 1.0              # tie -> even (1.0)
    assert bf16_round(1.0 + 1.5 * ulp) == 1.0 + 2 * ulp  # tie -> even (1 + 2 ulp)
    assert bf16_round(1.0 + 0.51 * ulp) == 1.0 + ulp
    # agrees with torch's float32 -> bfloat16 conversion (RNE) on float32 inputs
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(100000) * 10.0 ** rng.integers(-3, 4, 100000)).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    assert np.array_equal(bf16_round(x.astype(np.float64)), want)


def test_interpolation_band_golden():
    """Hand-derived frequencies inside the YaRN band (tests/golden/yarn_midband.json):
    the linear mix of f_i / s and f_i in the continuous turn count.  The fixture also
    records what a wavelength blend and a ramp over rounded dimension indices give, and
    those must be far from the expected values (so either misreading would fail)."""
    import json
    import os
    data = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "yarn_midband.json")))
    p = data["params"]
    f = yarn_inv_freq(p["head_dim"], p["theta"], p["factor"], p["original_max_pos"],
                      p["beta_fast"], p["beta_slow"])
    for case in data["cases"]:
        want = float(case["expected"])
        got = f[case["pair"]]
        assert abs(got - want) <= 1e-13 * want, (case["pair"], got, want)
        for name, alt in case["not_this"].items():
            assert abs(float(alt) - want) > 0.1 * want, name
