"""Checks of the seeded input generators (no attention arithmetic here)."""
import math

import numpy as np
from scipy import integrate

from lsh_attention_amd import inputs as I


def test_bf16_rounding_nearest_even():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -9, 3.0e-39], dtype=np.float32)
    bits = I.bf16_bits_from_f32(vals)
    # 1+2^-8 is halfway between 0x3F80 and 0x3F81 -> even 0x3F80;
    # 1+3*2^-8 is halfway between 0x3F81 and 0x3F82 -> even 0x3F82.
    assert bits.tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x3F80, 0x0021]
    np.testing.assert_array_equal(I.f32_from_bf16_bits(bits)[:4], [1.0, 1.0, 1.0 + 2 ** -6, -2.5])


def test_inputs_are_deterministic_and_bf16_exact():
    a = I.make_inputs("causal_lm_4k", B=1, H=2, L=256)
    b = I.make_inputs("causal_lm_4k", B=1, H=2, L=256)
    assert a.meta == b.meta
    assert a.qk.values.shape == (1, 2, 256, 64) and a.rot.values.shape == (4, 64, 32)
    np.testing.assert_array_equal(I.f32_from_bf16_bits(I.bf16_bits_from_f32(a.qk.values)), a.qk.values)


def test_rotation_rounds_are_shared_between_round_counts():
    two = I.make_inputs("peaked_vmf_16k", n_hashes=2, B=1, H=1, L=128)
    eight = I.make_inputs("peaked_vmf_16k", n_hashes=8, B=1, H=1, L=128)
    np.testing.assert_array_equal(eight.rot.values[:2], two.rot.values)


def test_vmf_mean_cosine_matches_marginal_density():
    """The cosine t = mu.x of a vMF(mu, kappa) draw on S^{d-1} has density
    proportional to exp(kappa t) (1 - t^2)^((d-3)/2); compare the sample mean
    with that integral (about 0.549 at d = 64, kappa = 50)."""
    d, kappa, N = 64, 50.0, 20000
    f = lambda t: math.exp(kappa * (t - 1)) * (1 - t * t) ** ((d - 3) / 2)
    z, _ = integrate.quad(f, -1, 1, points=[0.5], limit=200)
    m, _ = integrate.quad(lambda t: t * f(t), -1, 1, points=[0.5], limit=200)
    m2, _ = integrate.quad(lambda t: t * t * f(t), -1, 1, points=[0.5], limit=200)
    mean, sd = m / z, math.sqrt(m2 / z - (m / z) ** 2)
    rng = np.random.Generator(np.random.PCG64(1))
    mu = rng.standard_normal((N, d))
    mu /= np.linalg.norm(mu, axis=1, keepdims=True)
    x = I.vmf_wood(rng, mu, kappa)
    np.testing.assert_allclose(np.linalg.norm(x, axis=1), 1.0, atol=1e-12)
    t = np.sum(x * mu, axis=1)
    assert abs(mean - 0.549) < 0.002
    assert abs(t.mean() - mean) < 5 * sd / math.sqrt(N)
    assert abs(t.std() - sd) < 0.05 * sd
