"""Pins of oracle/rope.py. The pages name pre-RoPE key quantization without
defining the embedding, so these pin the textbook definition by properties
that a plausible mistake (a swapped sign, the wrong pairing, frequencies off
by a factor or an index) breaks: identity at position 0, a hand-computed
rotation, a rotation (norm kept) of each pair, q.k depending only on the
position difference, composition and inverse, the complex multiplication
form, and the frequency formula's end points."""
import numpy as np
import pytest

from oracle import rope as R
from oracle.cache import Config, RefCache


def _x(n=5, d=128, seed=0):
    return np.random.default_rng(seed).standard_normal((n, d))


def test_frequencies():
    f = R.frequencies(128, 10000.0)
    assert f.shape == (64,) and f[0] == 1.0
    assert np.isclose(f[32], 10000.0 ** -0.5, rtol=1e-15)
    assert np.isclose(f[63], 10000.0 ** (-126 / 128), rtol=1e-15)
    assert np.all(np.diff(f) < 0)


def test_position_zero_is_identity():
    x = _x()
    assert np.array_equal(R.rope(x, np.zeros(5)), x)


def test_hand_case():
    # channel 0 and its partner 64 at position 1 rotate by theta_0 = 1 rad;
    # channel 1 / 65 by theta_1 = 10000^(-1/64)
    x = np.zeros((1, 128))
    x[0, 0], x[0, 64] = 2.0, 3.0
    x[0, 1] = 1.0
    y = R.rope(x, [1])[0]
    assert np.isclose(y[0], 2 * np.cos(1) - 3 * np.sin(1), rtol=1e-15)
    assert np.isclose(y[64], 3 * np.cos(1) + 2 * np.sin(1), rtol=1e-15)
    t1 = 10000.0 ** (-1 / 64)
    assert np.isclose(y[1], np.cos(t1), rtol=1e-15) and np.isclose(y[65], np.sin(t1), rtol=1e-15)
    others = np.delete(y, [0, 1, 64, 65])
    assert np.all(others == 0)


def test_each_pair_is_rotated():
    x = _x(7)
    y = R.rope(x, np.arange(7) * 1000 + 3)
    n_in = x[:, :64] ** 2 + x[:, 64:] ** 2
    n_out = y[:, :64] ** 2 + y[:, 64:] ** 2
    assert np.allclose(n_in, n_out, rtol=1e-12)


def test_scores_depend_on_position_difference_only():
    rng = np.random.default_rng(1)
    q, k = rng.standard_normal((1, 128)), rng.standard_normal((1, 128))
    base = float((R.rope(q, [10]) @ R.rope(k, [3]).T)[0, 0])
    for shift in (1, 77, 5000, 30000):
        s = float((R.rope(q, [10 + shift]) @ R.rope(k, [3 + shift]).T)[0, 0])
        assert np.isclose(s, base, rtol=1e-9, atol=1e-9), shift
    # and does depend on it
    assert not np.isclose(float((R.rope(q, [11]) @ R.rope(k, [3]).T)[0, 0]), base)


def test_composition_and_inverse():
    x = _x(3)
    a, b = np.array([5, 900, 31000]), np.array([12, 7, 1])
    assert np.allclose(R.rope(R.rope(x, a), b), R.rope(x, a + b), atol=1e-10)
    assert np.allclose(R.rope(R.rope(x, a), -a), x, atol=1e-10)


def test_complex_multiplication_form():
    # pair (i, i + 64) as the complex number x_i + j x_{i+64}, times e^{j t theta_i}
    x = _x(4)
    t = np.array([0, 1, 4095, 32767])
    z = x[:, :64] + 1j * x[:, 64:]
    w = z * np.exp(1j * t[:, None] * R.frequencies(128, 10000.0)[None, :])
    y = R.rope(x, t)
    assert np.allclose(y[:, :64], w.real, atol=1e-10) and np.allclose(y[:, 64:], w.imag, atol=1e-10)


@pytest.mark.parametrize("base", [10000.0, 500000.0])
def test_cache_attention_with_rope_is_rotated_keys(base):
    """RefCache with k_rope attends with its dequantized keys rotated by
    position; the same cache without rotation differs."""
    cfg = Config(128, 1, 2, 4, 4, "channel", 32, 32, k_rope=1, rope_theta=base)
    c = RefCache(cfg, 1, 128)
    rng = np.random.default_rng(2)
    k = rng.standard_normal((70, 1, 128)).astype(np.float16)
    v = rng.standard_normal((70, 1, 128)).astype(np.float16)
    c.append(k, v, [70])
    q = rng.standard_normal((1, 2, 128)).astype(np.float16)
    out = c.attention(q, 0.1)
    K = R.rope(c.k_hat(0, 0), np.arange(70), base)
    V = c.v_hat(0, 0)
    for h in range(2):
        sc = 0.1 * (K @ q[0, h].astype(np.float64))
        p = np.exp(sc - sc.max())
        assert np.allclose(out[0, h], p @ V / p.sum(), atol=1e-12)
    cfg.k_rope = 0
    assert not np.allclose(c.attention(q, 0.1), out, atol=1e-3)
