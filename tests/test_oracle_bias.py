"""Pins for the oracle's load-balance bias update."""
import numpy as np

from oracle import esg_oracle as O


def test_fixed_point_when_balanced():
    G = 8
    tgt = 0.25
    bias = np.linspace(-0.3, 0.3, G)
    ema = np.full(G, tgt)
    nb, ne = O.update_load_balance_bias(bias, ema, np.full(G, tgt), tgt, 1e-3, 0.5, 0.99)
    assert np.array_equal(ne, ema) and np.array_equal(nb, bias)   # sign(0) = 0
    nb32, ne32 = O.update_load_balance_bias(bias, ema, np.full(G, tgt), tgt, 1e-3, 0.5, 0.99, np.float32)
    assert np.array_equal(ne32, ema.astype(np.float32)) and np.array_equal(nb32, bias.astype(np.float32))


def test_direction_and_step():
    """Over-used groups lose gamma, under-used gain gamma."""
    bias = np.zeros(4)
    ema = np.full(4, 0.5)
    cur = np.array([0.9, 0.1, 0.5, 0.5])
    nb, ne = O.update_load_balance_bias(bias, ema, cur, 0.5, 1e-3, 0.5, 0.9)
    np.testing.assert_allclose(ne, [0.54, 0.46, 0.5, 0.5], rtol=1e-15)
    assert nb.tolist() == [-1e-3, 1e-3, 0.0, 0.0]


def test_saturation():
    bias = np.array([0.4995, -0.4995, 0.5, -0.5])
    ema = np.array([0.0, 1.0, 0.0, 1.0])
    nb, _ = O.update_load_balance_bias(bias, ema, ema, 0.5, 1e-3, 0.5, 0.99)
    assert nb.tolist() == [0.5, -0.5, 0.5, -0.5]


def test_ema_converges_to_constant_frequency():
    """Repeated updates with a constant frequency: ema -> cur geometrically,
    ema_n - cur = momentum^n (ema_0 - cur)."""
    ema = np.array([0.0, 1.0])
    cur = np.array([0.3, 0.3])
    e = ema.copy()
    for _ in range(50):
        _, e = O.update_load_balance_bias(np.zeros(2), e, cur, 0.3, 1e-3, 0.5, 0.9)
    np.testing.assert_allclose(e, cur + 0.9 ** 50 * (ema - cur), rtol=1e-12)


def test_bias_walk_counts_steps():
    """With ema held below target the bias rises by exactly gamma per call
    until it saturates at bias_max (500 calls of 1e-3 reach 0.5)."""
    b = np.zeros(1)
    for _ in range(600):
        b, _ = O.update_load_balance_bias(b, np.zeros(1), np.zeros(1), 0.25, 1e-3, 0.5, 0.99)
    assert b[0] == 0.5


def test_frequency_from_counts_sums_to_k():
    counts = np.array([3, 1, 0, 4])          # 4 tokens, k = 2
    f = O.frequency_from_counts(counts, 4)
    assert f.tolist() == [0.75, 0.25, 0.0, 1.0] and f.sum() == 2.0
