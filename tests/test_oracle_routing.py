"""Pins for the sigmoid top-k routing oracle (CPU only)."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import routing_oracle as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _hand_cases():
    with open(os.path.join(GOLDEN, "sigmoid_topk_hand.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _hand_cases(), ids=lambda c: c["name"])
def test_hand_cases(case):
    probs, idx = R.sigmoid_topk_routing(np.array(case["logits"], dtype=np.float32),
                                        np.array(case["bias"], dtype=np.float32), case["k"], case["scaling"])
    assert idx.dtype == np.int64 and probs.dtype == np.float32
    assert idx.tolist() == case["indices"]
    if "probs" in case:
        assert probs.tolist() == case["probs"]
    if "probs_approx" in case:
        np.testing.assert_allclose(probs, np.array(case["probs_approx"]), rtol=0, atol=case["tol"])
    if "probs_first" in case:
        s = R.sigmoid_fp32(np.array(case["logits"], dtype=np.float32))[0]
        assert probs[0, 0] == np.float32(case["probs_first"])
        for j in range(1, case["k"]):
            assert probs[0, j] == np.float32(2.0) * s[idx[0, j]]


def test_total_order_key_orders_like_float_values():
    vals = np.array([0.0, -0.0, 1.0, -1.0, 1e-45, -1e-45, 3.4e38, -3.4e38, 0.5, -0.5, 2.0, 1e-38, -1e-38],
                    dtype=np.float32)
    rng = np.random.default_rng(0)
    vals = np.concatenate([vals, rng.standard_normal(200).astype(np.float32) * 10])
    u = R.total_order_key(vals).astype(np.int64)
    a, b = vals[:, None].astype(np.float64), vals[None, :].astype(np.float64)
    neg0 = np.signbit(vals) & (vals == 0)
    less = (a < b) | ((a == b) & neg0[:, None] & ~neg0[None, :])     # -0.0 just below +0.0
    assert np.array_equal(u[:, None] < u[None, :], less)


def _random_case(T, E, seed):
    g = torch.Generator().manual_seed(seed)
    logits = torch.randn(T, E, generator=g) * 2
    bias = (torch.rand(E, generator=g) - 0.5) * 0.2
    return logits.numpy(), bias.numpy()


@pytest.mark.parametrize("E,k", [(8, 2), (64, 6), (256, 8), (43, 11), (300, 32)])
def test_selection_set_matches_torch_topk(E, k):
    logits, bias = _random_case(50, E, E + k)
    probs, idx = R.sigmoid_topk_routing(logits, bias, k)
    keys = torch.sigmoid(torch.as_tensor(logits, dtype=torch.float64)).float() + torch.as_tensor(bias)
    ref = torch.topk(keys, k, dim=1).indices.numpy()
    for t in range(50):
        assert set(idx[t].tolist()) == set(ref[t].tolist())
        # distinct keys: the k-1 larger experts in ascending order, then the k-th largest
        assert list(idx[t, :-1]) == sorted(idx[t, :-1].tolist())
        assert idx[t, -1] == ref[t, -1]


@pytest.mark.parametrize("levels,k", [(2, 3), (3, 5), (5, 8)])
def test_ties_against_brute_force_order_statistic(levels, k):
    """Quantised logits tie often: the selected set is the first k experts of
    the list sorted by (key descending, expert ascending); above-threshold
    experts precede tied ones, each part ascending."""
    rng = np.random.default_rng(levels * 7 + k)
    E = 24
    logits = rng.integers(0, levels, size=(40, E)).astype(np.float32)
    bias = np.zeros(E, dtype=np.float32)
    probs, idx = R.sigmoid_topk_routing(logits, bias, k)
    s = R.sigmoid_fp32(logits)
    for t in range(40):
        order = sorted(range(E), key=lambda e: (-float(s[t, e]), e))
        assert set(idx[t].tolist()) == set(order[:k])
        tau = s[t, order[k - 1]]
        above = [e for e in idx[t] if s[t, e] > tau]
        tied = [e for e in idx[t] if s[t, e] == tau]
        assert list(idx[t]) == above + tied
        assert above == sorted(above) and tied == sorted(tied)


def test_sigmoid_fp32_against_torch_float32():
    z = np.concatenate([np.linspace(-30, 30, 20001), [0.0, 17.0, -17.0, 88.0, -88.0, -104.0, -200.0]]).astype(np.float32)
    ours = R.sigmoid_fp32(z)
    ref = torch.sigmoid(torch.as_tensor(z)).numpy()
    assert ours[np.where(z == 0)[0][0]] == np.float32(0.5)
    assert (ours >= 0).all() and (ours <= 1).all()
    # torch's fp32 sigmoid is within 2 ulp of the true value; ours is the correctly rounded one
    ulp = np.spacing(np.abs(ref)).astype(np.float64)
    assert (np.abs(ours.astype(np.float64) - ref.astype(np.float64)) <= 2 * ulp).all()
    # torch's fp64 sigmoid rounded once agrees exactly away from fp32 rounding midpoints
    ref64 = torch.sigmoid(torch.as_tensor(z, dtype=torch.float64)).float().numpy()
    keep = ~R.near_rounding_boundary(z)
    assert keep.mean() > 0.999 and np.array_equal(ours[keep], ref64[keep])
    # sigmoid(z) + sigmoid(-z) = 1 up to one rounding of each
    sym = ours.astype(np.float64) + R.sigmoid_fp32(-z).astype(np.float64)
    assert np.abs(sym - 1.0).max() <= 2 ** -24 * 2


def test_probabilities_sum_to_scaling_and_batch_invariance():
    logits, bias = _random_case(64, 96, 5)
    probs, idx = R.sigmoid_topk_routing(logits, bias, 7, scaling=2.5)
    np.testing.assert_allclose(probs.astype(np.float64).sum(1), 2.5, rtol=1e-6)
    p1, i1 = R.sigmoid_topk_routing(logits[13:14], bias, 7, scaling=2.5)
    assert np.array_equal(i1[0], idx[13]) and np.array_equal(p1[0], probs[13])


def test_near_rounding_boundary_is_rare_and_sound():
    z = np.random.default_rng(3).standard_normal(200000).astype(np.float32) * 4
    m = R.near_rounding_boundary(z)
    assert m.mean() < 1e-4
    v = 1.0 / (1.0 + np.exp(-z.astype(np.float64)))
    ok = ~m
    for f in (1 - 2.0 ** -50, 1 + 2.0 ** -50):       # perturbed fp64 values round alike
        assert np.array_equal((v[ok] * f).astype(np.float32), v[ok].astype(np.float32))


def test_rejects_bad_arguments():
    with pytest.raises(ValueError):
        R.sigmoid_topk_routing(np.zeros((2, 4), np.float32), np.zeros(3, np.float32), 2)
    with pytest.raises(ValueError):
        R.sigmoid_topk_routing(np.zeros((2, 4), np.float32), np.zeros(4, np.float32), 5)
    with pytest.raises(ValueError):
        R.sigmoid_topk_routing(np.full((2, 4), np.nan, np.float32), np.zeros(4, np.float32), 2)
