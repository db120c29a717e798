"""Pins for the oracle's grouped top-k selection (CPU only)."""
import itertools
import json
import os

import numpy as np
import pytest
import torch

from oracle import esg_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _hand_cases():
    with open(os.path.join(GOLDEN, "select_hand.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _hand_cases(), ids=lambda c: c["name"])
def test_hand_cases(case):
    idx, _ = O.grouped_topk_select(np.array(case["x"]), np.array(case["w_gate"]), case["group_size"],
                                   case["k"], case["sub"], case["spg"], case["bias"])
    assert idx.tolist() == case["expected"]


def test_energy_matches_torch_silu():
    """E computed with torch's own SiLU and a gather of the sampled rows."""
    g = torch.Generator().manual_seed(1)
    x = torch.randn(37, 24, generator=g, dtype=torch.float64)
    w = torch.randn(96, 24, generator=g, dtype=torch.float64)
    sub = O.make_subsample_index(96, 16, 5, 2)
    e = O.group_energy(x.numpy(), w.numpy(), 16, sub, 5)
    h = x @ w[torch.as_tensor(sub, dtype=torch.long)].T
    ref = torch.nn.functional.silu(h).abs().reshape(37, 6, 5).sum(-1)
    np.testing.assert_allclose(e, ref.numpy(), rtol=1e-13, atol=1e-14)


def _brute_force_topk(scores, k):
    """Exhaustive: the k-subset with the largest total score; among equal
    totals the lexicographically smallest id set."""
    T, G = scores.shape
    out = []
    for t in range(T):
        best, best_set = None, None
        for comb in itertools.combinations(range(G), k):
            tot = sum(scores[t, c] for c in comb)
            if best is None or tot > best + 1e-12:
                best, best_set = tot, comb
        out.append(list(best_set))
    return np.array(out)


@pytest.mark.parametrize("G,k", [(6, 1), (6, 3), (8, 4), (16, 4), (7, 6)])
def test_topk_brute_force(G, k):
    rng = np.random.default_rng(G * 10 + k)
    scores = rng.standard_normal((20, G))
    if G >= 8:   # C(16,4)=1820 subsets: keep the token count small
        scores = scores[:6]
    assert np.array_equal(O.topk_from_scores(scores, k), _brute_force_topk(scores, k))


def test_topk_ties_prefer_lower_ids():
    scores = np.array([[1.0, 2.0, 2.0, 2.0, 0.0], [3.0, 3.0, 3.0, 3.0, 3.0]])
    assert O.topk_from_scores(scores, 2).tolist() == [[1, 2], [0, 1]]
    assert O.topk_from_scores(scores, 4).tolist() == [[0, 1, 2, 3], [0, 1, 2, 3]]


def test_topk_matches_torch_topk_order_on_distinct_scores():
    rng = np.random.default_rng(5)
    s = rng.standard_normal((300, 43))
    ref = torch.sort(torch.topk(torch.as_tensor(s), 11, dim=1).indices, dim=1).values.numpy()
    assert np.array_equal(O.topk_from_scores(s, 11), ref)


def test_full_gate_equals_identity_subsample():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((50, 32))
    w = rng.standard_normal((128, 32)) / np.sqrt(32)
    a, sa = O.grouped_topk_select(x, w, 32, 2)
    sub = O.make_subsample_index(128, 32, 32, 9)   # spg = gs: all rows
    b, sb = O.grouped_topk_select(x, w, 32, 2, sub, 32)
    assert np.array_equal(a, b) and np.array_equal(sa, sb)


def test_batch_invariance():
    """A token's routing does not depend on the other tokens in the batch."""
    rng = np.random.default_rng(4)
    x = rng.standard_normal((64, 40))
    w = rng.standard_normal((320, 40)) / np.sqrt(40)
    bias = rng.uniform(-0.1, 0.1, 10)
    sub = O.make_subsample_index(320, 32, 8, 1)
    full, _ = O.grouped_topk_select(x, w, 32, 3, sub, 8, bias)
    part, _ = O.grouped_topk_select(x[17:29], w, 32, 3, sub, 8, bias)
    assert np.array_equal(full[17:29], part)


def test_group_permutation_equivariance():
    """Relabelling groups (rows of W_gate, bias and subsample) relabels the
    selection."""
    rng = np.random.default_rng(6)
    gs, G, spg = 16, 12, 4
    x = rng.standard_normal((40, 24))
    w = rng.standard_normal((G * gs, 24))
    bias = rng.uniform(-0.1, 0.1, G)
    sub = O.make_subsample_index(G * gs, gs, spg, 2)
    idx, _ = O.grouped_topk_select(x, w, gs, 4, sub, spg, bias)
    perm = rng.permutation(G)                       # new group n = old group perm[n]
    w2 = w.reshape(G, gs, 24)[perm].reshape(G * gs, 24)
    sub2 = np.concatenate([sub[perm[n] * spg:(perm[n] + 1) * spg] - perm[n] * gs + n * gs
                           for n in range(G)])
    idx2, _ = O.grouped_topk_select(x, w2, gs, 4, sub2, spg, bias[perm])
    inv = np.argsort(perm)                           # old group o is new group inv[o]
    assert np.array_equal(np.sort(inv[idx], axis=1), idx2)


def test_near_tie_band():
    s = np.array([[1.0, 1.0 + 5e-6, 0.0], [1.0, 0.9, 0.0], [2.0, 1.0, 1.0 - 1e-6]])
    assert O.near_tie_tokens(s, 1).tolist() == [True, False, False]
    assert O.near_tie_tokens(s, 2).tolist() == [False, False, True]


def test_group_counts():
    idx = np.array([[0, 2], [1, 2], [2, 3]])
    assert O.group_counts(idx, 5).tolist() == [1, 1, 3, 1, 0]
