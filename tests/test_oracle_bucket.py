"""Pins for the oracle's CSR bucketing (counting sort by group)."""
import numpy as np
import pytest

from oracle import esg_oracle as O


def _random_idx(T, G, k, seed):
    rng = np.random.default_rng(seed)
    return np.sort(np.stack([rng.choice(G, k, replace=False) for _ in range(T)]), axis=1).astype(np.int32)


@pytest.mark.parametrize("T,G,k", [(1, 2, 1), (37, 5, 2), (200, 16, 4), (513, 43, 11), (64, 8, 8)])
def test_bucket_invariants(T, G, k):
    idx = _random_idx(T, G, k, T + G)
    offsets, perm_token, inv = O.bucket_by_group(idx, G)
    counts = np.bincount(idx.reshape(-1), minlength=G)
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts)
    assert sorted(perm_token.tolist()) == sorted(np.repeat(np.arange(T), k).tolist())
    assert sorted(inv.reshape(-1).tolist()) == list(range(T * k))
    for g in range(G):
        toks = perm_token[offsets[g]:offsets[g + 1]]
        assert np.all(np.diff(toks) > 0), "tokens ascending inside a bucket"
        assert all(g in idx[t] for t in toks)
    for t in range(T):
        for j in range(k):
            p = inv[t, j]
            assert perm_token[p] == t and offsets[idx[t, j]] <= p < offsets[idx[t, j] + 1]


def test_bucket_brute_force_sorted():
    """Against Python's sorted() over (group, token, slot) triples."""
    idx = _random_idx(60, 7, 3, 1)
    triples = sorted((int(g), t, j) for t in range(60) for j, g in enumerate(idx[t]))
    offsets, perm_token, inv = O.bucket_by_group(idx, 7)
    assert perm_token.tolist() == [t for _, t, _ in triples]
    for pos, (_, t, j) in enumerate(triples):
        assert inv[t, j] == pos


def test_bucket_unsorted_slots_and_empty_groups():
    idx = np.array([[3, 0], [0, 3], [3, 1]], dtype=np.int32)
    offsets, perm_token, inv = O.bucket_by_group(idx, 6)
    assert offsets.tolist() == [0, 2, 3, 3, 6, 6, 6]
    assert perm_token.tolist() == [0, 1, 2, 0, 1, 2]
    assert inv.tolist() == [[3, 0], [1, 4], [5, 2]]


def test_bucket_empty_batch():
    offsets, perm_token, inv = O.bucket_by_group(np.zeros((0, 3), dtype=np.int32), 4)
    assert offsets.tolist() == [0] * 5 and perm_token.size == 0 and inv.shape == (0, 3)
