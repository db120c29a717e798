"""GPU parity: CSR bucketing is bit-exact with the oracle."""
import numpy as np
import pytest
import torch

import esg_inputs as I
import group_sparse_swiglu_amd as E
from gpu_common import DEV, note, require_gpu
from oracle import esg_oracle as O

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,G,k,shuffle", [(1, 2, 1, False), (100, 16, 4, False), (777, 43, 11, True),
                                           (8192, 32, 8, False), (32768, 43, 11, False), (5000, 1024, 3, True),
                                           (64, 8, 8, True), (129, 300, 128, True), (65, 43, 11, True),
                                           (64, 1024, 128, True), (0, 16, 4, False)])
def test_bucket_matches_oracle(T, G, k, shuffle):
    require_gpu()
    note(f"bucket T={T} G={G} k={k}")
    idx = I.random_group_idx(T, G, k, seed=T + G)
    if shuffle:   # slots need not be sorted
        g = torch.Generator().manual_seed(7)
        perm = torch.argsort(torch.rand(T, k, generator=g), dim=1)
        idx = torch.gather(idx, 1, perm)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    off, perm_t, inv = E.bucket_by_group(idx.to(DEV), G, status)
    torch.cuda.synchronize()
    o_off, o_perm, o_inv = O.bucket_by_group(idx.numpy(), G)
    assert np.array_equal(off.cpu().numpy(), o_off)
    assert np.array_equal(perm_t.cpu().numpy(), o_perm)
    assert np.array_equal(inv.cpu().numpy(), o_inv)
    assert status.item() == 0


def _invalid_idx(T, G, k, seed):
    """Ids drawn from [-3, G + 3) with many repeats: out-of-range ids and repeats in every block."""
    if T == 5:
        return torch.tensor([[1, 3, 5], [2, 2, 4], [-1, 9, 10], [7, 1000, 7], [0, 1, 2]], dtype=torch.int32)
    g = torch.Generator().manual_seed(seed)
    idx = torch.randint(-3, G + 3, (T, k), generator=g, dtype=torch.int32)
    idx[:, -1] = idx[:, 0]   # a repeat in every token
    return idx


@pytest.mark.parametrize("T,G,k", [(5, 10, 3), (300, 50, 6), (64, 40, 12)])
def test_bucket_skips_invalid_ids(T, G, k):
    require_gpu()
    note(f"bucket invalid ids T={T} G={G} k={k}")
    idx = _invalid_idx(T, G, k, seed=T)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    off, perm_t, inv = E.bucket_by_group(idx.to(DEV), G, status)
    torch.cuda.synchronize()
    # brute force over the valid (first occurrence, in range) pairs
    triples = []
    for t in range(idx.shape[0]):
        seen = set()
        for j, g in enumerate(idx[t].tolist()):
            if 0 <= g < G and g not in seen:
                seen.add(g)
                triples.append((g, t, j))
    triples.sort()
    counts = np.bincount([g for g, _, _ in triples], minlength=G)
    assert off.cpu().tolist() == [0] + np.cumsum(counts).tolist()
    assert perm_t.cpu().tolist()[:len(triples)] == [t for _, t, _ in triples]
    exp_inv = -np.ones(idx.shape, dtype=np.int64)
    for pos, (_, t, j) in enumerate(triples):
        exp_inv[t, j] = pos
    assert np.array_equal(inv.cpu().numpy(), exp_inv)
    assert status.item() == (E.STATUS_GROUP_OUT_OF_RANGE | E.STATUS_GROUP_DUPLICATE)


def test_bucket_deterministic():
    require_gpu()
    note("bucket determinism")
    idx = I.random_group_idx(20000, 43, 11, seed=2).to(DEV)
    a = E.bucket_by_group(idx, 43)
    b = E.bucket_by_group(idx, 43)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)
