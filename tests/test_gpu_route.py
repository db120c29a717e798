"""GPU parity: sigmoid top-k routing vs the oracle.  Indices and weights are
compared bit for bit on every row whose scores all lie away from an fp32
rounding midpoint (both sides round an fp64 sigmoid once; the rare rows with a
score within 2^-48 of a midpoint are checked for validity and closeness)."""
import numpy as np
import pytest
import torch

import esg_inputs as I
import group_sparse_swiglu_amd as E
from gpu_common import DEV, note, require_gpu
from oracle import routing_oracle as R

pytestmark = pytest.mark.gpu


def _compare(logits, bias, k, scaling, bias_dev=None):
    """Run the kernel and check it against the oracle (see the module doc)."""
    probs, idx = E.sigmoid_topk_routing(logits.to(DEV), bias.to(DEV) if bias_dev is None else bias_dev, k, scaling)
    torch.cuda.synchronize()
    probs, idx = probs.cpu().numpy(), idx.cpu().numpy()
    rp, ri = R.sigmoid_topk_routing(logits.numpy(), bias.numpy(), k, scaling)
    certain = ~R.near_rounding_boundary(logits.numpy()).any(axis=1)
    assert certain.mean() > 0.99
    assert np.array_equal(idx[certain], ri[certain])
    assert np.array_equal(probs[certain].view(np.uint32), rp[certain].view(np.uint32))
    for t in np.nonzero(~certain)[0]:
        assert len(set(idx[t].tolist())) == k and ((idx[t] >= 0) & (idx[t] < logits.shape[1])).all()
        np.testing.assert_allclose(np.sort(probs[t]), np.sort(rp[t]), rtol=1e-6)
    return probs, idx


CASES = [
    # name, T, E, k, scaling, logit options
    ("e256_k8_scaled", 4096, 256, 8, 2.5, {}),
    ("e43_k11", 1000, 43, 11, None, {}),
    ("e64_k2", 777, 64, 2, None, {"scale": 3.0}),
    ("e128_k6", 513, 128, 6, 1.0, {}),
    ("e300_k32", 130, 300, 32, None, {}),
    ("e301_k32_unaligned", 130, 301, 32, None, {}),
    ("e2048_k32_max", 64, 2048, 32, 2.5, {}),
    ("e1024_k8", 67, 1024, 8, None, {}),
    ("e1_k1", 9, 1, 1, None, {}),
    ("e16_k16_all", 100, 16, 16, None, {}),
    ("ties_levels3", 500, 64, 8, None, {"levels": 3}),
    ("ties_levels2_e256", 300, 256, 32, None, {"levels": 2}),
    ("saturated", 500, 96, 12, 2.0, {"saturate": True}),
    ("one_token", 1, 256, 8, 2.5, {}),
    # two distinct scores and no bias: over 64 experts tie at the top key
    ("ties_no_bias_e256", 200, 256, 8, None, {"levels": 2, "zero_bias": True}),
    ("saturated_no_bias_e2048", 40, 2048, 32, None, {"saturate": True, "zero_bias": True}),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_routing_matches_oracle(case):
    require_gpu()
    name, T, Ex, k, scaling, opts = case
    note(f"routing {name}")
    opts = dict(opts)
    zero_bias = opts.pop("zero_bias", False)
    logits, bias = I.make_routing_inputs(T, Ex, seed=T + Ex, **opts)
    if zero_bias:
        bias = torch.zeros_like(bias)
    _compare(logits, bias, k, scaling)


def test_routing_strided_bias_and_zero_tokens():
    require_gpu()
    note("routing strided bias")
    logits, bias = I.make_routing_inputs(257, 96, seed=4)
    big = torch.zeros(96, 3)
    big[:, 1] = bias
    view = big.to(DEV)[:, 1]
    assert view.stride(0) == 3
    _compare(logits, bias, 6, None, bias_dev=view)
    p, i = E.sigmoid_topk_routing(torch.zeros(0, 96, device=DEV), bias.to(DEV), 6)
    assert p.shape == (0, 6) and i.shape == (0, 6)


@pytest.mark.parametrize("wl", sorted(I.ROUTING_WORKLOADS))
def test_routing_workload_full(wl):
    """The bench shapes, every row against the oracle."""
    require_gpu()
    w = I.ROUTING_WORKLOADS[wl]
    note(f"routing workload {wl}")
    logits, bias = I.make_routing_inputs(w.tokens, w.experts, seed=0)
    _compare(logits, bias, w.k, w.scaling)


def test_routing_batch_invariant_bitwise():
    require_gpu()
    note("routing batch invariance")
    logits, bias = I.make_routing_inputs(4096, 256, seed=8)
    ld, bd = logits.to(DEV), bias.to(DEV)
    p_all, i_all = E.sigmoid_topk_routing(ld, bd, 8, 2.5)
    for lo, hi in ((0, 1), (1234, 1271), (4090, 4096)):
        p, i = E.sigmoid_topk_routing(ld[lo:hi].contiguous(), bd, 8, 2.5)
        assert torch.equal(i, i_all[lo:hi]) and torch.equal(p, p_all[lo:hi])
    p2, i2 = E.sigmoid_topk_routing(ld, bd, 8, 2.5)
    assert torch.equal(p2, p_all) and torch.equal(i2, i_all)
