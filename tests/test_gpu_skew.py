"""GPU parity of the sparse SwiGLU forward and backward under skewed routing.

The eugen_sparse README ("Pitfalls and limitations") notes that random inputs
spread tokens evenly over the groups while a trained model has popular groups,
so buckets are uneven: a hot group spans many tiles, others few or none.  y and
dx are compared on sampled tokens (each depends on its own token only), dW on
sampled neurons (hot groups included), against the fp64 oracle given the same
routing; groups that no token chose must get exact zeros.  Bounds: relative
max-abs 2e-2 (bf16)."""
import numpy as np
import pytest
import torch

import esg_inputs as I
import group_sparse_swiglu_amd as E
from gpu_common import DEV, f64, inputs, note, require_gpu, to_dev
from oracle import esg_oracle as O
from parity_util import assert_close

pytestmark = pytest.mark.gpu


def _hot(G):
    return sorted({0, G // 4, G // 2, (3 * G) // 4})


def _run(inp, idx):
    x, wg, wu, wd, dy = (to_dev(inp[n]) for n in ("x", "wg", "wu", "wd", "dy"))
    y, ctx = E.sparse_swiglu_fwd(x, wg, wu, wd, torch.as_tensor(idx, dtype=torch.int32).to(DEV), inp["gs"])
    grads = E.sparse_swiglu_bwd(dy, x, wg, wu, wd, ctx)
    torch.cuda.synchronize()
    return (y,) + tuple(grads)


def _sampled_compare(inp, idx, outs, neurons, seed=3):
    y, dx, dwg, dwu, dwd = outs
    T = idx.shape[0]
    gs = inp["gs"]
    rng = np.random.default_rng(seed)
    toks = np.sort(rng.choice(T, min(T, 256), replace=False))
    xs, dys = f64(inp["x"][toks]), f64(inp["dy"][toks])
    W = [f64(inp[n]) for n in ("wg", "wu", "wd")]
    assert_close("y", f64(y[toks]), O.swiglu_rows(xs, *W, idx[toks], gs), "bf16")
    assert_close("dx", f64(dx[toks]), O.dx_rows(dys, xs, *W, idx[toks], gs), "bf16")
    neu = np.asarray(sorted(neurons))
    rg, ru, rd = O.dw_neuron_rows(neu, f64(inp["dy"]), f64(inp["x"]), *W, idx, gs)
    assert_close("dW_gate", f64(dwg[neu]), rg, "bf16")
    assert_close("dW_up", f64(dwu[neu]), ru, "bf16")
    assert_close("dW_down", f64(dwd[:, neu]), rd, "bf16")


def _exact_zeros_for_unused(idx, outs, G, gs):
    used = set(np.unique(idx).tolist())
    empty = [g for g in range(G) if g not in used]
    for g in empty:
        sl = slice(g * gs, (g + 1) * gs)
        assert torch.count_nonzero(outs[2][sl]) == 0, f"dW_gate of unused group {g}"
        assert torch.count_nonzero(outs[3][sl]) == 0, f"dW_up of unused group {g}"
        assert torch.count_nonzero(outs[4][:, sl]) == 0, f"dW_down of unused group {g}"
    return len(empty)


HOT_CASES = [
    # name, T, d, F, gs, k, spg  (the skewed bench line's workload shapes)
    ("s128m_hot4", 8192, 768, 2048, 64, 8, 8),
    ("s1p3b_hot4", 32768, 2048, 5504, 128, 11, 16),
    # the other shapes the skewed bench line runs: 370M, and the README's layer (groups of 32)
    ("s370m_hot4", 16384, 1024, 2688, 128, 5, 16),
    ("gs32_readme_hot4", 16384, 512, 4096, 32, 8, 8),
]


@pytest.mark.parametrize("case", HOT_CASES, ids=[c[0] for c in HOT_CASES])
def test_hot_bias_on_four_groups(case):
    """The oracle's selection with +10 added to the bias of 4 groups: every
    token takes the hot groups, whose buckets hold all T tokens."""
    require_gpu()
    name, T, d, F, gs, k, spg = case
    G = F // gs
    hot = _hot(G)
    note(f"skew {name} hot={hot}")
    inp = inputs(T, d, F, gs, "bf16", seed=21, bias=True, spg=spg)
    inp["bias"] = inp["bias"].clone()
    inp["bias"][hot] += 10.0
    idx = O.grouped_topk_select(f64(inp["x"]), f64(inp["wg"]), gs, k, inp["sub"].numpy(), spg,
                                inp["bias"].numpy())[0]
    counts = np.bincount(idx.ravel(), minlength=G)
    assert all(counts[h] == T for h in hot)
    outs = _run(inp, idx)
    rng = np.random.default_rng(5)
    neurons = {h * gs + int(rng.integers(gs)) for h in hot}
    neurons |= {int(v) for v in rng.choice(F, 20, replace=False)}
    _sampled_compare(inp, idx, outs, neurons)
    _exact_zeros_for_unused(idx, outs, G, gs)


def test_one_group_holds_every_token():
    """T = 16384 tokens all routed to group 7 (plus two others each): one
    bucket of T positions, 128 tiles of one group.  Its weight gradients are
    summed by position chunks (the bucket is far above the mean load) added in
    a fixed order, so a second backward gives the same bits."""
    require_gpu()
    T, d, F, gs, G = 16384, 1024, 2688, 128, 21
    note(f"skew one group T={T}")
    inp = inputs(T, d, F, gs, "bf16", seed=23, bias=False)
    other = I.random_group_idx(T, G - 1, 2, seed=7).numpy()
    other = other + (other >= 7)          # skip group 7
    idx = np.sort(np.concatenate([np.full((T, 1), 7, np.int32), other], axis=1), axis=1).astype(np.int32)
    outs = _run(inp, idx)
    rng = np.random.default_rng(8)
    neurons = {7 * gs + int(v) for v in rng.choice(gs, 6, replace=False)}
    neurons |= {int(v) for v in rng.choice(F, 12, replace=False)}
    _sampled_compare(inp, idx, outs, neurons)
    again = _run(inp, idx)
    for name, a, b in zip(("y", "dx", "dW_gate", "dW_up", "dW_down"), outs, again):
        assert torch.equal(a, b), f"{name} differs between two runs"


def test_four_groups_only_leave_the_rest_exactly_zero():
    """Every token picks 2 of 4 groups: the other 28 groups get exact-zero
    weight gradients, the used ones hold about T/2 tokens each."""
    require_gpu()
    T, d, F, gs = 8192, 768, 2048, 64
    G = F // gs
    used = np.array([3, 9, 17, 30])
    note("skew four groups only")
    inp = inputs(T, d, F, gs, "bf16", seed=25, bias=False)
    pick = I.random_group_idx(T, 4, 2, seed=11).numpy()
    idx = np.sort(used[pick], axis=1).astype(np.int32)
    outs = _run(inp, idx)
    rng = np.random.default_rng(9)
    neurons = {int(g) * gs + int(rng.integers(gs)) for g in used} | {1 * gs + 5, 20 * gs + 7}
    _sampled_compare(inp, idx, outs, neurons)
    assert _exact_zeros_for_unused(idx, outs, G, gs) == G - 4


def test_hot_group_of_two_sub_blocks_and_a_ragged_d():
    """Groups of 256 neurons (two 128-neuron sub-blocks per group) at d = 1040
    (the last 256-wide d-block of the weight gradients is 16 wide), every
    token routed to group 3 plus one other: the hot bucket (8192 positions, 4x
    the mean) is summed in chunks whose slots hold both sub-blocks; two runs
    give the same bits."""
    require_gpu()
    T, d, F, gs = 8192, 1040, 2048, 256
    G = F // gs
    note(f"skew two sub-blocks T={T} d={d} gs={gs}")
    inp = inputs(T, d, F, gs, "bf16", seed=27, bias=False)
    other = I.random_group_idx(T, G - 1, 1, seed=13).numpy()
    other = other + (other >= 3)          # skip group 3
    idx = np.sort(np.concatenate([np.full((T, 1), 3, np.int32), other], axis=1), axis=1).astype(np.int32)
    outs = _run(inp, idx)
    rng = np.random.default_rng(10)
    neurons = {3 * gs + int(v) for v in rng.choice(gs, 8, replace=False)}   # both sub-blocks of the hot group
    neurons |= {int(v) for v in rng.choice(F, 12, replace=False)}
    _sampled_compare(inp, idx, outs, neurons)
    again = _run(inp, idx)
    for name, a, b in zip(("y", "dx", "dW_gate", "dW_up", "dW_down"), outs, again):
        assert torch.equal(a, b), f"{name} differs between two runs"



def test_hot_group_among_more_than_64_groups():
    """80 groups of 128 (the weight-gradient plan scans the groups' chunk
    counts in two 64-lane passes), every token routed to group 70 plus three
    others: the hot bucket (4096 positions, 20 times the mean) is summed in
    chunks; dW on neurons of the hot group and of groups past 64."""
    require_gpu()
    T, d, gs, G = 4096, 256, 128, 80
    F = G * gs
    note(f"skew {G} groups T={T}")
    inp = inputs(T, d, F, gs, "bf16", seed=29, bias=False)
    other = I.random_group_idx(T, G - 1, 3, seed=17).numpy()
    other = other + (other >= 70)          # skip group 70
    idx = np.sort(np.concatenate([np.full((T, 1), 70, np.int32), other], axis=1), axis=1).astype(np.int32)
    outs = _run(inp, idx)
    rng = np.random.default_rng(12)
    neurons = {70 * gs + int(v) for v in rng.choice(gs, 6, replace=False)}
    neurons |= {g * gs + int(rng.integers(gs)) for g in (64, 65, 79)}
    neurons |= {int(v) for v in rng.choice(F, 10, replace=False)}
    _sampled_compare(inp, idx, outs, neurons)
    _exact_zeros_for_unused(idx, outs, G, gs)
