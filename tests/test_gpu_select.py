"""GPU parity: grouped top-k selection vs the oracle."""
import numpy as np
import pytest
import torch

import group_sparse_swiglu_amd as E
from gpu_common import f64, inputs, note, require_gpu, to_dev
from oracle import esg_oracle as O
from parity_util import check_selection

pytestmark = pytest.mark.gpu


def _select(inp, k, **kw):
    return E.grouped_topk_select(to_dev(inp["x"]), to_dev(inp["wg"]), inp["gs"], k, to_dev(inp["sub"]),
                                 inp["spg"], to_dev(inp["bias"]), return_counts=True, **kw)


def _oracle(inp, k, rows=None):
    x = inp["x"] if rows is None else inp["x"][rows]
    return O.grouped_topk_select(f64(x), f64(inp["wg"]), inp["gs"], k,
                                 None if inp["sub"] is None else inp["sub"].numpy(), inp["spg"],
                                 None if inp["bias"] is None else inp["bias"].numpy())


CASES = [
    # name, T, d, F, gs, k, dtype, spg, bias, sample
    ("tiny_f32", 256, 128, 512, 32, 4, "f32", None, False, None),
    ("s128m_bf16", 8192, 768, 2048, 64, 8, "bf16", 8, True, None),
    ("s370m_bf16", 16384, 1024, 2688, 128, 5, "bf16", 16, True, None),
    ("s1p3b_bf16", 32768, 2048, 5504, 128, 11, "bf16", 16, True, 4096),
    ("one_token", 1, 64, 256, 16, 3, "bf16", 4, True, None),
    ("ragged_77", 77, 96, 384, 32, 2, "bf16", None, True, None),
    ("spg12", 200, 128, 1024, 32, 3, "bf16", 12, True, None),
    ("g256", 300, 64, 4096, 16, 7, "bf16", 5, True, None),
    ("g512_small_tile_path", 150, 32, 8192, 16, 3, "f32", None, True, None),
    ("k_equals_g", 100, 64, 128, 16, 8, "bf16", None, False, None),
    ("d16", 130, 16, 256, 16, 4, "bf16", 16, False, None),
    ("f32_subsample", 513, 256, 2048, 128, 5, "f32", 16, True, None),
    # 128-token workgroups (chosen from 128 tokens per CU up)
    ("rows256_t16384", 16384, 256, 2048, 64, 6, "bf16", 8, True, None),
    ("bm128_g24_ragged", 32900, 128, 1536, 64, 5, "bf16", 4, True, None),
    ("bm128_g100", 32768, 64, 1600, 16, 4, "bf16", 1, True, None),
    # the eugen_sparse README's layer: 128 groups of 32, 8 sampled rows each
    ("readme_g128", 16384, 512, 4096, 32, 8, "bf16", 8, True, None),
    ("g200_ragged", 333, 64, 3200, 16, 9, "bf16", 4, True, None),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_select_parity(case):
    require_gpu()
    name, T, d, F, gs, k, dtype, spg, bias, sample = case
    note(f"select {name} T={T} d={d} F={F} gs={gs} k={k} {dtype} spg={spg}")
    inp = inputs(T, d, F, gs, dtype, seed=0, bias=bias, spg=spg)
    idx, counts = _select(inp, k)
    torch.cuda.synchronize()
    idx_h = idx.cpu().numpy()
    rows = None
    if sample is not None:
        rows = np.sort(np.random.default_rng(1).choice(T, sample, replace=False))
    oidx, scores = _oracle(inp, k, rows)
    ties = check_selection(idx_h if rows is None else idx_h[rows], oidx, scores, k)
    assert np.array_equal(counts.cpu().numpy(), np.bincount(idx_h.ravel(), minlength=F // gs))
    print(f"  near-tie tokens exempted: {ties}")


def test_select_batch_invariant_and_deterministic():
    require_gpu()
    note("select batch invariance s128m")
    inp = inputs(8192, 768, 2048, 64, "bf16", seed=3, bias=True, spg=8)
    a, _ = _select(inp, 8)
    b, _ = _select(inp, 8)
    part = dict(inp, x=inp["x"][1000:3001])
    c, _ = _select(part, 8)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.equal(a[1000:3001], c)


@pytest.mark.parametrize("G", [6, 100, 200])
def test_select_exact_ties_take_lowest_ids(G):
    """Every group identical: the k lowest ids win (the rank rule's tie
    break), for the one-wave ranking (G <= 64) and the lane-held scores of
    64 < G <= 256."""
    require_gpu()
    note(f"select exact ties G={G}")
    T, d, gs, k = 70, 64, 16, 3
    inp = inputs(T, d, gs * G, gs, "bf16", seed=4, bias=False)
    inp["wg"] = inp["wg"][:gs].repeat(G, 1)           # every group identical
    idx, counts = _select(inp, k)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), np.tile(np.arange(k), (T, 1)))
    assert counts.cpu().tolist() == [T] * k + [0] * (G - k)


def test_select_skewed_bias():
    require_gpu()
    note("select skewed bias")
    import esg_inputs as I
    inp = inputs(4096, 256, 2048, 64, "bf16", seed=5, bias=False, spg=8)
    inp["bias"] = I.skewed_bias(32, hot=4, level=1000.0)   # far above any energy here
    idx, counts = _select(inp, 8)
    torch.cuda.synchronize()
    oidx, scores = _oracle(inp, 8)
    check_selection(idx.cpu().numpy(), oidx, scores, 8)
    assert counts[:4].cpu().tolist() == [4096] * 4


SPLIT_CASES = [
    # name, T, d, F, gs, k, dtype, spg, bias: batches with fewer 32-token blocks than CUs
    ("decode64_1p3b", 64, 2048, 5504, 128, 11, "bf16", 16, True),
    ("prefill4096_1p3b", 4096, 2048, 5504, 128, 11, "bf16", 16, True),
    ("t1000_128m", 1000, 768, 2048, 64, 8, "bf16", 8, True),
    ("one_token", 1, 64, 256, 16, 3, "bf16", 4, True),
    ("spg12_straddling", 333, 128, 1024, 32, 3, "bf16", 12, True),
    ("g100_200rows", 200, 64, 1600, 16, 4, "bf16", 2, True),
    ("g256", 300, 64, 4096, 16, 7, "bf16", 5, False),
    ("f32_full_rows", 150, 96, 1024, 64, 4, "f32", None, True),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=[c[0] for c in SPLIT_CASES])
def test_select_workspace_split_is_bitwise_the_one_launch_selection(case):
    """With the energy table the groups of a token block are spread over
    workgroups; the result is bitwise that of the one-launch selection, and
    both match the oracle."""
    require_gpu()
    name, T, d, F, gs, k, dtype, spg, bias = case
    note(f"select split {name}")
    inp = inputs(T, d, F, gs, dtype, seed=6, bias=bias, spg=spg)
    ws = torch.empty(E.select_workspace_size(T, F, gs), dtype=torch.uint8, device="cuda")
    a, ca = _select(inp, k, workspace=False)
    b, cb = _select(inp, k, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(ca, cb)
    rows = None if T <= 1024 else np.sort(np.random.default_rng(3).choice(T, 512, replace=False))
    oidx, scores = _oracle(inp, k, rows)
    b_h = b.cpu().numpy()
    check_selection(b_h if rows is None else b_h[rows], oidx, scores, k)
