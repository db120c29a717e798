"""GPU parity: sparse SwiGLU forward and backward vs the oracle, given the
oracle's routing.  Bounds: relative max-abs 1e-4 (fp32), 2e-2 (bf16)."""
import numpy as np
import pytest
import torch

import esg_inputs as I
import group_sparse_swiglu_amd as E
from gpu_common import DEV, f64, inputs, note, require_gpu, to_dev
from oracle import esg_oracle as O
from parity_util import assert_close

pytestmark = pytest.mark.gpu


def _run(inp, idx_dev, ws=None):
    x, wg, wu, wd, dy = (to_dev(inp[n]) for n in ("x", "wg", "wu", "wd", "dy"))
    y, ctx = E.sparse_swiglu_fwd(x, wg, wu, wd, idx_dev, inp["gs"], workspace=ws)
    grads = E.sparse_swiglu_bwd(dy, x, wg, wu, wd, ctx, workspace=ws)
    torch.cuda.synchronize()
    return (y,) + tuple(grads)


def _oracle_routing(inp, k):
    return O.grouped_topk_select(f64(inp["x"]), f64(inp["wg"]), inp["gs"], k,
                                 None if inp["sub"] is None else inp["sub"].numpy(), inp["spg"],
                                 None if inp["bias"] is None else inp["bias"].numpy())[0]


def _full_compare(inp, idx, dtype):
    outs = _run(inp, torch.as_tensor(idx, dtype=torch.int32).to(DEV))
    y = O.sparse_swiglu_forward(f64(inp["x"]), f64(inp["wg"]), f64(inp["wu"]), f64(inp["wd"]), idx, inp["gs"])
    grads = O.sparse_swiglu_backward(f64(inp["dy"]), f64(inp["x"]), f64(inp["wg"]), f64(inp["wu"]),
                                     f64(inp["wd"]), idx, inp["gs"])
    errs = {}
    for name, g, r in zip(("y", "dx", "dW_gate", "dW_up", "dW_down"), outs, (y,) + tuple(grads)):
        errs[name] = assert_close(name, f64(g), r, dtype)
    print("  rel errors:", {k: f"{v:.2e}" for k, v in errs.items()})
    return outs


WORKLOAD_FULL = [
    ("tiny_f32", 256, 128, 512, 32, 4, "f32", None, False),
    ("s128m_bf16", 8192, 768, 2048, 64, 8, "bf16", 8, True),
    # the eugen_sparse README's layer (groups of 32, 8 of 128 active) at 1024 tokens
    ("gs32_d512_1k", 1024, 512, 4096, 32, 8, "bf16", 8, True),
]


@pytest.mark.parametrize("case", WORKLOAD_FULL, ids=[c[0] for c in WORKLOAD_FULL])
def test_ffn_workload_full(case):
    require_gpu()
    name, T, d, F, gs, k, dtype, spg, bias = case
    note(f"ffn full {name}")
    inp = inputs(T, d, F, gs, dtype, seed=0, bias=bias, spg=spg)
    _full_compare(inp, _oracle_routing(inp, k), dtype)


WORKLOAD_SAMPLED = [
    ("s370m_bf16", 16384, 1024, 2688, 128, 5, "bf16", 16, True),
    ("s1p3b_bf16", 32768, 2048, 5504, 128, 11, "bf16", 16, True),
    # 64-neuron groups with partial rows past the cached-store limit (about 270 MB)
    ("gs64_partials_270mb", 16384, 2048, 4096, 64, 4, "bf16", 8, True),
    # at most 256 tiles (one workgroup per CU) whose partial rows (213 MB at d 4096)
    # still pass the cached-store limit: the four-wave nontemporal forward
    ("gs64_d4096_one_round", 12000, 4096, 1024, 64, 2, "bf16", 16, True),
    # the eugen_sparse README's layer at its full bench size: 32-neuron blocks
    ("gs32_d512_readme", 16384, 512, 4096, 32, 8, "bf16", 8, True),
    # groups of 256 (two 128-neuron sub-blocks) past the pair threshold (1039 tiles x 2)
    ("gs256_pairs_two_subblocks", 32768, 1024, 4096, 256, 4, "bf16", 16, True),
    # the ends of the active-fraction sweep at the 1.3B shape: one group per token
    # (single tiles), and every group (k = G = 43: pair tiles, 5.8 GB of partial rows)
    ("s1p3b_k1", 32768, 2048, 5504, 128, 1, "bf16", 16, True),
    ("s1p3b_k43", 32768, 2048, 5504, 128, 43, "bf16", 16, True),
]


@pytest.mark.parametrize("case", WORKLOAD_SAMPLED, ids=[c[0] for c in WORKLOAD_SAMPLED])
def test_ffn_workload_sampled(case):
    """Full-size run; y and dx checked on sampled tokens (each depends on its
    own token only), dW on sampled neurons (each needs that neuron's
    activations over all tokens)."""
    require_gpu()
    name, T, d, F, gs, k, dtype, spg, bias = case
    note(f"ffn sampled {name}")
    inp = inputs(T, d, F, gs, dtype, seed=0, bias=bias, spg=spg)
    idx = _oracle_routing(inp, k)
    y, dx, dwg, dwu, dwd = _run(inp, torch.as_tensor(idx).to(DEV))
    rng = np.random.default_rng(2)
    toks = np.sort(rng.choice(T, 256, replace=False))
    xs, dys = f64(inp["x"][toks]), f64(inp["dy"][toks])
    W = [f64(inp[n]) for n in ("wg", "wu", "wd")]
    assert_close("y", f64(y[toks]), O.swiglu_rows(xs, *W, idx[toks], gs), dtype)
    assert_close("dx", f64(dx[toks]), O.dx_rows(dys, xs, *W, idx[toks], gs), dtype)
    neu = np.sort(rng.choice(F, 24, replace=False))
    rg, ru, rd = O.dw_neuron_rows(neu, f64(inp["dy"]), f64(inp["x"]), *W, idx, gs)
    # rows of dW are compared against the scale of the sampled block
    assert_close("dW_gate", f64(dwg[neu]), rg, dtype)
    assert_close("dW_up", f64(dwu[neu]), ru, dtype)
    assert_close("dW_down", f64(dwd[:, neu]), rd, dtype)


EDGE = [
    # name, T, d, F, gs, k, dtype
    ("one_token", 1, 64, 256, 32, 2, "bf16"),
    ("ragged_300", 300, 96, 512, 64, 3, "bf16"),
    ("gs16_bf16", 200, 64, 256, 16, 5, "bf16"),
    ("gs16_f32", 150, 48, 128, 16, 3, "f32"),
    ("gs256_subblocks", 260, 128, 1024, 256, 2, "bf16"),
    ("gs128_f32_subblocks", 200, 64, 512, 128, 2, "f32"),
    ("f_not_pow2", 333, 80, 192, 64, 2, "bf16"),
    ("d16", 100, 16, 128, 32, 2, "bf16"),
    ("k1", 500, 128, 1024, 64, 1, "bf16"),
    ("k_equals_g", 120, 64, 256, 32, 8, "bf16"),
    ("empty_groups", 3, 64, 1024, 32, 2, "bf16"),
    ("f32_wide", 513, 256, 1024, 64, 4, "f32"),
    ("d16_gs64", 77, 16, 256, 64, 2, "bf16"),
    ("d208_gs128", 150, 208, 512, 128, 2, "bf16"),
    ("d1040_gs64_k3", 700, 1040, 640, 64, 3, "bf16"),
    ("d400_gs128_k3", 333, 400, 1024, 128, 3, "bf16"),  # ragged 256-d weight-gradient block
    # 128 groups: enough tiles (>= 128) for 128-neuron blocks; fewer tiles run 64-neuron blocks
    ("gs128_blocks_d208", 300, 208, 16384, 128, 4, "bf16"),
    ("gs128_blocks_d400_k3", 333, 400, 16384, 128, 3, "bf16"),
]


@pytest.mark.parametrize("case", EDGE, ids=[c[0] for c in EDGE])
def test_ffn_edge_shapes(case):
    require_gpu()
    name, T, d, F, gs, k, dtype = case
    note(f"ffn edge {name}")
    inp = inputs(T, d, F, gs, dtype, seed=11, bias=False)
    idx = I.random_group_idx(T, F // gs, k, seed=T).numpy()
    outs = _full_compare(inp, idx, dtype)
    used = set(idx.ravel().tolist())
    for g in range(F // gs):           # groups nobody chose: exact zeros
        if g not in used:
            sl = slice(g * gs, (g + 1) * gs)
            assert torch.count_nonzero(outs[2][sl]) == 0
            assert torch.count_nonzero(outs[3][sl]) == 0
            assert torch.count_nonzero(outs[4][:, sl]) == 0


# The bf16 forward runs as two launches (phase 1 over K ranges, phase 2 over
# d-block ranges) while the tile bound floor((T*k + G*127)/128) of 64-neuron
# blocks is at most 128, else as one.  With G = 16, k = 2: 7239 tokens give 128
# tiles, 7240 give 129; d = 80 leaves a ragged K stage and d-block.
@pytest.mark.parametrize("tokens", [7239, 7240])
def test_ffn_forward_split_boundary(tokens):
    require_gpu()
    G, gs, k, d = 16, 64, 2, 80
    assert (tokens * k + G * 127) // 128 == (128 if tokens == 7239 else 129)
    note(f"split boundary T={tokens} d={d} G={G}x{gs} k={k}")
    inp = inputs(tokens, d, G * gs, gs, "bf16", seed=tokens, bias=True, spg=16)
    _full_compare(inp, _oracle_routing(inp, k), "bf16")


def test_ffn_deterministic_and_unsorted_slots():
    require_gpu()
    note("ffn determinism")
    inp = inputs(4096, 256, 2048, 64, "bf16", seed=12, bias=False)
    idx = I.random_group_idx(4096, 32, 6, seed=3)
    a = _run(inp, idx.to(DEV))
    b = _run(inp, idx.to(DEV))
    perm = torch.argsort(torch.rand(4096, 6, generator=torch.Generator().manual_seed(1)), dim=1)
    c = _run(inp, torch.gather(idx, 1, perm).to(DEV))
    for u, v in zip(a, b):
        assert torch.equal(u, v)
    # slot order only changes the order of the k-way sum
    for name, u, v in zip(("y", "dx", "dWg", "dWu", "dWd"), a, c):
        assert_close(name, f64(u), f64(v), "bf16")
    for u, v in zip(a[2:], c[2:]):      # dW does not depend on slot order at all
        assert torch.equal(u, v)


def test_ffn_zero_tokens():
    require_gpu()
    note("ffn zero tokens")
    inp = inputs(0, 64, 256, 32, "bf16", seed=1, bias=False)
    idx = torch.zeros(0, 2, dtype=torch.int32)
    y, dx, dwg, dwu, dwd = _run(inp, idx.to(DEV))
    assert y.shape == (0, 64) and dx.shape == (0, 64)
    for t in (dwg, dwu, dwd):
        assert torch.count_nonzero(t) == 0


def test_ffn_invalid_ids_are_skipped():
    require_gpu()
    note("ffn invalid ids")
    T, d, F, gs = 64, 64, 256, 32
    inp = inputs(T, d, F, gs, "bf16", seed=2, bias=False)
    idx = I.random_group_idx(T, F // gs, 2, seed=5)
    bad = idx.clone()
    bad[::2, 1] = F // gs + 3            # out of range on even tokens
    bad[1::4, 1] = bad[1::4, 0]          # duplicates on some odd tokens
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    x = to_dev(inp["x"])
    y, _ = E.sparse_swiglu_fwd(x, to_dev(inp["wg"]), to_dev(inp["wu"]), to_dev(inp["wd"]), bad.to(DEV), gs,
                               status=status)
    torch.cuda.synchronize()
    assert status.item() == (E.STATUS_GROUP_OUT_OF_RANGE | E.STATUS_GROUP_DUPLICATE)
    keep = bad.clone()
    W = [f64(inp[n]) for n in ("wg", "wu", "wd")]
    for t in range(T):
        valid = [g for j, g in enumerate(bad[t].tolist()) if 0 <= g < F // gs and g not in bad[t, :j].tolist()]
        ref = O.swiglu_rows(f64(inp["x"][t:t + 1]), *W, np.array([valid]), gs)
        assert_close(f"y[{t}]", f64(y[t:t + 1]), ref, "bf16")


def test_autograd_wrapper_matches_entry_points():
    require_gpu()
    note("autograd wrapper")
    inp = inputs(512, 128, 512, 32, "bf16", seed=9, bias=False)
    idx = I.random_group_idx(512, 16, 3, seed=9).to(DEV)
    params = [to_dev(inp[n]).requires_grad_(True) for n in ("x", "wg", "wu", "wd")]
    y = E.sparse_swiglu_ffn(*params, idx, 32)
    y.backward(to_dev(inp["dy"]))
    ref = _run(inp, idx)
    assert torch.equal(y.detach(), ref[0])
    for p, r in zip(params, ref[1:]):
        assert torch.equal(p.grad, r)


@pytest.mark.parametrize("T", [8192, 300])
def test_backward_on_a_second_stream_is_bitwise_the_one_stream_backward(T):
    """esg_sparse_swiglu_bwd_overlap runs the weight gradients on a caller
    stream beside the dx sum; every gradient is bitwise the one-stream result
    (8192 tokens: the tile path of the 128M shape; 300: the split forward)."""
    require_gpu()
    note(f"bwd overlap T={T}")
    inp = inputs(T, 768, 2048, 64, "bf16", seed=13, bias=False)
    idx = I.random_group_idx(T, 32, 8, seed=13).to(DEV)
    x, wg, wu, wd, dy = (to_dev(inp[n]) for n in ("x", "wg", "wu", "wd", "dy"))
    _, ctx = E.sparse_swiglu_fwd(x, wg, wu, wd, idx, 64)
    one = E.sparse_swiglu_bwd(dy, x, wg, wu, wd, ctx)
    two = E.sparse_swiglu_bwd(dy, x, wg, wu, wd, ctx, aux_stream=torch.cuda.Stream())
    torch.cuda.synchronize()
    for u, v in zip(one, two):
        assert torch.equal(u, v)


def _ragged_pair_routing(T, k, G, special):
    """Token t takes special group g iff t < special[g] (so group g holds
    exactly special[g] tokens), then fills its k slots from groups
    len(special) .. G-1 by a fixed stride pattern (distinct per token)."""
    ns = len(special)
    rest = G - ns
    idx = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        row = [g for g in range(ns) if t < special[g]]
        j = 0
        while len(row) < k:
            row.append(ns + (t * 7 + j * 3) % rest)
            j += 1
        idx[t] = row
    return idx


def test_pair_tiles_with_ragged_and_empty_groups():
    """23335 tokens of the 1.3B shape: the first size whose training layout
    pads groups to pairs of tiles (2048 single tiles by the bound).  Groups of
    0, 1, 128, 129, 255, 256, 257, 383, 384 and 385 tokens give pairs with one
    real row, a whole padding tile, a ragged second tile, and no pair at all.
    y and dx on sampled tokens (the group boundaries among them), dW on
    neurons of every special group, against the fp64 oracle; the empty group's
    weight gradients are exact zeros."""
    require_gpu()
    T, d, F, gs, k = 23335, 2048, 5504, 128, 11
    G = F // gs
    special = [1, 128, 129, 255, 256, 257, 0, 383, 384, 385]
    assert (T * k + G * 127) // 128 == 2048
    note(f"pair tiles ragged T={T}")
    inp = inputs(T, d, F, gs, "bf16", seed=57, bias=False)
    idx = _ragged_pair_routing(T, k, G, special)
    counts = np.bincount(idx.ravel(), minlength=G)
    assert list(counts[:len(special)]) == special and all(len(set(r)) == k for r in idx[:400])
    y, dx, dwg, dwu, dwd = _run(inp, torch.as_tensor(idx).to(DEV))
    rng = np.random.default_rng(58)
    toks = np.unique(np.concatenate([[0, 1, 127, 128, 129, 254, 255, 256, 257, 382, 383, 384, 385, T - 1],
                                     rng.choice(T, 40, replace=False)]))
    W = [f64(inp[n]) for n in ("wg", "wu", "wd")]
    xs, dys = f64(inp["x"][toks]), f64(inp["dy"][toks])
    assert_close("y", f64(y[toks]), O.swiglu_rows(xs, *W, idx[toks], gs), "bf16")
    assert_close("dx", f64(dx[toks]), O.dx_rows(dys, xs, *W, idx[toks], gs), "bf16")
    neu = np.array([g * gs + o for g in range(len(special)) if special[g] > 0 for o in (0, 77, gs - 1)]
                   + [30 * gs + 5])
    rg, ru, rd = O.dw_neuron_rows(neu, f64(inp["dy"]), f64(inp["x"]), *W, idx, gs)
    assert_close("dW_gate", f64(dwg[neu]), rg, "bf16")
    assert_close("dW_up", f64(dwu[neu]), ru, "bf16")
    assert_close("dW_down", f64(dwd[:, neu]), rd, "bf16")
    sl = slice(6 * gs, 7 * gs)       # group 6 holds no token
    assert torch.count_nonzero(dwg[sl]) == 0 and torch.count_nonzero(dwu[sl]) == 0
    assert torch.count_nonzero(dwd[:, sl]) == 0
