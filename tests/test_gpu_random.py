"""GPU parity on seeded random shapes: selection, then the forward and backward
given the oracle's routing, against the oracle.  The shapes mix group sizes,
widths, ragged token counts, k, subsampling and bias, so that the launch rules
(block widths, stage counts, bucketing and selection paths) meet in
combinations the hand-picked cases do not list.  Bounds as in the other parity
tests: selection exact outside near-ties, relative max-abs 1e-4 (fp32) and
2e-2 (bf16) for outputs and gradients."""
import numpy as np
import pytest
import torch

import group_sparse_swiglu_amd as E
from gpu_common import DEV, f64, inputs, note, require_gpu, to_dev
from oracle import esg_oracle as O
from parity_util import assert_close, check_selection

pytestmark = pytest.mark.gpu


def _shapes(n=15, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        gs = [16, 32, 64, 128, 256][i % 5]
        groups = int(rng.integers(2, 41))
        d = 16 * int(rng.integers(1, 66))               # 16 .. 1040
        tokens = int(rng.integers(1, 2001))
        k = int(rng.integers(1, groups + 1))
        dtype = "f32" if i % 4 == 3 else "bf16"
        spg = None if rng.random() < 0.4 else int(rng.integers(1, gs + 1))
        bias = bool(rng.random() < 0.6)
        # keep the fp64 oracle within seconds
        while tokens * groups * gs * d > 6e8:
            tokens = max(1, tokens // 2)
        out.append((f"r{i}_T{tokens}_d{d}_G{groups}x{gs}_k{k}_{dtype}", tokens, d, groups * gs, gs, k, dtype, spg,
                    bias))
    return out


SHAPES = _shapes()


@pytest.mark.parametrize("case", SHAPES, ids=[c[0] for c in SHAPES])
def test_random_shape_parity(case):
    require_gpu()
    name, T, d, F, gs, k, dtype, spg, bias = case
    note(f"random {name} spg={spg} bias={bias}")
    inp = inputs(T, d, F, gs, dtype, seed=T + d, bias=bias, spg=spg)
    bias_h = None if inp["bias"] is None else inp["bias"].numpy()
    sub_h = None if inp["sub"] is None else inp["sub"].numpy()
    # selection (whichever path the batch size picks)
    idx, counts = E.grouped_topk_select(to_dev(inp["x"]), to_dev(inp["wg"]), gs, k, to_dev(inp["sub"]), spg,
                                        to_dev(inp["bias"]), return_counts=True)
    torch.cuda.synchronize()
    oidx, scores = O.grouped_topk_select(f64(inp["x"]), f64(inp["wg"]), gs, k, sub_h, spg, bias_h)
    check_selection(idx.cpu().numpy(), oidx, scores, k)
    assert np.array_equal(counts.cpu().numpy(), np.bincount(idx.cpu().numpy().ravel(), minlength=F // gs))
    # forward and backward given the oracle's routing
    x, wg, wu, wd, dy = (to_dev(inp[n]) for n in ("x", "wg", "wu", "wd", "dy"))
    y, ctx = E.sparse_swiglu_fwd(x, wg, wu, wd, torch.as_tensor(oidx, dtype=torch.int32).to(DEV), gs)
    grads = E.sparse_swiglu_bwd(dy, x, wg, wu, wd, ctx)
    torch.cuda.synchronize()
    ry = O.sparse_swiglu_forward(f64(inp["x"]), f64(inp["wg"]), f64(inp["wu"]), f64(inp["wd"]), oidx, gs)
    rg = O.sparse_swiglu_backward(f64(inp["dy"]), f64(inp["x"]), f64(inp["wg"]), f64(inp["wu"]), f64(inp["wd"]),
                                  oidx, gs)
    for nm, g, r in zip(("y", "dx", "dW_gate", "dW_up", "dW_down"), (y,) + tuple(grads), (ry,) + tuple(rg)):
        assert_close(nm, f64(g), r, dtype)
