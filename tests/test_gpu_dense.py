"""GPU parity of the dense limit (idx = NULL, every group active): the fused
dense forward and the recompute backward against the oracle with every group
selected.  Bounds: relative max-abs 2e-2 (bf16)."""
import numpy as np
import pytest
import torch

import group_sparse_swiglu_amd as E
from gpu_common import DEV, f64, inputs, note, require_gpu, to_dev
from oracle import esg_oracle as O
from parity_util import assert_close

pytestmark = pytest.mark.gpu


def _run_dense(inp, ws=None):
    x, wg, wu, wd, dy = (to_dev(inp[n]) for n in ("x", "wg", "wu", "wd", "dy"))
    y, ctx = E.sparse_swiglu_fwd(x, wg, wu, wd, None, inp["gs"], workspace=ws)
    grads = E.sparse_swiglu_bwd(dy, x, wg, wu, wd, ctx, workspace=ws)
    torch.cuda.synchronize()
    return (y,) + tuple(grads)


def _all_groups(T, G):
    return np.tile(np.arange(G, dtype=np.int32), (T, 1))


DENSE = [
    # name, T, d, F, gs   (notes)
    ("small", 200, 128, 512, 64),            # one chunk, whole 128-neuron blocks
    ("ragged_f448_d208", 257, 208, 448, 64),  # last neuron block half full, d not a multiple of 64
    ("d16", 70, 16, 256, 32),
    ("ragged_d400", 300, 400, 384, 64),      # second 256-d weight-gradient block: 128 + 16 d
    ("d2048_max", 100, 2048, 256, 128),      # widest d the fused forward holds
    ("two_chunks", 9000, 64, 256, 128),      # backward over 2 token chunks (fp32 dW accumulation)
    ("three_chunks", 20000, 32, 128, 64),    # 3 chunks: first / middle / last accumulation modes
]


@pytest.mark.parametrize("case", DENSE, ids=[c[0] for c in DENSE])
def test_dense_matches_oracle(case):
    require_gpu()
    name, T, d, F, gs = case
    note(f"dense {name}")
    inp = inputs(T, d, F, gs, "bf16", seed=21, bias=False)
    idx = _all_groups(T, F // gs)
    outs = _run_dense(inp)
    W = [f64(inp[n]) for n in ("wg", "wu", "wd")]
    y = O.sparse_swiglu_forward(f64(inp["x"]), *W, idx, gs)
    grads = O.sparse_swiglu_backward(f64(inp["dy"]), f64(inp["x"]), *W, idx, gs)
    errs = {}
    for nm, g, r in zip(("y", "dx", "dW_gate", "dW_up", "dW_down"), outs, (y,) + tuple(grads)):
        errs[nm] = assert_close(nm, f64(g), r, "bf16")
    print("  rel errors:", {k: f"{v:.2e}" for k, v in errs.items()})


def test_dense_equals_all_groups_listed():
    """idx = NULL with k = G computes what the routed path computes when every
    token lists every group (to bf16 rounding: different kernels)."""
    require_gpu()
    note("dense vs routed all-groups")
    T, d, F, gs = 640, 256, 1024, 128
    inp = inputs(T, d, F, gs, "bf16", seed=22, bias=False)
    dense = _run_dense(inp)
    x, wg, wu, wd, dy = (to_dev(inp[n]) for n in ("x", "wg", "wu", "wd", "dy"))
    idx = torch.as_tensor(_all_groups(T, F // gs)).to(DEV)
    y, ctx = E.sparse_swiglu_fwd(x, wg, wu, wd, idx, gs)
    routed = (y,) + tuple(E.sparse_swiglu_bwd(dy, x, wg, wu, wd, ctx))
    torch.cuda.synchronize()
    for nm, a, b in zip(("y", "dx", "dW_gate", "dW_up", "dW_down"), dense, routed):
        assert_close(nm, f64(a), f64(b), "bf16")


def test_dense_deterministic():
    require_gpu()
    note("dense determinism")
    inp = inputs(9000, 64, 256, 128, "bf16", seed=23, bias=False)
    a = _run_dense(inp)
    b = _run_dense(inp)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_dense_zero_tokens():
    require_gpu()
    note("dense zero tokens")
    inp = inputs(0, 64, 256, 64, "bf16", seed=1, bias=False)
    y, dx, dwg, dwu, dwd = _run_dense(inp)
    assert y.shape == (0, 64)
    for t in (dwg, dwu, dwd):
        assert torch.count_nonzero(t) == 0


def test_dense_1p3b_sampled():
    """Full dense 1.3B shape (65536 tokens, d 2048, d_ff 5504, 43 groups of
    128): y and dx on sampled tokens, dW on sampled neurons."""
    require_gpu()
    T, d, F, gs = 65536, 2048, 5504, 128
    note("dense sampled dense1p3b")
    inp = inputs(T, d, F, gs, "bf16", seed=0, bias=False)
    y, dx, dwg, dwu, dwd = _run_dense(inp)
    idx = _all_groups(T, F // gs)
    rng = np.random.default_rng(5)
    toks = np.sort(rng.choice(T, 64, replace=False))
    xs, dys = f64(inp["x"][toks]), f64(inp["dy"][toks])
    W = [f64(inp[n]) for n in ("wg", "wu", "wd")]
    assert_close("y", f64(y[toks]), O.swiglu_rows(xs, *W, idx[toks], gs), "bf16")
    assert_close("dx", f64(dx[toks]), O.dx_rows(dys, xs, *W, idx[toks], gs), "bf16")
    neu = np.sort(rng.choice(F, 12, replace=False))
    rg, ru, rd = O.dw_neuron_rows(neu, f64(inp["dy"]), f64(inp["x"]), *W, idx, gs)
    assert_close("dW_gate", f64(dwg[neu]), rg, "bf16")
    assert_close("dW_up", f64(dwu[neu]), ru, "bf16")
    assert_close("dW_down", f64(dwd[:, neu]), rd, "bf16")
