"""Forward-only (inference) path: saved = NULL keeps nothing for a backward.
y must equal the training forward's y bit for bit, and match the oracle at
decode-size batches (a handful of tokens, mostly padding in every tile)."""
import numpy as np
import pytest
import torch

import esg_inputs as I
import group_sparse_swiglu_amd as E
from gpu_common import DEV, f64, inputs, note, require_gpu, to_dev
from oracle import esg_oracle as O
from parity_util import assert_close

pytestmark = pytest.mark.gpu

DECODE = [
    # name, T, d, F, gs, k, spg, dtype
    ("decode1_1p3b", 1, 2048, 5504, 128, 11, 16, "bf16"),
    ("decode8_1p3b", 8, 2048, 5504, 128, 11, 16, "bf16"),
    ("decode64_1p3b", 64, 2048, 5504, 128, 11, 16, "bf16"),
    ("decode5_128m", 5, 768, 2048, 64, 8, 8, "bf16"),
    ("decode3_f32", 3, 128, 512, 32, 4, None, "f32"),
]


@pytest.mark.parametrize("case", DECODE, ids=[c[0] for c in DECODE])
def test_inference_decode_matches_oracle(case):
    require_gpu()
    name, T, d, F, gs, k, spg, dtype = case
    note(f"inference {name}")
    inp = inputs(T, d, F, gs, dtype, seed=41, bias=True, spg=spg)
    x, wg, wu, wd = (to_dev(inp[n]) for n in ("x", "wg", "wu", "wd"))
    idx, _ = E.grouped_topk_select(x, wg, gs, k, to_dev(inp["sub"]), spg, to_dev(inp["bias"]), return_counts=True)
    y, ctx = E.sparse_swiglu_fwd(x, wg, wu, wd, idx, gs, for_backward=False)
    torch.cuda.synchronize()
    assert ctx.saved is None
    idx_h = idx.cpu().numpy()
    ref = O.sparse_swiglu_forward(f64(inp["x"]), f64(inp["wg"]), f64(inp["wu"]), f64(inp["wd"]), idx_h, gs)
    assert_close("y", f64(y), ref, dtype)
    with pytest.raises(E.EsgError):
        E.sparse_swiglu_bwd(to_dev(inp["dy"]), x, wg, wu, wd, ctx)


@pytest.mark.parametrize("gs", [64, 128])
def test_inference_equals_training_forward(gs):
    require_gpu()
    note(f"inference vs training gs={gs}")
    T, d, F, k = 3000, 512, 2048, 6
    inp = inputs(T, d, F, gs, "bf16", seed=42, bias=False)
    x, wg, wu, wd = (to_dev(inp[n]) for n in ("x", "wg", "wu", "wd"))
    idx = I.random_group_idx(T, F // gs, k, seed=42).to(DEV)
    y_train, _ = E.sparse_swiglu_fwd(x, wg, wu, wd, idx, gs)
    y_inf, _ = E.sparse_swiglu_fwd(x, wg, wu, wd, idx, gs, for_backward=False)
    torch.cuda.synchronize()
    assert torch.equal(y_train, y_inf)
