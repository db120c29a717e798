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
from parity_util import assert_close, check_selection

pytestmark = pytest.mark.gpu

DECODE = [
    # name, T, d, F, gs, k, spg, dtype
    ("decode1_1p3b", 1, 2048, 5504, 128, 11, 16, "bf16"),
    ("decode8_1p3b", 8, 2048, 5504, 128, 11, 16, "bf16"),
    ("decode64_1p3b", 64, 2048, 5504, 128, 11, 16, "bf16"),
    ("decode5_128m", 5, 768, 2048, 64, 8, 8, "bf16"),
    ("decode3_f32", 3, 128, 512, 32, 4, None, "f32"),
]


def _routed_forward(inp, k, spg):
    """The inference path's two steps, each against the oracle: the selection
    kernel's ids against the oracle's selection (near ties exempt), and the
    forward (saved = NULL) given the oracle's routing against the oracle's
    forward for that routing.  Returns (y, oracle routing)."""
    gs = inp["gs"]
    x, wg, wu, wd = (to_dev(inp[n]) for n in ("x", "wg", "wu", "wd"))
    sub = None if inp["sub"] is None else to_dev(inp["sub"])
    bias = None if inp["bias"] is None else to_dev(inp["bias"])
    idx_gpu, _ = E.grouped_topk_select(x, wg, gs, k, sub, spg, bias, return_counts=True)
    oidx, scores = O.grouped_topk_select(f64(inp["x"]), f64(inp["wg"]), gs, k,
                                         None if inp["sub"] is None else inp["sub"].numpy(), spg,
                                         None if inp["bias"] is None else inp["bias"].numpy())
    y, ctx = E.sparse_swiglu_fwd(x, wg, wu, wd, torch.as_tensor(oidx, dtype=torch.int32).to(DEV), gs,
                                 for_backward=False)
    torch.cuda.synchronize()
    assert ctx.saved is None
    check_selection(idx_gpu.cpu().numpy(), oidx, scores, k)
    return y, ctx, oidx


@pytest.mark.parametrize("case", DECODE, ids=[c[0] for c in DECODE])
def test_inference_decode_matches_oracle(case):
    require_gpu()
    name, T, d, F, gs, k, spg, dtype = case
    note(f"inference {name}")
    inp = inputs(T, d, F, gs, dtype, seed=41, bias=True, spg=spg)
    y, ctx, oidx = _routed_forward(inp, k, spg)
    ref = O.sparse_swiglu_forward(f64(inp["x"]), f64(inp["wg"]), f64(inp["wu"]), f64(inp["wd"]), oidx, gs)
    assert_close("y", f64(y), ref, dtype)
    x, wg, wu, wd = (to_dev(inp[n]) for n in ("x", "wg", "wu", "wd"))
    with pytest.raises(E.EsgError):
        E.sparse_swiglu_bwd(to_dev(inp["dy"]), x, wg, wu, wd, ctx)


# At 24576 tokens of the 1.3B shape (2154 single tiles) the training forward
# pads each group to a pair of tiles and runs the pair kernel, the inference
# forward pads to one tile: the two layouts differ, the results must not.
@pytest.mark.parametrize("T,d,F,gs,k", [(3000, 512, 2048, 64, 6), (3000, 512, 2048, 128, 6),
                                        (24576, 2048, 5504, 128, 11)])
def test_inference_equals_training_forward(T, d, F, gs, k):
    require_gpu()
    note(f"inference vs training T={T} d={d} gs={gs}")
    inp = inputs(T, d, F, gs, "bf16", seed=42, bias=False)
    x, wg, wu, wd = (to_dev(inp[n]) for n in ("x", "wg", "wu", "wd"))
    idx = I.random_group_idx(T, F // gs, k, seed=42).to(DEV)
    y_train, _ = E.sparse_swiglu_fwd(x, wg, wu, wd, idx, gs)
    y_inf, _ = E.sparse_swiglu_fwd(x, wg, wu, wd, idx, gs, for_backward=False)
    torch.cuda.synchronize()
    assert torch.equal(y_train, y_inf)


def test_inference_prefill_1p3b_sampled():
    """The prefill bench shape (4096 tokens of the 1.3B layer, forward only):
    selection and forward each against the oracle, y on sampled tokens."""
    require_gpu()
    T, d, F, gs, k, spg = 4096, 2048, 5504, 128, 11, 16
    note("inference prefill 4096 x 1.3B")
    inp = inputs(T, d, F, gs, "bf16", seed=43, bias=True, spg=spg)
    y, _, oidx = _routed_forward(inp, k, spg)
    toks = np.sort(np.random.default_rng(5).choice(T, 256, replace=False))
    W = [f64(inp[n]) for n in ("wg", "wu", "wd")]
    assert_close("y", f64(y[toks]), O.swiglu_rows(f64(inp["x"][toks]), *W, oidx[toks], gs), "bf16")
