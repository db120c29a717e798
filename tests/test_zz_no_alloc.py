"""The allocation-free inference forward (esg_sparse_swiglu_fwd_noalloc),
called through the C ABI, against the inference forward with a caller
scratch (esg_sparse_swiglu_fwd, saved = NULL): two calls in a row on the
library's own scratch array, the second with fewer tokens (first
2048 tokens, then 64 on the split forward), each bitwise equal to the
existing entry point's y."""
import ctypes

import numpy as np
import pytest
import torch

import esg_inputs as I
import group_sparse_swiglu_amd as E
from gpu_common import DEV, f64, inputs, note, require_gpu, to_dev
from oracle import esg_oracle as O
from parity_util import assert_close

pytestmark = pytest.mark.gpu


def _noalloc(x, wg, wu, wd, idx, gs, y):
    T, d = x.shape
    F = wg.shape[0]
    st = E.lib().esg_sparse_swiglu_fwd_noalloc(
        x.data_ptr(), wg.data_ptr(), wu.data_ptr(), wd.data_ptr(), E.ESG_BF16, T, d, F, gs, idx.shape[1],
        idx.data_ptr(), y.data_ptr(), None, torch.cuda.current_stream().cuda_stream)
    assert st == 0, E.lib().esg_status_string(st)


def test_noalloc_forward_matches_the_scratch_forward_twice():
    require_gpu()
    d, F, gs, k = 2048, 5504, 128, 11
    for T, seed in ((2048, 31), (64, 32)):
        note(f"noalloc fwd T={T}")
        inp = inputs(T, d, F, gs, "bf16", seed=seed, bias=False)
        idx = I.random_group_idx(T, F // gs, k, seed=seed).to(DEV)
        x, wg, wu, wd = (to_dev(inp[n]) for n in ("x", "wg", "wu", "wd"))
        y_ref, _ = E.sparse_swiglu_fwd(x, wg, wu, wd, idx, gs, for_backward=False)
        y = torch.full_like(y_ref, float("nan"))
        _noalloc(x, wg, wu, wd, idx, gs, y)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), f"T={T}: noalloc y differs from the scratch forward"
        rows = np.arange(0, T, max(1, T // 64))
        W = [f64(inp[n]) for n in ("wg", "wu", "wd")]
        assert_close("y", f64(y[rows]), O.swiglu_rows(f64(inp["x"][rows]), *W, idx.cpu().numpy()[rows], gs),
                     "bf16")


def test_noalloc_rejects_a_batch_beyond_its_scratch():
    """2483 tokens at the 1.3B shape need more forward scratch than the
    library's array holds: the call returns ESG_ERR_WORKSPACE before any launch."""
    require_gpu()
    stub = torch.zeros(16, dtype=torch.int32, device=DEV)   # never read: the size check fails first
    p = stub.data_ptr()
    st = E.lib().esg_sparse_swiglu_fwd_noalloc(p, p, p, p, E.ESG_BF16, 2483, 2048, 5504, 128, 11, p, p, None,
                                               None)
    assert st == 3                     # ESG_ERR_WORKSPACE
    st = E.lib().esg_sparse_swiglu_fwd_noalloc(p, p, p, p, E.ESG_BF16, 2483, 2048, 5504, 128, 11, None, p, None,
                                               None)
    assert st == 1                     # idx = NULL is the dense limit, which needs k = G
