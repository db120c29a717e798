"""GPU parity: the LeakyReLU(0.5)^2 MLP with a stored activation gradient vs
the oracle.  Bound: relative max-abs 2e-2 (bf16 inputs and outputs, fp32
accumulation, post / act_grad / dpre rounded to bf16 between products)."""
import numpy as np
import pytest
import torch

import esg_inputs as I
import group_sparse_swiglu_amd as E
from gpu_common import DEV, f64, note, require_gpu
from oracle import mlp_oracle as M
from parity_util import assert_close

pytestmark = pytest.mark.gpu


def _run(x, wu, wd, dy, ws=None):
    X, WU, WD, DY = (t.to(DEV) for t in (x, wu, wd, dy))
    y, saved = E.leaky_mlp_fwd(X, WU, WD)
    dx, dwu, dwd = E.leaky_mlp_bwd(DY, X, WU, WD, saved, workspace=ws)
    torch.cuda.synchronize()
    post, act = E.leaky_mlp_saved_views(saved, x.shape[0], wu.shape[0])
    return y, dx, dwu, dwd, post, act


CASES = [
    # name, tokens, d_model, d_ff: tails in every dimension, then the page's widths
    ("tiny", 100, 64, 128),
    ("ragged", 1000, 136, 456),
    ("one_token", 1, 512, 1792),
    ("d512_f1792_t3000", 3000, 512, 1792),
    ("wide_d", 700, 1032, 264),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_mlp_matches_oracle(case):
    require_gpu()
    name, T, d, F = case
    note(f"mlp {name}")
    x, wu, wd, dy = I.make_mlp_inputs(T, d, F, seed=T + d)
    y, dx, dwu, dwd, post, act = _run(x, wu, wd, dy)
    ry, rpost, ract = M.mlp_forward(f64(x), f64(wu), f64(wd))
    rdx, rdwu, rdwd = M.mlp_backward(f64(dy), f64(x), f64(wu), f64(wd), rpost, ract)
    errs = {}
    for nm, g, r in (("y", y, ry), ("post", post, rpost), ("act_grad", act, ract), ("dx", dx, rdx),
                     ("dW_up", dwu, rdwu), ("dW_down", dwd, rdwd)):
        errs[nm] = assert_close(nm, f64(g), r, "bf16")
    print("  rel errors:", {k: f"{v:.2e}" for k, v in errs.items()})


def test_mlp_activation_signs_exact():
    """post and act_grad follow the sign rule of the stored gradient: a
    positive pre gives act_grad = 2 pre and post = pre^2, a negative one
    act_grad = pre / 2 and post = pre^2 / 4 (checked against the bf16 act_grad
    the kernel itself stored)."""
    require_gpu()
    note("mlp activation signs")
    x, wu, wd, dy = I.make_mlp_inputs(256, 64, 256, seed=7)
    _, _, _, _, post, act = _run(x, wu, wd, dy)
    _, rpost, ract = M.mlp_forward(f64(x), f64(wu), f64(wd))
    a, p = f64(act), f64(post)
    assert np.array_equal(np.sign(a), np.sign(np.where(np.abs(ract) < 1e-3, a, ract)))
    assert (p >= 0).all()


def test_mlp_deterministic_and_zero_tokens():
    require_gpu()
    note("mlp determinism")
    x, wu, wd, dy = I.make_mlp_inputs(5000, 512, 1792, seed=3)
    a = _run(x, wu, wd, dy)
    b = _run(x, wu, wd, dy)
    for u, v in zip(a, b):
        assert torch.equal(u, v)
    note("mlp zero tokens")
    x0 = torch.zeros(0, 512, dtype=torch.bfloat16)
    y, dx, dwu, dwd, _, _ = _run(x0, wu, wd, x0)
    assert y.shape == (0, 512) and dx.shape == (0, 512)
    assert torch.count_nonzero(dwu) == 0 and torch.count_nonzero(dwd) == 0


@pytest.mark.parametrize("wl", sorted(I.MLP_WORKLOADS))
def test_mlp_workload_sampled(wl):
    """Full bench size; y and dx on sampled tokens, dW on sampled neurons."""
    require_gpu()
    w = I.MLP_WORKLOADS[wl]
    note(f"mlp workload {wl}")
    x, wu, wd, dy = I.make_mlp_inputs(w.tokens, w.d_model, w.d_ff, seed=0)
    y, dx, dwu, dwd, _, _ = _run(x, wu, wd, dy)
    rng = np.random.default_rng(1)
    toks = np.sort(rng.choice(w.tokens, 128, replace=False))
    W = (f64(wu), f64(wd))
    assert_close("y", f64(y[toks]), M.mlp_rows(f64(x[toks]), *W), "bf16")
    assert_close("dx", f64(dx[toks]), M.dx_rows(f64(dy[toks]), f64(x[toks]), *W), "bf16")
    neu = np.sort(rng.choice(w.d_ff, 16, replace=False))
    ru, rd = M.dw_columns(neu, f64(dy), f64(x), *W)
    assert_close("dW_up", f64(dwu[neu]), ru, "bf16")
    assert_close("dW_down", f64(dwd[:, neu]), rd, "bf16")
