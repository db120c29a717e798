"""GPU parity: the FlashFFN multi-head sub-network core vs the oracle.
Bound: relative max-abs 2e-2 (bf16 inputs and output, fp32 accumulation, the
router-scaled intermediate rounded to bf16 before its product with V)."""
import numpy as np
import pytest
import torch

import esg_inputs as I
import group_sparse_swiglu_amd as E
from gpu_common import DEV, f64, note, require_gpu
from oracle import mhffn_oracle as M
from parity_util import assert_close

pytestmark = pytest.mark.gpu

CASES = [
    # name, tokens, heads, subnets, d_sub: chunk tails, token tails, single token
    ("tiny", 100, 2, 3, 96),
    ("ragged_d200", 300, 3, 2, 200),
    ("d8", 50, 1, 1, 8),
    ("one_token", 1, 2, 4, 192),
    ("e15_d384_two_heads", 1000, 2, 15, 384),
    ("e32_max", 130, 1, 32, 40),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_mhffn_forward_matches_oracle(case):
    require_gpu()
    name, T, H, Es, de = case
    note(f"mhffn {name}")
    q, r, k, u, v, _ = I.make_mhffn_inputs(T, H, 128, Es, de, seed=T + Es)
    o = E.mhffn_fwd(*(t.to(DEV) for t in (q, r, k, u, v)))
    torch.cuda.synchronize()
    ref = M.mhffn_forward(f64(q), f64(r), f64(k), f64(u), f64(v))
    print("  rel error:", f"{assert_close('O', f64(o), ref, 'bf16'):.2e}")


def test_mhffn_zero_router_and_zero_tokens():
    require_gpu()
    note("mhffn zero router / zero tokens")
    q, r, k, u, v, _ = I.make_mhffn_inputs(64, 2, 128, 3, 96, seed=1)
    o = E.mhffn_fwd(q.to(DEV), torch.zeros_like(r).to(DEV), k.to(DEV), u.to(DEV), v.to(DEV))
    assert torch.count_nonzero(o) == 0
    o0 = E.mhffn_fwd(q[:0].to(DEV), r[:0].to(DEV), k.to(DEV), u.to(DEV), v.to(DEV))
    assert o0.shape == (0, 2, 128)


def test_mhffn_deterministic():
    require_gpu()
    note("mhffn determinism")
    args = [t.to(DEV) for t in I.make_mhffn_inputs(777, 3, 128, 5, 200, seed=2)[:5]]
    assert torch.equal(E.mhffn_fwd(*args), E.mhffn_fwd(*args))


@pytest.mark.parametrize("wl", sorted(I.MHFFN_WORKLOADS))
def test_mhffn_workload_sampled(wl):
    """Bench size; every head of sampled tokens (a token's output depends on its own row)."""
    require_gpu()
    w = I.MHFFN_WORKLOADS[wl]
    note(f"mhffn workload {wl}")
    q, r, k, u, v, _ = I.make_mhffn_inputs(w.tokens, w.heads, w.d_head, w.subnets, w.d_sub, seed=0)
    o = E.mhffn_fwd(*(t.to(DEV) for t in (q, r, k, u, v)))
    torch.cuda.synchronize()
    toks = np.sort(np.random.default_rng(3).choice(w.tokens, 96, replace=False))
    ref = M.mhffn_forward(f64(q[toks]), f64(r[toks]), f64(k), f64(u), f64(v))
    assert_close("O", f64(o[toks]), ref, "bf16")


GRAD_CASES = [
    ("tiny", 100, 2, 3, 96),
    ("ragged_d200", 300, 3, 2, 200),
    ("d8", 50, 1, 1, 8),
    ("one_token", 1, 2, 4, 192),
    ("e15_d384", 700, 1, 15, 384),
    ("e32_max", 130, 1, 32, 40),
]


@pytest.mark.parametrize("case", GRAD_CASES, ids=[c[0] for c in GRAD_CASES])
def test_mhffn_backward_matches_oracle(case):
    require_gpu()
    name, T, H, Es, de = case
    note(f"mhffn bwd {name}")
    q, r, k, u, v, do = I.make_mhffn_inputs(T, H, 128, Es, de, seed=T + Es + 1)
    grads = E.mhffn_bwd(*(t.to(DEV) for t in (do, q, r, k, u, v)))
    torch.cuda.synchronize()
    ref = M.mhffn_backward(f64(do), f64(q), f64(r), f64(k), f64(u), f64(v))
    errs = {nm: assert_close(nm, f64(g), rr, "bf16") for nm, g, rr in zip(("dQ", "dR", "dK", "dU", "dV"), grads, ref)}
    print("  rel errors:", {k_: f"{v_:.2e}" for k_, v_ in errs.items()})


def test_mhffn_backward_deterministic_and_zero_tokens():
    require_gpu()
    note("mhffn bwd determinism / zero tokens")
    args = [t.to(DEV) for t in I.make_mhffn_inputs(500, 2, 128, 4, 144, seed=4)]
    q, r, k, u, v, do = args
    a = E.mhffn_bwd(do, q, r, k, u, v)
    b = E.mhffn_bwd(do, q, r, k, u, v)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    dq, dr, dk, du, dv = E.mhffn_bwd(do[:0], q[:0], r[:0], k, u, v)
    for t in (dk, du, dv):
        assert torch.count_nonzero(t) == 0


@pytest.mark.parametrize("wl", sorted(I.MHFFN_WORKLOADS))
def test_mhffn_backward_workload_sampled(wl):
    """Bench size: dQ, dR on sampled tokens (their rows depend on that token
    only), dK/dU/dV on sampled (head, sub-network) pairs over all tokens."""
    require_gpu()
    w = I.MHFFN_WORKLOADS[wl]
    note(f"mhffn bwd workload {wl}")
    q, r, k, u, v, do = I.make_mhffn_inputs(w.tokens, w.heads, w.d_head, w.subnets, w.d_sub, seed=0)
    dq, dr, dk, du, dv = E.mhffn_bwd(*(t.to(DEV) for t in (do, q, r, k, u, v)))
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    toks = np.sort(rng.choice(w.tokens, 64, replace=False))
    rq, rr, _, _, _ = M.mhffn_backward(f64(do[toks]), f64(q[toks]), f64(r[toks]), f64(k), f64(u), f64(v))
    assert_close("dQ", f64(dq[toks]), rq, "bf16")
    assert_close("dR", f64(dr[toks]), rr, "bf16")
    for h, e in ((0, 0), (7, 14), (15, 3)):
        sl = lambda t: t[:, h:h + 1]
        _, _, gk, gu, gv = M.mhffn_backward(f64(sl(do)), f64(sl(q)), f64(r[:, h:h + 1, e:e + 1]),
                                            f64(k[h:h + 1, e:e + 1]), f64(u[h:h + 1, e:e + 1]),
                                            f64(v[h:h + 1, e:e + 1]))
        assert_close(f"dK[{h},{e}]", f64(dk[h, e]), gk[0, 0], "bf16")
        assert_close(f"dU[{h},{e}]", f64(du[h, e]), gu[0, 0], "bf16")
        assert_close(f"dV[{h},{e}]", f64(dv[h, e]), gv[0, 0], "bf16")
