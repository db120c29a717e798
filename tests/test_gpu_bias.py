"""GPU parity: the load-balance bias update is bit-exact with the oracle
taken in float32 (the sign decision is made in the kernel's precision)."""
import numpy as np
import pytest
import torch

import group_sparse_swiglu_amd as E
from gpu_common import DEV, note, require_gpu
from oracle import esg_oracle as O

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("G,steps", [(32, 1), (43, 50), (1024, 7), (3, 600)])
def test_bias_update_bit_exact(G, steps):
    require_gpu()
    note(f"bias G={G} steps={steps}")
    rng = np.random.default_rng(G)
    bias = rng.uniform(-0.1, 0.1, G).astype(np.float32)
    ema = np.full(G, 0.25, dtype=np.float32)
    b_d, e_d = torch.from_numpy(bias.copy()).to(DEV), torch.from_numpy(ema.copy()).to(DEV)
    for s in range(steps):
        cur = rng.dirichlet(np.ones(G)).astype(np.float32) * np.float32(G * 0.25)
        if s % 5 == 0:
            cur[: G // 2] = ema[: G // 2]      # exercise sign(0) where ema is unchanged
        E.update_load_balance_bias(b_d, e_d, torch.from_numpy(cur).to(DEV), 0.25, 1e-3, 0.5, 0.99)
        bias, ema = O.update_load_balance_bias(bias, ema, cur, 0.25, 1e-3, 0.5, 0.99, np.float32)
    torch.cuda.synchronize()
    assert np.array_equal(b_d.cpu().numpy(), bias)
    assert np.array_equal(e_d.cpu().numpy(), ema)


def test_bias_update_from_counts_bit_exact():
    require_gpu()
    note("bias from counts")
    G, T, k = 32, 8192, 8
    rng = np.random.default_rng(0)
    counts = rng.multinomial(T * k, np.ones(G) / G).astype(np.int32)
    bias = rng.uniform(-0.1, 0.1, G).astype(np.float32)
    ema = np.full(G, k / G, dtype=np.float32)
    b_d, e_d = torch.from_numpy(bias.copy()).to(DEV), torch.from_numpy(ema.copy()).to(DEV)
    E.update_load_balance_bias_from_counts(b_d, e_d, torch.from_numpy(counts).to(DEV), T, k / G, 1e-3, 0.5, 0.99)
    cur = O.frequency_from_counts(counts, T, np.float32)
    bias, ema = O.update_load_balance_bias(bias, ema, cur, np.float32(k / G), 1e-3, 0.5, 0.99, np.float32)
    torch.cuda.synchronize()
    assert np.array_equal(b_d.cpu().numpy(), bias)
    assert np.array_equal(e_d.cpu().numpy(), ema)


@pytest.mark.parametrize("T,d,F,gs,k", [(8192, 768, 2048, 64, 8), (333, 96, 640, 64, 3), (64, 2048, 5504, 128, 11)])
def test_bias_update_from_routing_equals_from_counts(T, d, F, gs, k):
    """The bias update from a training forward's saved routing reproduces the
    update from the selection's counts bit for bit."""
    require_gpu()
    note(f"bias from routing T={T} G={F // gs} k={k}")
    from gpu_common import inputs, to_dev
    inp = inputs(T, d, F, gs, "bf16", seed=9, bias=True, spg=min(8, gs))
    x, wg, wu, wd = (to_dev(inp[n]) for n in ("x", "wg", "wu", "wd"))
    idx, counts = E.grouped_topk_select(x, wg, gs, k, to_dev(inp["sub"]), inp["spg"], to_dev(inp["bias"]),
                                        return_counts=True)
    _, ctx = E.sparse_swiglu_fwd(x, wg, wu, wd, idx, gs)
    G = F // gs
    rng = np.random.default_rng(T)
    bias0 = torch.from_numpy(rng.uniform(-0.1, 0.1, G).astype(np.float32))
    ema0 = torch.from_numpy(rng.uniform(0.0, 2.0 * k / G, G).astype(np.float32))
    b1, e1 = bias0.to(DEV), ema0.to(DEV)
    b2, e2 = bias0.to(DEV), ema0.to(DEV)
    E.update_load_balance_bias_from_counts(b1, e1, counts, T, k / G, 1e-3, 0.5, 0.99)
    E.update_load_balance_bias_from_routing(b2, e2, ctx, k / G, 1e-3, 0.5, 0.99)
    torch.cuda.synchronize()
    assert torch.equal(b1, b2) and torch.equal(e1, e2)
