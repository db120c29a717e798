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
