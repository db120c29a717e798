"""GPU parity at sizes past the 32-bit buffer limits.

* 65536 tokens at the 1.3B shape (k = 11 of 43 groups of 128): about 3 GB of
  bf16 partial rows per direction.  The tile kernels address each tile's
  partial rows from a per-tile base, so this size runs the same pipelined
  kernels as the benchmark shapes.
* 524288 tokens of width 2048: x, dy, y and dx are 2 GiB each, past what the
  pipelined kernels gather with 32-bit offsets, so the generic kernels run,
  with group blocks of 128 and of 64 neurons.

y and dx are checked on sampled tokens, dW on sampled neurons (eugen_sparse
README, "What it does": sparse_swiglu_ffn and its gradients), against the fp64
oracle given the same routing.  Bound: relative max-abs 2e-2 (bf16)."""
import numpy as np
import pytest
import torch

import esg_inputs as I
import group_sparse_swiglu_amd as E
from gpu_common import DEV, f64, inputs, note, require_gpu, to_dev
from oracle import esg_oracle as O
from parity_util import assert_close

pytestmark = pytest.mark.gpu


def test_partial_rows_beyond_2gib_run_the_tile_kernels():
    require_gpu()
    T, d, F, gs, k = 65536, 2048, 5504, 128, 11
    note(f"large T={T} 1.3B shape")
    inp = inputs(T, d, F, gs, "bf16", seed=41, bias=False)
    idx = I.random_group_idx(T, F // gs, k, seed=41).numpy()
    x, wg, wu, wd, dy = (to_dev(inp[n]) for n in ("x", "wg", "wu", "wd", "dy"))
    y, ctx = E.sparse_swiglu_fwd(x, wg, wu, wd, torch.as_tensor(idx).to(DEV), gs)
    dx, dwg, dwu, dwd = E.sparse_swiglu_bwd(dy, x, wg, wu, wd, ctx)
    torch.cuda.synchronize()
    rows = (T * k + (F // gs) * 127) // 128 * 128
    assert rows * d * 2 > 2 ** 31          # the partial rows of one direction exceed 2 GiB
    rng = np.random.default_rng(4)
    toks = np.sort(rng.choice(T, 128, replace=False))
    W = [f64(inp[n]) for n in ("wg", "wu", "wd")]
    xs, dys = f64(inp["x"][toks]), f64(inp["dy"][toks])
    assert_close("y", f64(y[toks]), O.swiglu_rows(xs, *W, idx[toks], gs), "bf16")
    assert_close("dx", f64(dx[toks]), O.dx_rows(dys, xs, *W, idx[toks], gs), "bf16")
    neu = np.sort(rng.choice(F, 12, replace=False))
    rg, ru, rd = O.dw_neuron_rows(neu, f64(inp["dy"]), f64(inp["x"]), *W, idx, gs)
    assert_close("dW_gate", f64(dwg[neu]), rg, "bf16")
    assert_close("dW_up", f64(dwu[neu]), ru, "bf16")
    assert_close("dW_down", f64(dwd[:, neu]), rd, "bf16")


@pytest.mark.parametrize("gs", [128, 64])
def test_inputs_of_2gib_run_the_generic_kernels(gs):
    """524288 tokens x 2048: every 512th token takes group 0 (1024 tokens),
    the others one of groups 1..G-1.  Inputs drawn on the GPU from a seeded
    generator (N(0,1) activations, N(0, 1/fan_in) weights), rows copied back
    for the oracle."""
    require_gpu()
    T, d, F, k = 524288, 2048, 2048, 1
    G = F // gs
    note(f"large T={T} d={d} gs={gs} (generic kernels)")
    gen = torch.Generator(device=DEV).manual_seed(43 + gs)
    x = torch.randn(T, d, generator=gen, device=DEV).to(torch.bfloat16)
    dy = torch.randn(T, d, generator=gen, device=DEV).to(torch.bfloat16)
    wg = (torch.randn(F, d, generator=gen, device=DEV) / d ** 0.5).to(torch.bfloat16)
    wu = (torch.randn(F, d, generator=gen, device=DEV) / d ** 0.5).to(torch.bfloat16)
    wd = (torch.randn(d, F, generator=gen, device=DEV) / F ** 0.5).to(torch.bfloat16)
    assert x.numel() * 2 >= 2 ** 31
    t = np.arange(T)
    idx = np.where(t % 512 == 0, 0, 1 + (t * 7919) % (G - 1)).astype(np.int32)[:, None]
    y, ctx = E.sparse_swiglu_fwd(x, wg, wu, wd, torch.as_tensor(idx).to(DEV), gs)
    dx, dwg, dwu, dwd = E.sparse_swiglu_bwd(dy, x, wg, wu, wd, ctx)
    torch.cuda.synchronize()
    W = [f64(w) for w in (wg, wu, wd)]
    rng = np.random.default_rng(6)
    toks = np.sort(np.concatenate([rng.choice(T, 48, replace=False), np.arange(0, T, 512)[:16]]))
    tt = torch.as_tensor(toks, device=DEV)
    xs, dys = f64(x[tt]), f64(dy[tt])
    assert_close("y", f64(y[tt]), O.swiglu_rows(xs, *W, idx[toks], gs), "bf16")
    assert_close("dx", f64(dx[tt]), O.dx_rows(dys, xs, *W, idx[toks], gs), "bf16")
    # group 0: its 1024 tokens hold every contribution to its weight gradients
    g0 = torch.as_tensor(np.flatnonzero(idx[:, 0] == 0), device=DEV)
    neu = np.array([0, 5, gs - 1])
    rg, ru, rd = O.dw_neuron_rows(neu, f64(dy[g0]), f64(x[g0]), *W, idx[g0.cpu().numpy()], gs)
    assert_close("dW_gate g0", f64(dwg[neu]), rg, "bf16")
    assert_close("dW_up g0", f64(dwu[neu]), ru, "bf16")
    assert_close("dW_down g0", f64(dwd[:, neu]), rd, "bf16")
