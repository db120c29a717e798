"""The hot path captured as one HIP graph: every replay must reproduce the
eagerly launched step bit for bit (the kernels are deterministic), also with
other GPU work and synchronisations between the replays.  Covers the routed
path with selection and the bias update (also with the weight gradients on a
second caller stream, forked and joined inside the captured backward), and
the dense limit."""
import pytest
import torch

import group_sparse_swiglu_amd as E
from gpu_common import DEV, inputs, note, require_gpu, to_dev

pytestmark = pytest.mark.gpu


def _bufs(T, d, F, G, k, dtype):
    return dict(idx=torch.empty(T, k, dtype=torch.int32, device=DEV),
                cnt=torch.empty(G, dtype=torch.int32, device=DEV),
                y=torch.empty(T, d, dtype=dtype, device=DEV),
                grads=(torch.empty(T, d, dtype=dtype, device=DEV), torch.empty(F, d, dtype=dtype, device=DEV),
                       torch.empty(F, d, dtype=dtype, device=DEV), torch.empty(d, F, dtype=dtype, device=DEV)))


@pytest.mark.parametrize("dense,overlap", [(False, False), (False, True), (True, False)],
                         ids=["routed", "routed_aux_stream", "dense"])
def test_graph_replays_match_eager(dense, overlap):
    require_gpu()
    T, d, F, gs, k, spg = 2048, 256, 1024, 64, 4, 8
    note(f"graph replay {'dense' if dense else 'routed'} overlap={overlap}")
    aux = torch.cuda.Stream() if overlap else None
    inp = inputs(T, d, F, gs, "bf16", seed=31, bias=True, spg=spg)
    x, wg, wu, wd, dy = (to_dev(inp[n]) for n in ("x", "wg", "wu", "wd", "dy"))
    sub = to_dev(inp["sub"])
    G = F // gs
    bias0 = to_dev(inp["bias"])
    b = _bufs(T, d, F, G, G if dense else k, x.dtype)
    bias, ema = bias0.clone(), torch.full((G,), k / G, dtype=torch.float32, device=DEV)
    ws, saved = {}, [None]

    def step():
        if dense:
            _, ctx = E.sparse_swiglu_fwd(x, wg, wu, wd, None, gs, workspace=ws, out=b["y"], saved=saved[0])
        else:
            E.grouped_topk_select(x, wg, gs, k, sub, spg, bias, return_counts=True, out=b["idx"],
                                  counts_out=b["cnt"])
            _, ctx = E.sparse_swiglu_fwd(x, wg, wu, wd, b["idx"], gs, workspace=ws, out=b["y"], saved=saved[0])
        saved[0] = ctx.saved
        E.sparse_swiglu_bwd(dy, x, wg, wu, wd, ctx, workspace=ws, outs=b["grads"], aux_stream=aux)
        if not dense:
            E.update_load_balance_bias_from_counts(bias, ema, b["cnt"], T, k / G, 1e-3, 0.5, 0.99)

    def snapshot():
        torch.cuda.synchronize()
        routing = () if dense else (b["idx"], b["cnt"], bias, ema)
        return [t.clone() for t in (*routing, b["y"], *b["grads"])]

    # eager reference sequence of three steps from the initial state
    step()
    torch.cuda.synchronize()
    bias.copy_(bias0), ema.fill_(k / G)
    ref = []
    for _ in range(3):
        step()
        ref.append(snapshot())

    # capture (after a warm-up on a side stream), then replay from the same initial state
    bias.copy_(bias0), ema.fill_(k / G)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    bias.copy_(bias0), ema.fill_(k / G)
    junk = torch.randn(1 << 20, device=DEV)
    for i in range(3):
        for t in (b["y"], *b["grads"]):   # poison the outputs: every replay must rewrite them
            t.fill_(float("nan"))
        b["idx"].fill_(-7)
        b["cnt"].fill_(-7)
        junk.mul_(1.0001).sum().item()   # unrelated eager work and a host synchronisation
        g.replay()
        got = snapshot()
        for j, (u, v) in enumerate(zip(got, ref[i])):
            assert torch.equal(u, v), f"replay {i}: tensor {j} differs from the eager step"
