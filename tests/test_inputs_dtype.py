"""The seeded input generators fix their dtypes themselves: a test module that
changes torch's default dtype must not change what the generators return."""
import torch

import esg_inputs as I


def test_generators_ignore_the_default_dtype():
    old = torch.get_default_dtype()
    try:
        for default in (torch.float32, torch.float64):
            torch.set_default_dtype(default)
            logits, bias = I.make_routing_inputs(8, 16, seed=1)
            assert logits.dtype == bias.dtype == torch.float32
            q, r, k, u, v, do = I.make_mhffn_inputs(8, 2, 128, 3, 16, seed=1)
            assert r.dtype == torch.float32
            assert all(t.dtype == torch.bfloat16 for t in (q, k, u, v, do))
            assert all(t.dtype == torch.bfloat16 for t in I.make_mlp_inputs(8, 16, 24, seed=1))
            xs = I.make_routing_inputs(8, 16, seed=1, levels=4, saturate=True)
            assert all(t.dtype == torch.float32 for t in xs)
    finally:
        torch.set_default_dtype(old)
