"""Shared plumbing for the GPU parity tests (inputs to the device, oracle
inputs in fp64).  No arithmetic of the layer lives here."""
from __future__ import annotations

import sys

import numpy as np
import torch

import esg_inputs as I
import group_sparse_swiglu_amd as E

DEV = "cuda"


def note(msg: str) -> None:
    """Name the case on stdout before GPU work, flushed."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need an MI355X; none is visible")
    E.lib()


def inputs(T, d, F, gs, dtype, seed=0, bias=True, spg=None):
    x, wg, wu, wd, dy, b = I.make_inputs(T, d, F, gs, dtype, seed, bias)
    sub = E.make_subsample_index(F, gs, spg, seed)[0] if spg is not None else None
    return dict(x=x, wg=wg, wu=wu, wd=wd, dy=dy, bias=b, sub=sub, spg=spg, gs=gs, dtype=dtype)


def to_dev(t):
    return None if t is None else t.to(DEV)
