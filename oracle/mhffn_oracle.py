"""CPU oracle for the multi-head sub-network FFN core of FlashFFN.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or run
this module: only the tests and the benchmark's CPU-baseline leg use it.  It
shares no code with the HIP library.

Written from the FlashFFN README ("FlashFFN: Multi-Head Decomposition Enables
I/O-Aware Feed-Forward Networks"), section "Overview", which defines, per head
h with width d_h and E dense sub-networks,

    O_h = sum_e R_e * ((SiLU(Q_h K_e^T) (*) (Q_h U_e^T)) V_e)

with Q_h the head's (RMS-normalised) input projection and R_e the router
weights, and from its "Model configurations" table (1.3B: d_model 2048,
16 heads of d_h = 128, E = 15, intermediate size 5760).

Readings taken (the page gives the formula only):

* F1 the fused core takes Q [T, H, d_h] and R [T, H, E] as inputs; the
  projection, the per-head RMS normalisation and the router that produce them
  (the page's prologue) are outside it, as is the output projection;
* F2 every head has its own sub-networks: K, U, V are [H, E, d_e, d_h]
  (K_e, U_e map d_h to d_e; V_e maps d_e back to d_h); the table's
  intermediate size is E * d_e per head (5760 = 15 * 384), which matches the
  SwiGLU parameter count of the same table (16 * 3 * 5760 * 128 = 35.4 M vs
  3 * 2048 * 5504 = 33.8 M per layer);
* F3 R scales the sub-network's output for that token (a scalar per token,
  head and sub-network); the gradient reaches R as well.

Everything is evaluated in float64 on the exact stored values.  Pinned by
``tests/test_oracle_mhffn.py`` (torch autograd of the fp64 formula, the
E = 1 case against a plain SwiGLU written with torch.nn.functional.silu,
finite differences, and invariants).
"""
from __future__ import annotations

import numpy as np


def _silu(z):
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def _sigmoid(z):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def mhffn_forward(q, r, k, u, v):
    """O [T, H, d_h] for q [T, H, d_h], r [T, H, E], k, u, v [H, E, d_e, d_h]."""
    q = np.asarray(q, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    k, u, v = (np.asarray(a, dtype=np.float64) for a in (k, u, v))
    T, H, dh = q.shape
    E = k.shape[1]
    out = np.zeros((T, H, dh))
    for h in range(H):
        for e in range(E):
            h1 = q[:, h] @ k[h, e].T          # [T, d_e]
            h2 = q[:, h] @ u[h, e].T
            a = _silu(h1) * h2
            out[:, h] += r[:, h, e:e + 1] * (a @ v[h, e])
    return out


def mhffn_backward(do, q, r, k, u, v):
    """(dQ, dR, dK, dU, dV) given the upstream gradient dO [T, H, d_h]."""
    do = np.asarray(do, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    k, u, v = (np.asarray(a, dtype=np.float64) for a in (k, u, v))
    T, H, dh = q.shape
    E = k.shape[1]
    dq = np.zeros_like(q)
    dr = np.zeros_like(r)
    dk, du, dv = np.zeros_like(k), np.zeros_like(u), np.zeros_like(v)
    for h in range(H):
        for e in range(E):
            h1 = q[:, h] @ k[h, e].T
            h2 = q[:, h] @ u[h, e].T
            s = _sigmoid(h1)
            a = h1 * s * h2
            g = do[:, h] @ v[h, e].T             # dL/d(a V) pulled back through V
            dr[:, h, e] = np.sum(a * g, axis=1)
            da = r[:, h, e:e + 1] * g
            dh2 = da * h1 * s
            dh1 = da * h2 * s * (1.0 + h1 * (1.0 - s))
            dq[:, h] += dh1 @ k[h, e] + dh2 @ u[h, e]
            dk[h, e] = dh1.T @ q[:, h]
            du[h, e] = dh2.T @ q[:, h]
            dv[h, e] = (r[:, h, e:e + 1] * a).T @ do[:, h]
    return dq, dr, dk, du, dv
