"""CPU oracle for the LeakyReLU(0.5)-squared MLP with a stored activation
gradient.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or run
this module: only the tests and the benchmark's CPU-baseline leg use it.  It
shares no code with the HIP library.

Written from the parameter-golf pull request 1105 page, section "1. Fused MLP
Kernels: Triton TMA Forward + CUTLASS EVT Backward" (and its architecture
table A.7: d_model 512, MLP width 3.5x = 1792, LeakyReLU(0.5) squared).  The
page defines, for pre = x . W_up^T:

* act_grad = 2*pre where pre > 0, else 0.5*pre -- the derivative of the
  activation, computed once in the forward and stored;
* post = 0.5 * act_grad * pre, which equals LeakyReLU(0.5)(pre)^2 on both
  sides of zero (pre^2 above, (0.5*pre)^2 below);
* y = post . W_down^T;
* in the backward, dpre = (dy . W_down) * act_grad (the GEMM with the product
  in its epilogue), and then the plain gradients dW_down = dy^T . post,
  dW_up = dpre^T . x, dx = dpre . W_up.

Weights use nn.Linear layout: W_up [d_ff, d_model], W_down [d_model, d_ff].
Everything is evaluated in float64 on the exact stored values.  Pinned by
``tests/test_oracle_mlp.py`` (torch's leaky_relu and autograd, hand values,
finite differences).
"""
from __future__ import annotations

import numpy as np


def activation(pre):
    """(post, act_grad) of the pre-activation, float64."""
    pre = np.asarray(pre, dtype=np.float64)
    act_grad = np.where(pre > 0, 2.0 * pre, 0.5 * pre)
    post = 0.5 * act_grad * pre
    return post, act_grad


def mlp_forward(x, w_up, w_down):
    """y [T, d_model], and the saved (post, act_grad) [T, d_ff]."""
    x = np.asarray(x, dtype=np.float64)
    pre = x @ np.asarray(w_up, dtype=np.float64).T
    post, act_grad = activation(pre)
    y = post @ np.asarray(w_down, dtype=np.float64).T
    return y, post, act_grad


def mlp_backward(dy, x, w_up, w_down, post, act_grad):
    """(dx, dW_up, dW_down) from the upstream gradient and the saved tensors."""
    dy = np.asarray(dy, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    w_up = np.asarray(w_up, dtype=np.float64)
    w_down = np.asarray(w_down, dtype=np.float64)
    dpre = (dy @ w_down) * np.asarray(act_grad, dtype=np.float64)
    dw_down = dy.T @ np.asarray(post, dtype=np.float64)
    dw_up = dpre.T @ x
    dx = dpre @ w_up
    return dx, dw_up, dw_down


def mlp_rows(x_rows, w_up, w_down):
    """y for a subset of tokens (each token's output depends on its row only)."""
    return mlp_forward(x_rows, w_up, w_down)[0]


def dx_rows(dy_rows, x_rows, w_up, w_down):
    """dx for a subset of tokens."""
    _, post, act_grad = mlp_forward(x_rows, w_up, w_down)
    return mlp_backward(dy_rows, x_rows, w_up, w_down, post, act_grad)[0]


def dw_columns(neurons, dy, x, w_up, w_down):
    """Rows `neurons` of dW_up and the same columns of dW_down, over all
    tokens (each neuron's weight gradient needs only that neuron's
    activations)."""
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    w_up = np.asarray(w_up, dtype=np.float64)
    w_down = np.asarray(w_down, dtype=np.float64)
    pre = x @ w_up[neurons].T
    post, act_grad = activation(pre)
    dpre = (dy @ w_down[:, neurons]) * act_grad
    return dpre.T @ x, dy.T @ post
