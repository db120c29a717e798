"""Pins for the LeakyReLU(0.5)-squared MLP oracle (CPU only)."""
import json
import os

import numpy as np
import torch

from oracle import mlp_oracle as M

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    with open(os.path.join(GOLDEN, "leaky_relu2_hand.json")) as f:
        return json.load(f)


def test_activation_hand_values():
    g = _golden()
    post, ag = M.activation(np.array(g["pre"]))
    assert post.tolist() == g["post"] and ag.tolist() == g["act_grad"]


def test_mlp_hand_case():
    c = _golden()["mlp_case"]
    y, post, ag = M.mlp_forward(c["x"], c["w_up"], c["w_down"])
    assert y.tolist() == c["y"]
    dx, dwu, dwd = M.mlp_backward(c["dy"], c["x"], c["w_up"], c["w_down"], post, ag)
    assert dx.tolist() == c["dx"] and dwu.tolist() == c["dw_up"] and dwd.tolist() == c["dw_down"]


def test_activation_is_leaky_relu_squared_and_its_derivative():
    pre = torch.linspace(-6, 6, 1001, dtype=torch.float64, requires_grad=True)
    ref = torch.nn.functional.leaky_relu(pre, 0.5).square()
    (grad,) = torch.autograd.grad(ref.sum(), pre)
    post, ag = M.activation(pre.detach().numpy())
    np.testing.assert_allclose(post, ref.detach().numpy(), rtol=1e-15, atol=0)
    np.testing.assert_allclose(ag, grad.numpy(), rtol=1e-15, atol=0)


def test_gradients_match_torch_autograd():
    g = torch.Generator().manual_seed(3)
    T, d, F = 37, 24, 56
    x = torch.randn(T, d, generator=g, dtype=torch.float64, requires_grad=True)
    wu = (torch.randn(F, d, generator=g, dtype=torch.float64) / d ** 0.5).requires_grad_(True)
    wd = (torch.randn(d, F, generator=g, dtype=torch.float64) / F ** 0.5).requires_grad_(True)
    dy = torch.randn(T, d, generator=g, dtype=torch.float64)
    y = torch.nn.functional.leaky_relu(x @ wu.T, 0.5).square() @ wd.T
    y.backward(dy)
    yo, post, ag = M.mlp_forward(x.detach().numpy(), wu.detach().numpy(), wd.detach().numpy())
    np.testing.assert_allclose(yo, y.detach().numpy(), rtol=1e-12, atol=1e-12)
    dx, dwu, dwd = M.mlp_backward(dy.numpy(), x.detach().numpy(), wu.detach().numpy(), wd.detach().numpy(), post, ag)
    for ours, ref in ((dx, x.grad), (dwu, wu.grad), (dwd, wd.grad)):
        np.testing.assert_allclose(ours, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_finite_differences():
    rng = np.random.default_rng(4)
    T, d, F = 9, 6, 10
    x, wu, wd, dy = (rng.standard_normal(s) for s in ((T, d), (F, d), (d, F), (T, d)))
    _, post, ag = M.mlp_forward(x, wu, wd)
    dx, dwu, dwd = M.mlp_backward(dy, x, wu, wd, post, ag)
    loss = lambda a, b, c: float((M.mlp_forward(a, b, c)[0] * dy).sum())
    h = 1e-6
    for arr, grad, which in ((x, dx, 0), (wu, dwu, 1), (wd, dwd, 2)):
        for _ in range(5):
            i = tuple(rng.integers(0, n) for n in arr.shape)
            p, m = [a.copy() for a in (x, wu, wd)], [a.copy() for a in (x, wu, wd)]
            p[which][i] += h
            m[which][i] -= h
            fd = (loss(*p) - loss(*m)) / (2 * h)
            assert abs(fd - grad[i]) <= 1e-6 * max(1.0, abs(fd))


def test_row_and_column_helpers_agree_with_full():
    rng = np.random.default_rng(5)
    T, d, F = 20, 8, 16
    x, wu, wd, dy = (rng.standard_normal(s) for s in ((T, d), (F, d), (d, F), (T, d)))
    y, post, ag = M.mlp_forward(x, wu, wd)
    dx, dwu, dwd = M.mlp_backward(dy, x, wu, wd, post, ag)
    rows = np.array([0, 7, 19])
    np.testing.assert_allclose(M.mlp_rows(x[rows], wu, wd), y[rows], rtol=1e-13)
    np.testing.assert_allclose(M.dx_rows(dy[rows], x[rows], wu, wd), dx[rows], rtol=1e-13)
    neu = np.array([1, 5, 15])
    cu, cd = M.dw_columns(neu, dy, x, wu, wd)
    np.testing.assert_allclose(cu, dwu[neu], rtol=1e-13)
    np.testing.assert_allclose(cd, dwd[:, neu], rtol=1e-13)
