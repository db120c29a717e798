"""Pins for the oracle's dense-masked sparse SwiGLU forward and backward."""
import numpy as np
import pytest
import torch

from oracle import esg_oracle as O



@pytest.fixture(autouse=True)
def _fp64_default():
    """This module's torch pins run in fp64; the default is restored after each
    test so that no other module sees it."""
    old = torch.get_default_dtype()
    torch.set_default_dtype(torch.float64)
    yield
    torch.set_default_dtype(old)


def _rand(T, d, F, seed=0):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(T, d, generator=g)
    wg = torch.randn(F, d, generator=g) / d ** 0.5
    wu = torch.randn(F, d, generator=g) / d ** 0.5
    wd = torch.randn(d, F, generator=g) / F ** 0.5
    dy = torch.randn(T, d, generator=g)
    return x, wg, wu, wd, dy


def _torch_dense_swiglu(x, wg, wu, wd):
    """Textbook dense SwiGLU with torch library routines."""
    return torch.nn.functional.linear(
        torch.nn.functional.silu(torch.nn.functional.linear(x, wg)) * torch.nn.functional.linear(x, wu), wd)


def test_all_groups_active_is_dense_swiglu_and_autograd():
    """k = G (and idx = None) equals a textbook fp64 SwiGLU; the gradients
    equal torch.autograd of that graph."""
    T, d, F, gs = 19, 24, 64, 16
    x, wg, wu, wd, dy = _rand(T, d, F)
    params = [t.clone().requires_grad_(True) for t in (x, wg, wu, wd)]
    y_ref = _torch_dense_swiglu(*params)
    y_ref.backward(dy)
    G = F // gs
    idx_all = np.tile(np.arange(G), (T, 1))
    for idx in (None, idx_all):
        y = O.sparse_swiglu_forward(x.numpy(), wg.numpy(), wu.numpy(), wd.numpy(), idx, gs)
        np.testing.assert_allclose(y, y_ref.detach().numpy(), rtol=1e-12, atol=1e-12)
        grads = O.sparse_swiglu_backward(dy.numpy(), x.numpy(), wg.numpy(), wu.numpy(), wd.numpy(), idx, gs)
        for got, p in zip(grads, params):
            np.testing.assert_allclose(got, p.grad.numpy(), rtol=1e-11, atol=1e-12)


def _gathered_reference(x, wg, wu, wd, idx, gs):
    """Per token, sum over its listed groups of the group's own SwiGLU,
    computed with torch on gathered weight slices (a different formulation
    from the oracle's mask)."""
    rows = []
    for t in range(x.shape[0]):
        acc = torch.zeros(wd.shape[0])
        for g in idx[t]:
            sl = slice(int(g) * gs, (int(g) + 1) * gs)
            h = torch.nn.functional.silu(wg[sl] @ x[t]) * (wu[sl] @ x[t])
            acc = acc + wd[:, sl] @ h
        rows.append(acc)
    return torch.stack(rows)


@pytest.mark.parametrize("k", [1, 3, 5])
def test_forward_matches_per_group_gather(k):
    T, d, F, gs = 23, 16, 96, 16
    x, wg, wu, wd, _ = _rand(T, d, F, seed=k)
    rng = np.random.default_rng(k)
    idx = np.sort(np.stack([rng.choice(F // gs, k, replace=False) for _ in range(T)]), axis=1)
    y = O.sparse_swiglu_forward(x.numpy(), wg.numpy(), wu.numpy(), wd.numpy(), idx, gs)
    ref = _gathered_reference(x, wg, wu, wd, idx, gs)
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-13)


def test_backward_matches_autograd_of_gathered_form():
    T, d, F, gs, k = 11, 16, 64, 16, 2
    x, wg, wu, wd, dy = _rand(T, d, F, seed=9)
    rng = np.random.default_rng(9)
    idx = np.sort(np.stack([rng.choice(F // gs, k, replace=False) for _ in range(T)]), axis=1)
    params = [t.clone().requires_grad_(True) for t in (x, wg, wu, wd)]
    _gathered_reference(*params, idx, gs).backward(dy)
    grads = O.sparse_swiglu_backward(dy.numpy(), x.numpy(), wg.numpy(), wu.numpy(), wd.numpy(), idx, gs)
    for got, p in zip(grads, params):
        np.testing.assert_allclose(got, p.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_finite_differences():
    """Central differences of L = sum(y * dy) with the routing held fixed."""
    T, d, F, gs, k = 7, 8, 48, 16, 2
    x, wg, wu, wd, dy = [t.numpy() for t in _rand(T, d, F, seed=4)]
    rng = np.random.default_rng(4)
    idx = np.sort(np.stack([rng.choice(F // gs, k, replace=False) for _ in range(T)]), axis=1)
    grads = O.sparse_swiglu_backward(dy, x, wg, wu, wd, idx, gs)

    def loss(xx, a, b, c):
        return float((O.sparse_swiglu_forward(xx, a, b, c, idx, gs) * dy).sum())

    h = 1e-6
    args = [x, wg, wu, wd]
    for which in range(4):
        for _ in range(6):
            pos = tuple(rng.integers(0, s) for s in args[which].shape)
            plus = [a.copy() for a in args]
            minus = [a.copy() for a in args]
            plus[which][pos] += h
            minus[which][pos] -= h
            fd = (loss(*plus) - loss(*minus)) / (2 * h)
            assert abs(fd - grads[which][pos]) <= 1e-7 * max(1.0, abs(fd)), (which, pos)


def test_unselected_groups_get_exact_zero_and_no_influence():
    T, d, F, gs = 30, 16, 128, 16
    x, wg, wu, wd, dy = [t.numpy() for t in _rand(T, d, F, seed=2)]
    rng = np.random.default_rng(2)
    idx = np.sort(np.stack([rng.choice([0, 2, 5], 2, replace=False) for _ in range(T)]), axis=1)
    y = O.sparse_swiglu_forward(x, wg, wu, wd, idx, gs)
    dx, dwg, dwu, dwd = O.sparse_swiglu_backward(dy, x, wg, wu, wd, idx, gs)
    unused = [g for g in range(F // gs) if g not in (0, 2, 5)]
    for g in unused:
        sl = slice(g * gs, (g + 1) * gs)
        assert np.all(dwg[sl] == 0) and np.all(dwu[sl] == 0) and np.all(dwd[:, sl] == 0)
        # perturbing the unused group's weights changes nothing, bit for bit
        wg2, wu2, wd2 = wg.copy(), wu.copy(), wd.copy()
        wg2[sl] += 1.0
        wu2[sl] -= 2.0
        wd2[:, sl] *= 3.0
        assert np.array_equal(O.sparse_swiglu_forward(x, wg2, wu2, wd2, idx, gs), y)
        assert np.array_equal(O.sparse_swiglu_backward(dy, x, wg2, wu2, wd2, idx, gs)[0], dx)


def test_token_permutation_invariance():
    T, d, F, gs, k = 40, 16, 96, 16, 3
    x, wg, wu, wd, dy = [t.numpy() for t in _rand(T, d, F, seed=8)]
    rng = np.random.default_rng(8)
    idx = np.sort(np.stack([rng.choice(F // gs, k, replace=False) for _ in range(T)]), axis=1)
    p = rng.permutation(T)
    y = O.sparse_swiglu_forward(x, wg, wu, wd, idx, gs)
    y2 = O.sparse_swiglu_forward(x[p], wg, wu, wd, idx[p], gs)
    np.testing.assert_allclose(y2, y[p], rtol=1e-13, atol=1e-14)
    g1 = O.sparse_swiglu_backward(dy, x, wg, wu, wd, idx, gs)
    g2 = O.sparse_swiglu_backward(dy[p], x[p], wg, wu, wd, idx[p], gs)
    np.testing.assert_allclose(g2[0], g1[0][p], rtol=1e-13, atol=1e-14)
    for a, b in zip(g1[1:], g2[1:]):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


def test_chunking_does_not_change_results():
    T, d, F, gs, k = 50, 16, 64, 16, 2
    x, wg, wu, wd, dy = [t.numpy() for t in _rand(T, d, F, seed=12)]
    rng = np.random.default_rng(12)
    idx = np.sort(np.stack([rng.choice(F // gs, k, replace=False) for _ in range(T)]), axis=1)
    a = O.sparse_swiglu_backward(dy, x, wg, wu, wd, idx, gs, chunk=7)
    b = O.sparse_swiglu_backward(dy, x, wg, wu, wd, idx, gs, chunk=4096)
    for u, v in zip(a, b):
        np.testing.assert_allclose(u, v, rtol=1e-12, atol=1e-13)


def test_scalar_closed_form():
    """d=1, two single-neuron groups, token routed to group 0 only:
    y = SiLU(x wg0) (x wu0) wd0, and the gradients by the chain rule with
    SiLU' taken from torch autograd of torch's SiLU."""
    x, wg, wu, wd, dy = 2.0, [1.0, -1.0], [3.0, 1.0], [0.5, 2.0], 1.0
    z = torch.tensor(x * wg[0], requires_grad=True)
    s = torch.nn.functional.silu(z)
    s.backward()
    silu2, dsilu2 = float(s.detach()), float(z.grad)
    idx = np.array([[0]])
    y = O.sparse_swiglu_forward(np.array([[x]]), np.array([[v] for v in wg]), np.array([[v] for v in wu]),
                                np.array([wd]), idx, 1)
    assert y[0, 0] == pytest.approx(silu2 * (x * wu[0]) * wd[0], rel=1e-14)
    dx, dwg, dwu, dwd = O.sparse_swiglu_backward(np.array([[dy]]), np.array([[x]]),
                                                 np.array([[v] for v in wg]), np.array([[v] for v in wu]),
                                                 np.array([wd]), idx, 1)
    da = dy * wd[0]
    assert dx[0, 0] == pytest.approx(da * (x * wu[0]) * dsilu2 * wg[0] + da * silu2 * wu[0], rel=1e-13)
    assert dwg[:, 0].tolist() == pytest.approx([da * (x * wu[0]) * dsilu2 * x, 0.0], rel=1e-13)
    assert dwu[:, 0].tolist() == pytest.approx([da * silu2 * x, 0.0], rel=1e-13)
    assert dwd[0].tolist() == pytest.approx([dy * silu2 * x * wu[0], 0.0], rel=1e-13)


def test_sampled_helpers_match_full():
    T, d, F, gs, k = 33, 16, 96, 16, 2
    x, wg, wu, wd, dy = [t.numpy() for t in _rand(T, d, F, seed=21)]
    rng = np.random.default_rng(21)
    idx = np.sort(np.stack([rng.choice(F // gs, k, replace=False) for _ in range(T)]), axis=1)
    y = O.sparse_swiglu_forward(x, wg, wu, wd, idx, gs)
    dx, dwg, dwu, dwd = O.sparse_swiglu_backward(dy, x, wg, wu, wd, idx, gs)
    rows = np.array([0, 5, 32])
    np.testing.assert_allclose(O.swiglu_rows(x[rows], wg, wu, wd, idx[rows], gs), y[rows], rtol=1e-13)
    np.testing.assert_allclose(O.dx_rows(dy[rows], x[rows], wg, wu, wd, idx[rows], gs), dx[rows], rtol=1e-13)
    neu = np.array([0, 17, 95])
    a, b, c = O.dw_neuron_rows(neu, dy, x, wg, wu, wd, idx, gs, chunk=10)
    np.testing.assert_allclose(a, dwg[neu], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(b, dwu[neu], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(c, dwd[:, neu], rtol=1e-12, atol=1e-14)
    a, b, c = O.dw_neuron_rows(neu, dy, x, wg, wu, wd, None, gs)
    full = O.sparse_swiglu_backward(dy, x, wg, wu, wd, None, gs)
    np.testing.assert_allclose(c, full[3][:, neu], rtol=1e-12, atol=1e-14)


def test_routing_preconditions():
    x, wg, wu, wd, _ = [t.numpy() for t in _rand(4, 8, 32)]
    with pytest.raises(ValueError):
        O.sparse_swiglu_forward(x, wg, wu, wd, np.array([[0, 0]] * 4), 16)
    with pytest.raises(ValueError):
        O.sparse_swiglu_forward(x, wg, wu, wd, np.array([[0, 2]] * 4), 16)
