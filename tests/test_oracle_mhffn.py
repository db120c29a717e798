"""Pins for the FlashFFN multi-head sub-network core oracle (CPU only)."""
import numpy as np
import torch

from oracle import mhffn_oracle as M


def _inputs(T, H, dh, E, de, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(T, H, dh, generator=g, dtype=torch.float64)
    r = torch.rand(T, H, E, generator=g, dtype=torch.float64)
    k = torch.randn(H, E, de, dh, generator=g, dtype=torch.float64) / dh ** 0.5
    u = torch.randn(H, E, de, dh, generator=g, dtype=torch.float64) / dh ** 0.5
    v = torch.randn(H, E, de, dh, generator=g, dtype=torch.float64) / de ** 0.5
    do = torch.randn(T, H, dh, generator=g, dtype=torch.float64)
    return q, r, k, u, v, do


def _torch_core(q, r, k, u, v):
    """The page's formula written with torch einsum over heads and sub-networks."""
    h1 = torch.einsum("thd,hefd->thef", q, k)
    h2 = torch.einsum("thd,hefd->thef", q, u)
    a = torch.nn.functional.silu(h1) * h2
    return torch.einsum("thef,the,hefd->thd", a, r, v)


def test_forward_and_gradients_match_torch_autograd():
    q, r, k, u, v, do = _inputs(23, 3, 16, 4, 12, 1)
    ts = [t.clone().requires_grad_(True) for t in (q, r, k, u, v)]
    out = _torch_core(*ts)
    out.backward(do)
    o = M.mhffn_forward(q.numpy(), r.numpy(), k.numpy(), u.numpy(), v.numpy())
    np.testing.assert_allclose(o, out.detach().numpy(), rtol=1e-12, atol=1e-12)
    grads = M.mhffn_backward(do.numpy(), q.numpy(), r.numpy(), k.numpy(), u.numpy(), v.numpy())
    for ours, t in zip(grads, ts):
        np.testing.assert_allclose(ours, t.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_one_head_one_subnetwork_is_swiglu():
    """E = 1 and R = 1: each head is a SwiGLU of width d_e on its d_h inputs."""
    q, _, k, u, v, _ = _inputs(17, 2, 8, 1, 20, 2)
    r = torch.ones(17, 2, 1, dtype=torch.float64)
    o = M.mhffn_forward(q.numpy(), r.numpy(), k.numpy(), u.numpy(), v.numpy())
    for h in range(2):
        ref = (torch.nn.functional.silu(q[:, h] @ k[h, 0].T) * (q[:, h] @ u[h, 0].T)) @ v[h, 0]
        np.testing.assert_allclose(o[:, h], ref.numpy(), rtol=1e-13, atol=1e-13)


def test_router_linearity_and_zero_router():
    q, r, k, u, v, _ = _inputs(9, 2, 8, 3, 6, 3)
    args = [a.numpy() for a in (q, r, k, u, v)]
    o = M.mhffn_forward(*args)
    o2 = M.mhffn_forward(args[0], 2.0 * args[1], *args[2:])
    np.testing.assert_allclose(o2, 2.0 * o, rtol=1e-13)
    z = M.mhffn_forward(args[0], np.zeros_like(args[1]), *args[2:])
    assert np.count_nonzero(z) == 0
    # sub-networks add: the sum of single-sub-network outputs
    parts = sum(M.mhffn_forward(args[0], args[1][:, :, e:e + 1], args[2][:, e:e + 1], args[3][:, e:e + 1],
                                args[4][:, e:e + 1]) for e in range(3))
    np.testing.assert_allclose(parts, o, rtol=1e-12, atol=1e-14)


def test_finite_differences():
    q, r, k, u, v, do = _inputs(5, 2, 4, 2, 3, 4)
    args = [a.numpy().copy() for a in (q, r, k, u, v)]
    dn = do.numpy()
    grads = M.mhffn_backward(dn, *args)
    loss = lambda a: float((M.mhffn_forward(*a) * dn).sum())
    rng = np.random.default_rng(0)
    h = 1e-6
    for which in range(5):
        for _ in range(4):
            i = tuple(rng.integers(0, n) for n in args[which].shape)
            p = [a.copy() for a in args]
            m = [a.copy() for a in args]
            p[which][i] += h
            m[which][i] -= h
            fd = (loss(p) - loss(m)) / (2 * h)
            assert abs(fd - grads[which][i]) <= 1e-6 * max(1.0, abs(fd))


def test_heads_are_independent():
    q, r, k, u, v, _ = _inputs(7, 3, 8, 2, 5, 5)
    args = [a.numpy() for a in (q, r, k, u, v)]
    o = M.mhffn_forward(*args)
    o1 = M.mhffn_forward(args[0][:, 1:2], args[1][:, 1:2], args[2][1:2], args[3][1:2], args[4][1:2])
    np.testing.assert_allclose(o1[:, 0], o[:, 1], rtol=1e-13)
