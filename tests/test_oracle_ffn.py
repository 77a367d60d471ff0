"""Pins of the oracle's expert FFN and weighted collect: a library SwiGLU,
a numpy per-expert evaluation, invariants and a scalar closed form. CPU."""
from decimal import Decimal, getcontext

import numpy as np
import scipy.special
import torch

import oracle


def _rand(shape, rng, scale=1.0):
    return (rng.standard_normal(shape) * scale).astype(np.float32)


def numpy_layer(x, idx, w, Wg, Wu, Wd):
    """y_t = sum_j w_tj * FFN_{idx_tj}(x_t), each expert evaluated on every
    token with numpy matmul, then gathered."""
    x64 = x.astype(np.float64)
    E = Wg.shape[0]
    outs = []
    for e in range(E):
        g = x64 @ Wg[e].astype(np.float64).T
        u = x64 @ Wu[e].astype(np.float64).T
        h = g * scipy.special.expit(g) * u
        outs.append(h @ Wd[e].astype(np.float64).T)
    outs = np.stack(outs)  # [E, T, d]
    T = x.shape[0]
    y = np.zeros((T, x.shape[1]))
    for j in range(idx.shape[1]):
        y += w[:, j:j + 1] * outs[idx[:, j], np.arange(T)]
    return y, outs


def test_single_expert_is_library_swiglu():
    rng = np.random.default_rng(11)
    T, d, f = 37, 24, 40
    x = _rand((T, d), rng)
    Wg, Wu = _rand((1, f, d), rng, 0.2), _rand((1, f, d), rng, 0.2)
    Wd = _rand((1, d, f), rng, 0.2)
    idx, w = oracle.route(np.zeros((T, 1), np.float32), 1)
    y = oracle.forward_tokens(np.arange(T), idx, w, x, Wg, Wu, Wd)
    xt = torch.from_numpy(x).double()
    ref = (torch.nn.functional.silu(xt @ torch.from_numpy(Wg[0]).double().T)
           * (xt @ torch.from_numpy(Wu[0]).double().T)) @ torch.from_numpy(Wd[0]).double().T
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-13)


def test_multi_expert_matches_numpy_per_expert():
    rng = np.random.default_rng(12)
    T, E, k, d, f = 50, 5, 2, 16, 24
    logits = _rand((T, E), rng)
    x = _rand((T, d), rng)
    Wg, Wu = _rand((E, f, d), rng, 0.3), _rand((E, f, d), rng, 0.3)
    Wd = _rand((E, d, f), rng, 0.3)
    idx, w = oracle.route(logits, k)
    y = oracle.forward_tokens(np.arange(T), idx, w, x, Wg, Wu, Wd)
    ref, outs = numpy_layer(x, idx, w, Wg, Wu, Wd)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-13)
    # per-assignment outputs and h
    a_list = np.arange(T * k)
    h, o = oracle.assignment_outputs(a_list, idx, x, Wg, Wu, Wd, want_h=True)
    flat = idx.reshape(-1)
    np.testing.assert_allclose(o, outs[flat, a_list // k], rtol=1e-12,
                               atol=1e-13)
    xa = x[a_list // k].astype(np.float64)
    g = np.einsum("si,sqi->sq", xa, Wg[flat].astype(np.float64))
    u = np.einsum("si,sqi->sq", xa, Wu[flat].astype(np.float64))
    np.testing.assert_allclose(h, g * scipy.special.expit(g) * u, rtol=1e-12,
                               atol=1e-13)


def test_identical_experts_give_single_ffn():
    rng = np.random.default_rng(13)
    T, E, k, d, f = 30, 6, 3, 8, 12
    x = _rand((T, d), rng)
    g1, u1, d1 = _rand((f, d), rng, 0.4), _rand((f, d), rng, 0.4), _rand((d, f), rng, 0.4)
    Wg = np.stack([g1] * E)
    Wu = np.stack([u1] * E)
    Wd = np.stack([d1] * E)
    idx, w = oracle.route(_rand((T, E), rng), k)
    y = oracle.forward_tokens(np.arange(T), idx, w, x, Wg, Wu, Wd)
    idx1, w1 = oracle.route(np.zeros((T, 1), np.float32), 1)
    y1 = oracle.forward_tokens(np.arange(T), idx1, w1, x, Wg[:1], Wu[:1], Wd[:1])
    np.testing.assert_allclose(y, y1, rtol=1e-13, atol=1e-14)


def test_zero_input_gives_zero_output():
    rng = np.random.default_rng(14)
    T, E, k, d, f = 10, 4, 2, 8, 8
    x = np.zeros((T, d), np.float32)
    Wg, Wu, Wd = _rand((E, f, d), rng), _rand((E, f, d), rng), _rand((E, d, f), rng)
    idx, w = oracle.route(_rand((T, E), rng), k)
    y = oracle.forward_tokens(np.arange(T), idx, w, x, Wg, Wu, Wd)
    assert np.all(y == 0.0)


def test_scalar_closed_form():
    """d = f = 1, two experts, k = 2, equal logits (w = 1/2 each):
    y = 1/2 * c0*silu(a0 x)*(b0 x) + 1/2 * c1*silu(a1 x)*(b1 x),
    silu(z) = z / (1 + e^-z), evaluated with 40-digit decimals."""
    getcontext().prec = 40
    x, a, b, c = 2.0, [0.5, -1.0], [3.0, 1.0], [-1.0, 2.0]

    def silu(z):
        z = Decimal(z)
        return z / (1 + (-z).exp())

    exact = sum(Decimal("0.5") * Decimal(c[e]) * silu(a[e] * x) * Decimal(b[e] * x)
                for e in range(2))
    Wg = np.array(a, np.float32).reshape(2, 1, 1)
    Wu = np.array(b, np.float32).reshape(2, 1, 1)
    Wd = np.array(c, np.float32).reshape(2, 1, 1)
    idx, w = oracle.route(np.zeros((1, 2), np.float32), 2)
    assert idx.tolist() == [[0, 1]] and w.tolist() == [[0.5, 0.5]]
    y = oracle.forward_tokens(np.arange(1), idx, w,
                              np.array([[x]], np.float32), Wg, Wu, Wd)
    assert abs(Decimal(float(y[0, 0])) - exact) <= abs(exact) * Decimal(1e-15)
