"""Pins of the oracle's backward (CPU, fp64), none of which retypes its
formulas: central finite differences of the pinned forward for every
gradient entry of a small layer; torch's fp64 autograd of a plain SwiGLU
FFN (E = k = 1, where the layer is that FFN); and properties that hold for
any input (the router gradient sums to zero over a token's experts, is zero
off the chosen experts and for k = 1, and an unused expert gets no weight
gradient)."""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def small_layer(T=6, E=4, k=2, d=5, f=3, seed=3):
    rng = np.random.default_rng(seed)
    f32 = np.float32
    return dict(
        logits=rng.standard_normal((T, E)).astype(f32),
        x=rng.standard_normal((T, d)).astype(f32),
        Wg=(rng.standard_normal((E, f, d)) * 0.6).astype(f32),
        Wu=(rng.standard_normal((E, f, d)) * 0.6).astype(f32),
        Wd=(rng.standard_normal((E, d, f)) * 0.6).astype(f32),
        dy=rng.standard_normal((T, d)).astype(f32), k=k)


def loss(L):
    """sum_t <y_t, dy_t> through the oracle's forward (fp64)."""
    idx, w = oracle.route(L["logits"], L["k"])
    T = L["x"].shape[0]
    y = oracle.forward_tokens(np.arange(T), idx, w, L["x"], L["Wg"], L["Wu"],
                              L["Wd"])
    return float(np.sum(y * L["dy"].astype(np.float64))), idx


def central_difference(L, name, pos, eps=2e-3):
    """(L(+) - L(-)) / (actual fp32 step), the step rounded as the input is."""
    base = L[name][pos]
    plus, minus = np.float32(base + eps), np.float32(base - eps)
    out = []
    for v in (plus, minus):
        L2 = dict(L)
        L2[name] = L[name].copy()
        L2[name][pos] = v
        out.append(loss(L2))
    (lp, ip), (lm, im) = out
    return (lp - lm) / (float(plus) - float(minus)), ip, im


def grads(L):
    idx, w = oracle.route(L["logits"], L["k"])
    T = L["x"].shape[0]
    E = L["Wg"].shape[0]
    dx, dl = oracle.backward_tokens(np.arange(T), idx, w, L["x"], L["Wg"],
                                    L["Wu"], L["Wd"], L["dy"])
    dW = [oracle.weight_grads(e, idx, w, L["x"], L["Wg"], L["Wu"], L["Wd"],
                              L["dy"]) for e in range(E)]
    return idx, dx, dl, dW


@pytest.mark.parametrize("k", [1, 2, 3])
def test_every_gradient_entry_against_central_differences(k):
    L = small_layer(k=k)
    idx, dx, dl, dW = grads(L)
    checks = [("x", dx, lambda p: p)]
    for name, which in (("Wg", 0), ("Wu", 1), ("Wd", 2)):
        checks.append((name, None, which))
    worst = 0.0
    for pos in np.ndindex(L["x"].shape):
        fd, _, _ = central_difference(L, "x", pos)
        worst = max(worst, abs(fd - dx[pos]))
    for name, which in (("Wg", 0), ("Wu", 1), ("Wd", 2)):
        for pos in np.ndindex(L[name].shape):
            fd, _, _ = central_difference(L, name, pos)
            worst = max(worst, abs(fd - dW[pos[0]][which][pos[1:]]))
    for pos in np.ndindex(L["logits"].shape):
        fd, ip, im = central_difference(L, "logits", pos, eps=1e-3)
        if not (np.array_equal(ip, idx) and np.array_equal(im, idx)):
            continue  # the step changed the selection: no derivative there
        worst = max(worst, abs(fd - dl[pos]))
    # central differences in fp64 of an fp64 loss: O(eps^2) + rounding
    assert worst < 2e-5, worst


def test_swiglu_ffn_against_torch_autograd():
    """E = k = 1: the layer is SwiGLU(x) with weight 1, so its gradients are
    those of torch's autograd on the FFN (fp64)."""
    torch = pytest.importorskip("torch")
    L = small_layer(T=8, E=1, k=1, d=16, f=12, seed=5)
    idx, dx, dl, dW = grads(L)
    t = {n: torch.tensor(L[n].astype(np.float64), requires_grad=True)
         for n in ("x", "Wg", "Wu", "Wd")}
    F = torch.nn.functional
    y = (F.silu(t["x"] @ t["Wg"][0].T) * (t["x"] @ t["Wu"][0].T)) @ t["Wd"][0].T
    (y * torch.tensor(L["dy"].astype(np.float64))).sum().backward()
    np.testing.assert_allclose(dx, t["x"].grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dW[0][0], t["Wg"].grad[0].numpy(), rtol=1e-12,
                               atol=1e-12)
    np.testing.assert_allclose(dW[0][1], t["Wu"].grad[0].numpy(), rtol=1e-12,
                               atol=1e-12)
    np.testing.assert_allclose(dW[0][2], t["Wd"].grad[0].numpy(), rtol=1e-12,
                               atol=1e-12)
    assert np.all(dl == 0.0)


@pytest.mark.parametrize("k", [1, 2, 4])
def test_router_gradient_properties(k):
    L = small_layer(T=20, E=6, k=k, d=8, f=7, seed=k)
    idx, dx, dl, _ = grads(L)
    chosen = np.zeros_like(dl, dtype=bool)
    np.put_along_axis(chosen, idx.astype(np.int64), True, axis=1)
    assert np.all(dl[~chosen] == 0.0)
    np.testing.assert_allclose(dl.sum(axis=1), 0.0, atol=1e-12)
    if k == 1:
        assert np.all(dl == 0.0)


def test_unused_expert_has_no_weight_gradient():
    L = small_layer(T=10, E=5, k=1, d=6, f=4, seed=9)
    L["logits"][:, 4] = -50.0  # expert 4 is never chosen
    idx, _, _, dW = grads(L)
    assert not np.any(idx == 4)
    for g in dW[4]:
        assert np.all(g == 0.0)
