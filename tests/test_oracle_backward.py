"""Pins of the backward oracle (oracle/deco_backward.py), CPU only.

The hand-written chain rule is checked against things it does not share code
with: central finite differences of the objective (the forward oracle plus
the entropy term) on small inputs whose routing cannot flip under the step,
and a torch float64 autograd of a forward written here independently.  The
coefficient rule and the entropy are checked against closed forms.
"""
import numpy as np
import pytest
import torch

import oracle
from synthetic import make_custom

NAMES = ["W_r", "b_r", "lam", "W_up", "W_down", "Ws_up", "Ws_down"]
GRAD = {"W_r": "dW_r", "b_r": "db_r", "lam": "dlam", "W_up": "dW_up", "W_down": "dW_down",
        "Ws_up": "dWs_up", "Ws_down": "dWs_down"}


def _layer(seed, d=8, E=4, F=4, Fs=6, T=6, ratio=0.4, margin=0.02, top_k=0):
    """A small fp32 layer whose routing has a margin: no |z| below `margin`
    (ReLU routing) or no k-th / (k+1)-th logit gap below it (TopK), so a
    finite-difference step cannot change the active sets."""
    for s in range(seed, seed + 200):
        L = make_custom(d, E, F, Fs, T, "f32", seed=s, ratio=ratio)
        z = L.x @ L.W_r + L.b_r
        if top_k:
            zs = -np.sort(-z, axis=1)
            ok = np.all(zs[:, top_k - 1] - zs[:, top_k] > margin) if top_k < E else True
        else:
            act = z > 0
            ok = np.all(np.abs(z) > margin) and act.any() and not act.all()
        if ok:
            return L
    raise RuntimeError("no seed with the routing margin")


def _dout(L, seed=3):
    return np.random.default_rng(seed).standard_normal((L.T, L.d))


def _fd_check(L, dout, reg=0.0, top_k=0, h=1e-6, rtol=2e-6):
    w = {k: np.array(v, np.float64) for k, v in L.weights().items()}
    x = np.array(L.x, np.float64)
    G = oracle.backward(x, **w, dout=dout, eps=L.eps, reg_coef=reg, top_k=top_k)

    def f(xx, ww):
        return oracle.objective(xx, **ww, dout=dout, eps=L.eps, reg_coef=reg, top_k=top_k)

    def fd_of(arr_get, arr_set, shape):
        out = np.zeros(shape)
        for idx in np.ndindex(shape):
            base = arr_get()[idx]
            arr_set(idx, base + h)
            fp = f(x, w)
            arr_set(idx, base - h)
            fm = f(x, w)
            arr_set(idx, base)
            out[idx] = (fp - fm) / (2 * h)
        return out

    checks = {"dx": fd_of(lambda: x, lambda i, v: x.__setitem__(i, v), x.shape)}
    for n in NAMES:
        arr = w[n]
        checks[GRAD[n]] = fd_of(lambda a=arr: a, lambda i, v, a=arr: a.__setitem__(i, v), arr.shape)
    for k, fd in checks.items():
        got = getattr(G, k)
        scale = max(np.max(np.abs(fd)), 1e-3)
        assert np.max(np.abs(got - fd)) <= rtol * scale + 1e-8, (k, np.max(np.abs(got - fd)), scale)
    return G


def test_backward_matches_finite_differences_relu():
    L = _layer(100)
    _fd_check(L, _dout(L))


def test_backward_matches_finite_differences_with_entropy_term():
    L = _layer(200, E=5, ratio=0.5)
    # some token must have two or more active experts, or the term vanishes
    z = L.x @ L.W_r + L.b_r
    assert ((z > 0).sum(axis=1) >= 2).any()
    _fd_check(L, _dout(L, 4), reg=0.7)


def test_backward_matches_finite_differences_topk():
    L = _layer(300, E=5, top_k=2)
    _fd_check(L, _dout(L, 5), top_k=2)


def _torch_objective(x, W_r, b_r, lam, W_up, W_down, Ws_up, Ws_down, dout, eps, reg, active):
    """The layer written with torch ops (masks as constants): autograd gives
    an independent gradient."""
    z = x @ W_r + b_r
    g = torch.where(active, lam[None, :] * torch.relu(z), torch.zeros_like(z))
    Wbar = W_up.mean(dim=0)
    m = x @ Wbar
    out = torch.nn.functional.silu(x @ Ws_up) @ Ws_down
    for e in range(W_up.shape[0]):
        h = x @ W_up[e] - m
        r = torch.sqrt((h * h).mean(dim=1, keepdim=True) + eps)
        y = torch.nn.functional.silu(h / r) @ W_down[e]
        out = out + g[:, e:e + 1] * y      # zero gate rows contribute nothing
    L = (dout * out).sum()
    if reg:
        Hs = []
        for t in range(x.shape[0]):
            gt = g[t][active[t]]
            if gt.numel() == 0:
                Hs.append(torch.zeros((), dtype=x.dtype))
                continue
            p = gt / gt.sum()
            Hs.append(-(p * torch.log(p)).sum())
        L = L + reg * torch.stack(Hs).mean()
    return L


@pytest.mark.parametrize("reg", [0.0, 0.5])
def test_backward_matches_torch_autograd(reg):
    L = make_custom(32, 6, 16, 24, 20, "f32", seed=12, ratio=0.3)
    dout = _dout(L, 9)
    G = oracle.backward(L.x, **L.weights(), dout=dout, eps=L.eps, reg_coef=reg)
    t = {k: torch.tensor(np.asarray(v, np.float64), requires_grad=True) for k, v in L.weights().items()}
    xt = torch.tensor(np.asarray(L.x, np.float64), requires_grad=True)
    z = L.x @ L.W_r + L.b_r
    active = torch.tensor((z > 0) & (L.lam != 0)[None, :])
    obj = _torch_objective(xt, t["W_r"], t["b_r"], t["lam"], t["W_up"], t["W_down"], t["Ws_up"],
                           t["Ws_down"], torch.tensor(dout), L.eps, reg, active)
    obj.backward()
    assert np.isclose(obj.item(), oracle.objective(L.x, **L.weights(), dout=dout, eps=L.eps, reg_coef=reg),
                      rtol=1e-12, atol=1e-12)
    pairs = [("dx", xt)] + [(GRAD[n], t[n]) for n in NAMES]
    for k, tt in pairs:
        want = tt.grad.numpy()
        got = getattr(G, k)
        assert np.max(np.abs(got - want)) <= 1e-10 * max(np.max(np.abs(want)), 1e-12), k
    assert G.n_active == int(active.sum())


def test_no_active_expert_leaves_only_the_shared_gradient():
    L = make_custom(16, 4, 8, 12, 5, "f32", seed=2)
    L.b_r = np.full_like(L.b_r, -1e3)
    dout = _dout(L, 1)
    G = oracle.backward(L.x, **L.weights(), dout=dout, eps=L.eps, reg_coef=0.3)
    us = L.x @ L.Ws_up
    sig = 1 / (1 + np.exp(-us))
    dus = (dout @ L.Ws_down.T) * (sig * (1 + us * (1 - sig)))
    assert np.allclose(G.dx, dus @ L.Ws_up.T, rtol=1e-12, atol=1e-12)
    for k in ("dW_r", "db_r", "dlam", "dW_down"):
        assert not np.any(getattr(G, k)), k
    # the mean term still reaches W_up only through active experts: none here
    assert not np.any(G.dW_up)
    assert G.n_active == 0


def test_dsilu_closed_forms_and_difference_quotient():
    assert oracle.dsilu(np.array([0.0]))[0] == 0.5
    u = np.linspace(-30, 30, 241)
    h = 1e-6
    fd = (oracle.silu(u + h) - oracle.silu(u - h)) / (2 * h)
    assert np.max(np.abs(oracle.dsilu(u) - fd)) < 1e-8
    assert np.allclose(oracle.dsilu(np.array([60.0, -60.0])), [1.0, 0.0], atol=1e-20)


def test_router_entropy_closed_forms():
    g = np.array([[1.0, 1.0, 1.0, 0.0], [2.0, 0.0, 0.0, 0.0], [0.0] * 4, [3.0, 1.0, 0.0, 0.0]])
    act = g > 0
    H = oracle.router_entropy(g, act)
    assert np.isclose(H[0], np.log(3))
    assert H[1] == 0.0 and H[2] == 0.0
    assert np.isclose(H[3], -(0.75 * np.log(0.75) + 0.25 * np.log(0.25)))
    # scale invariance in the gates
    assert np.allclose(oracle.router_entropy(5 * g, act), H)


def test_sparsity_coef_update_rule():
    c = 0.1
    assert oracle.sparsity_coef_update(c, 0.25, 0.20) == c * 1.002
    assert oracle.sparsity_coef_update(c, 0.15, 0.20) == c / 1.002
    assert oracle.sparsity_coef_update(c, 0.20, 0.20) == c
    for _ in range(10):
        c = oracle.sparsity_coef_update(c, 0.3, 0.2)
    assert np.isclose(c, 0.1 * 1.002 ** 10, rtol=1e-15)


def test_backward_gradient_is_linear_in_dout_without_regulariser():
    L = make_custom(16, 5, 8, 8, 7, "f32", seed=8, ratio=0.4)
    a, b = _dout(L, 1), _dout(L, 2)
    Ga = oracle.backward(L.x, **L.weights(), dout=a, eps=L.eps)
    Gb = oracle.backward(L.x, **L.weights(), dout=b, eps=L.eps)
    Gab = oracle.backward(L.x, **L.weights(), dout=2 * a - b, eps=L.eps)
    for k in ("dx", "dW_r", "dlam", "dW_up", "dW_down", "dWs_up"):
        assert np.allclose(getattr(Gab, k), 2 * getattr(Ga, k) - getattr(Gb, k), rtol=1e-10, atol=1e-12), k
