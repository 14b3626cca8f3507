"""Plain float64 oracle of the DECO layer's backward pass and of the adaptive
sparsity-coefficient rule.

TEST INFRASTRUCTURE, like `deco_oracle`: numpy float64, the chain rule written
out step by step in the reverse order of the forward pass, one matmul per
step.  It shares no code with the HIP library.

Sources:
  [P-DECO]  "DECO: Sparse Mixture-of-Experts with Dense-Comparable Performance
            on End-Side Devices": Sec. 2 "Router design", "Expert design" and
            "Auxiliary training objective" (an adaptive sparsity
            regularisation whose coefficient scales itself, with router
            entropy in place of an L1 norm).
  [W-CN]    qidianchuan.cn write-up, section 三 (sparsity control): the
            penalty is the router entropy; after every training iteration the
            coefficient is multiplied by a factor slightly above 1 (1.002 in
            the example) when the activation ratio is above the target and
            divided by it when below.

Readings taken where the text is silent:
  * the objective whose gradient is returned is
        L = sum(dout * out) + reg_coef * (1/T) * sum_t H_t,
    dout being the upstream gradient of the layer output;
  * router entropy of token t (the formula is not on the pages): the entropy
    of the token's gates normalised over its active experts,
        p_te = g_te / sum_{e active} g_te,   H_t = -sum_{e active} p_te log p_te,
    0 for a token with no active expert.  It is high when many experts share
    the weight and low when few do, as the write-up describes.  Used with the
    ReLU routing only (reg_coef must be 0 with TopK);
  * the mean term Wbar = mean_e W_up[e] is a function of W_up during
    training: every expert's W_up receives (1/E) x^T dm, whether or not it is
    active;
  * the ReLU's derivative at z = 0 is 0 (the mask is strict), and an expert
    with lambda_e = 0 is inactive and gets no gradient (its output is never
    formed);
  * TopK variant: the kept set is a constant; the softmax over the kept
    logits is differentiated;
  * coefficient rule: equal ratio and target leave the coefficient unchanged.

Pinned by central finite differences of `objective` on small inputs and by a
torch float64 autograd of an independently written forward
(tests/test_oracle_backward.py).
"""
from __future__ import annotations

import dataclasses

import numpy as np

from .deco_oracle import mean_up, router, router_topk, silu


def dsilu(u: np.ndarray) -> np.ndarray:
    """d/du SiLU(u) = sigma(u) * (1 + u * (1 - sigma(u)))."""
    u = np.asarray(u, np.float64)
    s = 0.5 * (1.0 + np.tanh(0.5 * u))   # sigma(u) without overflow
    return s * (1.0 + u * (1.0 - s))


def router_entropy(g: np.ndarray, active: np.ndarray) -> np.ndarray:
    """Per-token entropy of the gates normalised over the active experts
    (the reading above); 0 for tokens with no active expert.  [T]."""
    g = np.asarray(g, np.float64)
    H = np.zeros(g.shape[0])
    for t in range(g.shape[0]):
        A = np.nonzero(active[t])[0]
        S = g[t, A].sum()
        if A.size == 0 or S <= 0.0:
            continue
        p = g[t, A] / S
        H[t] = -np.sum(p * np.log(p))
    return H


def sparsity_coef_update(coef: float, ratio: float, target: float, factor: float = 1.002) -> float:
    """One step of the adaptive coefficient ([W-CN] 三): multiply by `factor`
    when the measured activation ratio is above the target, divide when below."""
    if ratio > target:
        return coef * factor
    if ratio < target:
        return coef / factor
    return coef


def objective(x, W_r, b_r, lam, W_up, W_down, Ws_up, Ws_down, dout, eps=1e-6,
              reg_coef: float = 0.0, top_k: int = 0) -> float:
    """L = sum(dout * out) + reg_coef * mean_t H_t (the function whose
    gradient `backward` returns), evaluated straight from the forward pass."""
    from .deco_oracle import forward
    r = forward(x, W_r, b_r, lam, W_up, W_down, Ws_up, Ws_down, eps=eps, top_k=top_k)
    L = float(np.sum(np.asarray(dout, np.float64) * r.out))
    if reg_coef:
        L += reg_coef * float(np.mean(router_entropy(r.g, r.active)))
    return L


@dataclasses.dataclass
class Grads:
    dx: np.ndarray       # [T, d]
    dW_r: np.ndarray     # [d, E]
    db_r: np.ndarray     # [E]
    dlam: np.ndarray     # [E]
    dW_up: np.ndarray    # [E, d, F]
    dW_down: np.ndarray  # [E, F, d]
    dWs_up: np.ndarray   # [d, Fs]
    dWs_down: np.ndarray # [Fs, d]
    n_active: int        # active (token, expert) pairs of the call


def backward(x, W_r, b_r, lam, W_up, W_down, Ws_up, Ws_down, dout, eps=1e-6,
             reg_coef: float = 0.0, top_k: int = 0) -> Grads:
    """Gradients of `objective` with respect to x and every weight."""
    f64 = lambda a: np.asarray(a, np.float64)
    x, W_r, lam, W_up, W_down, Ws_up, Ws_down, dout = map(
        f64, (x, W_r, lam, W_up, W_down, Ws_up, Ws_down, dout))
    T, d = x.shape
    E, _, F = W_up.shape
    if top_k > 0 and reg_coef:
        raise ValueError("the entropy regulariser belongs to the ReLU routing")

    # forward quantities the chain rule needs
    if top_k > 0:
        z, active, g = router_topk(x, W_r, b_r, top_k)
    else:
        z, active, g = router(x, W_r, b_r, lam)
    Wbar = mean_up(W_up)
    m = x @ Wbar
    us = x @ Ws_up
    s = silu(us)

    # shared expert: out += SiLU(x Ws_up) Ws_down
    dWs_down = s.T @ dout
    dus = (dout @ Ws_down.T) * dsilu(us)
    dWs_up = x.T @ dus
    dx = dus @ Ws_up.T

    # routed experts: out[S] += g[S, e] * (NormSiLU(x_S W_up[e] - m_S) W_down[e])
    dg = np.zeros((T, E))
    dm = np.zeros((T, F))
    dW_up = np.zeros((E, d, F))
    dW_down = np.zeros((E, F, d))
    for e in range(E):
        S = np.nonzero(active[:, e])[0]
        if S.size == 0:
            continue
        xs, gs = x[S], g[S, e][:, None]
        ht = xs @ W_up[e] - m[S]                                   # NormSiLU step 1
        r = np.sqrt(np.mean(ht * ht, axis=1, keepdims=True) + eps)  # step 2
        u = ht / r
        a = silu(u)
        q = dout[S] @ W_down[e].T                                  # d(out . dout)/dy, ungated
        dW_down[e] = a.T @ (gs * dout[S])
        dg[S, e] = np.sum(a * q, axis=1)
        du = gs * q * dsilu(u)
        # through u = ht / r with r = sqrt(mean(ht^2) + eps)
        dht = du / r - ht * np.sum(du * ht, axis=1, keepdims=True) / (F * r ** 3)
        dW_up[e] += xs.T @ dht
        dx[S] += dht @ W_up[e].T
        dm[S] -= dht
    # the mean term: m = x Wbar with Wbar = (1/E) sum_e W_up[e]
    dWbar = x.T @ dm
    dW_up += dWbar[None, :, :] / E
    dx += dm @ Wbar.T

    # sparsity regulariser: reg_coef * mean_t H_t, through the gates
    if reg_coef:
        for t in range(T):
            A = np.nonzero(active[t])[0]
            Sg = g[t, A].sum()
            if A.size == 0 or Sg <= 0.0:
                continue
            p = g[t, A] / Sg
            H = -np.sum(p * np.log(p))
            dg[t, A] += reg_coef / T * (-(np.log(p) + H) / Sg)

    # router
    if top_k > 0:
        dz = np.zeros((T, E))
        for t in range(T):
            K = np.nonzero(active[t])[0]
            p = g[t, K]
            dz[t, K] = p * (dg[t, K] - np.sum(p * dg[t, K]))
        dlam = np.zeros(E)
    else:
        dz = np.where(active, lam[None, :] * dg, 0.0)
        dlam = np.sum(np.where(active, np.maximum(z, 0.0) * dg, 0.0), axis=0)
    dW_r = x.T @ dz
    db_r = dz.sum(axis=0)
    dx += dz @ W_r.T
    return Grads(dx=dx, dW_r=dW_r, db_r=db_r, dlam=dlam, dW_up=dW_up, dW_down=dW_down,
                 dWs_up=dWs_up, dWs_down=dWs_down, n_active=int(active.sum()))
