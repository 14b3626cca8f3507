"""Plain float64 oracle of one DECO MoE feed-forward layer, forward pass.

TEST INFRASTRUCTURE.  Slow and obviously correct on purpose: numpy float64,
one BLAS matmul per step, no blocking, fusion or reordering.  It shares no
code with the HIP library; only `tests/`, the smoke check and the benchmark's
CPU-baseline leg may call it.

Sources (the method's equations section is missing from the available text of
the DECO paper, so the steps below follow its prose):
  [P-DECO]  "DECO: Sparse Mixture-of-Experts with Dense-Comparable Performance
            on End-Side Devices" (arXiv 2605.10933, HTML version):
            Sec. 1 Introduction; Sec. 2 Related work, paragraphs "Router design"
            and "Expert design".
  [W-CN]    Chinese write-up of the same paper (qidianchuan.cn), section 二
            (core design of DECO): the router part, and the expert-design part
            on NormSiLU and non-gated experts.
  The TopK variant follows the baseline of [P-DECO] Sec. 4 (the acceleration
  paragraph and its Table 4), which replaces the ReLU routing by conventional
  TopK at the same average activation ratio.

Readings taken where the text is silent:
  * router = linear projection with a bias b_r, then ReLU, then a learned
    per-expert scale lambda_e applied after the ReLU; no softmax / unit-sum;
  * an expert is active for a token iff its logit is strictly positive
    (zero or negative scores are ignored) and lambda_e != 0;
  * NormSiLU mean term uses the mean of ALL routed experts' up-projection
    weights (fixed at inference, so it cannot depend on the active set);
    the shared expert is excluded;
  * intra-expert RMS over the d_ff entries of one (token, expert) row, with
    epsilon inside the square root and no learnable gain;
  * experts are non-gated two-matrix MLPs with no biases;
  * shared expert: non-gated MLP with plain SiLU, weight 1, no lambda;
  * no residual: the result is the FFN sublayer output only.
  * gated variant ("DECO (gated)", [W-CN] 二 and [P-DECO] Sec. 2 "Expert
    design", which compare it with the non-gated experts): a routed expert
    has a gate projection W_gate[e] next to W_up[e]; NormSiLU acts on the gate
    projection (its mean term from the mean of ALL experts' gate projections,
    its RMS over the gate row) and multiplies the up projection elementwise:
    a = NormSiLU(x.W_gate[e]) * (x.W_up[e]), y = a.W_down[e]; the shared
    expert is unchanged;
  * ablation switches ([W-CN] 二 reports the two NormSiLU steps removed one
    at a time and a scalar router scale in place of the per-expert one; the
    pages give no further detail): `normsilu_mean=False` drops step 1 (no
    mean term), `normsilu_rms=False` drops step 2 (r = 1, eps unused), both
    off give vanilla SiLU experts; `scalar_lambda=True` uses lambda[0] for
    every expert; `shared_rms=True` gives the shared expert an RMS-only
    NormSiLU (RMS over its Fs entries, eps inside the root, no mean term:
    there is one shared expert);
  * TopK variant (top_k = k > 0): the same router projection; each token keeps
    the k experts with the largest logits, ties going to the lower expert
    index; gates are the softmax of the kept logits (conventional TopK
    gating); no expert-wise scale (lambda belongs to the ReLU routing it
    replaces); experts and shared expert unchanged.

The pages print no worked numeric example of the layer, so no value here is
compared with a printed one; every function is pinned instead by invariants,
closed forms, dense brute force and library cross-checks
(tests/test_oracle_pins.py).
"""
from __future__ import annotations

import dataclasses

import numpy as np


def silu(v: np.ndarray) -> np.ndarray:
    """SiLU(v) = v * sigmoid(v), evaluated without overflow for large |v|."""
    v = np.asarray(v, dtype=np.float64)
    out = np.empty_like(v)
    pos = v >= 0
    out[pos] = v[pos] / (1.0 + np.exp(-v[pos]))
    ev = np.exp(v[~pos])
    out[~pos] = v[~pos] * ev / (1.0 + ev)
    return out


def router(x, W_r, b_r, lam):
    """ReLU router with expert-wise scaling.

    [P-DECO] Sec. 2 "Router design": a linear projection, an activation, and a
    post-processing of the scores; DECO uses ReLU as the activation and a
    learnable per-expert scaling factor in place of a fixed scalar.
    [W-CN] Sec. 二, router part: an expert with a positive score is used, a
    zero or negative score is ignored.

    Returns logits z [T,E], the active mask [T,E] (bool) and gates g [T,E]
    with g = lambda_e * max(z, 0) on active entries and 0 elsewhere.
    """
    z = np.asarray(x, np.float64) @ np.asarray(W_r, np.float64) + np.asarray(b_r, np.float64)
    lam = np.asarray(lam, np.float64)
    active = (z > 0.0) & (lam != 0.0)[None, :]
    g = np.where(active, lam[None, :] * np.maximum(z, 0.0), 0.0)
    return z, active, g


def router_topk(x, W_r, b_r, k: int):
    """TopK routing variant, the baseline of [P-DECO] Sec. 4 (acceleration
    paragraph, Table 4): conventional TopK in place of the ReLU routing.

    z = x . W_r + b_r as in `router`; per token the k largest logits are kept
    (a stable descending sort, so equal logits go to the lower expert index),
    and their gates are the softmax of the kept logits; every other gate is 0.
    Returns z [T,E], the active mask [T,E] (bool, exactly k per row) and g.
    """
    z = np.asarray(x, np.float64) @ np.asarray(W_r, np.float64) + np.asarray(b_r, np.float64)
    T, E = z.shape
    if not 1 <= k <= E:
        raise ValueError(f"top_k must be in 1..{E}")
    active = np.zeros((T, E), dtype=bool)
    g = np.zeros((T, E))
    for t in range(T):
        keep = np.argsort(-z[t], kind="stable")[:k]
        active[t, keep] = True
        w = np.exp(z[t, keep] - z[t, keep].max())
        g[t, keep] = w / w.sum()
    return z, active, g


def mean_up(W_up) -> np.ndarray:
    """Inter-expert mean of the up-projection weights, Wbar = (1/E) sum_e W_up[e].

    [W-CN] Sec. 二, expert design: the average over all experts' up-projection
    weights; at inference the weights are fixed, so this matrix is computed
    once and stored.  W_up: [E, d, F] -> [d, F].
    """
    W_up = np.asarray(W_up, np.float64)
    return W_up.sum(axis=0) / W_up.shape[0]


def normsilu(h, m, eps, use_mean: bool = True, use_rms: bool = True):
    """NormSiLU on up-projection rows.

    [W-CN] Sec. 二 and [P-DECO] Sec. 1/2: first subtract the inter-expert mean
    term m = x . Wbar from the expert's intermediate activation h, then
    normalise the scale inside the expert (RMS over the F entries of the row),
    then apply SiLU.  h, m: [n, F].  use_mean / use_rms = False drop step 1 /
    step 2 (the ablations of [W-CN] 二).
    """
    ht = np.asarray(h, np.float64)
    if use_mean:
        ht = ht - np.asarray(m, np.float64)
    if not use_rms:
        return silu(ht)
    r = np.sqrt(np.mean(ht * ht, axis=-1, keepdims=True) + eps)
    return silu(ht / r)


def expert_mlp(x_rows, m_rows, W_up_e, W_down_e, eps, use_mean: bool = True, use_rms: bool = True):
    """One non-gated routed expert: up-projection -> NormSiLU -> down-projection.

    [W-CN] Sec. 二 (non-gated MLP experts: two matrices, no gate matrix);
    [P-DECO] Sec. 2 "Expert design".  x_rows [n,d], m_rows [n,F] -> [n,d].
    """
    h = np.asarray(x_rows, np.float64) @ np.asarray(W_up_e, np.float64)
    return normsilu(h, m_rows, eps, use_mean, use_rms) @ np.asarray(W_down_e, np.float64)


def expert_mlp_gated(x_rows, m_rows, W_gate_e, W_up_e, W_down_e, eps, use_mean: bool = True,
                     use_rms: bool = True):
    """One gated routed expert ("DECO (gated)"): NormSiLU of the gate
    projection times the up projection, then the down-projection.

    [W-CN] Sec. 二 (gated MLP experts carry an extra multiplicative
    interaction); [P-DECO] Sec. 2 "Expert design".  m_rows is x . Wbar with
    Wbar the mean of the gate projections.  x_rows [n,d] -> [n,d].
    """
    x_rows = np.asarray(x_rows, np.float64)
    hg = x_rows @ np.asarray(W_gate_e, np.float64)
    u = x_rows @ np.asarray(W_up_e, np.float64)
    return (normsilu(hg, m_rows, eps, use_mean, use_rms) * u) @ np.asarray(W_down_e, np.float64)


def shared_expert(x, Ws_up, Ws_down, rms: bool = False, eps: float = 1e-6):
    """Always-on shared expert: non-gated MLP with plain SiLU, weight 1.

    [W-CN] Sec. 二 (a shared expert takes part for every token);
    [P-DECO] Sec. 1.  x [T,d] -> [T,d].  rms=True: the RMS-only NormSiLU
    ablation (u / sqrt(mean_j u_j^2 + eps) before the SiLU).
    """
    u = np.asarray(x, np.float64) @ np.asarray(Ws_up, np.float64)
    if rms:
        u = u / np.sqrt(np.mean(u * u, axis=-1, keepdims=True) + eps)
    return silu(u) @ np.asarray(Ws_down, np.float64)


@dataclasses.dataclass
class OracleResult:
    out: np.ndarray      # [T, d] float64
    z: np.ndarray        # [T, E] router logits
    active: np.ndarray   # [T, E] bool
    g: np.ndarray        # [T, E] gates
    routed: np.ndarray   # [T, d] routed part of out
    shared: np.ndarray   # [T, d] shared-expert part of out


def forward(x, W_r, b_r, lam, W_up, W_down, Ws_up, Ws_down, eps=1e-6, top_k: int = 0,
            W_gate=None, normsilu_mean: bool = True, normsilu_rms: bool = True,
            scalar_lambda: bool = False, shared_rms: bool = False) -> OracleResult:
    """Sparse evaluation of one DECO layer, expert by expert.

    Steps: router (the ReLU router, or with top_k > 0 the TopK variant);
    Wbar and m = x . Wbar; for each expert e the tokens S_e that activate it,
    in ascending order (per-expert bucketing), the expert MLP on those rows,
    and out[S_e] += g[S_e, e] * y (gate-weighted combine, [P-DECO] Sec. 2
    "Router design": the router assigns a weight to each expert); finally the
    shared expert is added.  With W_gate [E,d,F] the routed experts are the
    gated variant (`expert_mlp_gated`) and the mean term comes from W_gate.
    The last four switches are the ablations described in the module notes.
    """
    x = np.asarray(x, np.float64)
    T, d = x.shape
    W_up = np.asarray(W_up, np.float64)
    E = W_up.shape[0]
    if scalar_lambda:
        lam = np.full(E, np.asarray(lam, np.float64)[0])
    z, active, g = router_topk(x, W_r, b_r, top_k) if top_k > 0 else router(x, W_r, b_r, lam)
    m = x @ mean_up(W_up if W_gate is None else W_gate)
    routed = np.zeros((T, d))
    for e in range(E):
        S = np.nonzero(active[:, e])[0]
        if S.size == 0:
            continue
        if W_gate is None:
            y = expert_mlp(x[S], m[S], W_up[e], W_down[e], eps, normsilu_mean, normsilu_rms)
        else:
            y = expert_mlp_gated(x[S], m[S], np.asarray(W_gate, np.float64)[e], W_up[e], W_down[e], eps,
                                 normsilu_mean, normsilu_rms)
        routed[S] += g[S, e][:, None] * y
    shared = shared_expert(x, Ws_up, Ws_down, shared_rms, eps)
    return OracleResult(out=routed + shared, z=z, active=active, g=g, routed=routed, shared=shared)


def _topk_gates_by_subsets(z_row: np.ndarray, k: int) -> np.ndarray:
    """TopK gates of one token found by enumerating every k-subset of the
    experts: the subset with the largest logit sum (first in lexicographic
    order among equal sums), softmax-weighted.  Exponential; tiny E only."""
    import itertools
    E = z_row.shape[0]
    best, best_sum = None, -np.inf
    for sub in itertools.combinations(range(E), k):
        s = float(sum(z_row[list(sub)]))
        if s > best_sum:
            best, best_sum = sub, s
    g = np.zeros(E)
    w = np.array([np.exp(z_row[e] - max(z_row[list(best)])) for e in best])
    g[list(best)] = w / w.sum()
    return g


def forward_dense_bruteforce(x, W_r, b_r, lam, W_up, W_down, Ws_up, Ws_down, eps=1e-6,
                             top_k: int = 0, W_gate=None, normsilu_mean: bool = True,
                             normsilu_rms: bool = True, scalar_lambda: bool = False,
                             shared_rms: bool = False) -> np.ndarray:
    """Dense brute force for small inputs: every expert for every token.

    Ignores the mask: each (token, expert) pair is evaluated one at a time,
    the mean term is rebuilt per token as the average of that token's E
    up-projections (no precomputed Wbar), and the result is weighted by the
    gate, which is zero for inactive pairs.  With top_k > 0 the gates come
    from an enumeration of expert subsets instead of a sort.  Used only to
    pin `forward`.
    """
    x = np.asarray(x, np.float64)
    T, d = x.shape
    W_up = np.asarray(W_up, np.float64)
    W_down = np.asarray(W_down, np.float64)
    E = W_up.shape[0]
    if top_k > 0:
        zz = x @ np.asarray(W_r, np.float64) + np.asarray(b_r, np.float64)
        g = np.stack([_topk_gates_by_subsets(zz[t], top_k) for t in range(T)])
    else:
        lam_e = np.asarray(lam, np.float64)
        _, _, g = router(x, W_r, b_r, np.array([lam_e[0] if scalar_lambda else lam_e[e] for e in range(E)]))
    out = np.zeros((T, d))
    Wn = W_up if W_gate is None else np.asarray(W_gate, np.float64)   # NormSiLU input
    for t in range(T):
        h_all = np.stack([x[t] @ Wn[e] for e in range(E)])      # [E, F]
        m_t = h_all.sum(axis=0) / E
        for e in range(E):
            ht = h_all[e] - m_t if normsilu_mean else h_all[e]
            r = np.sqrt(np.mean(ht * ht) + eps) if normsilu_rms else 1.0
            a = silu(ht / r)
            if W_gate is not None:
                a = a * (x[t] @ W_up[e])
            out[t] += g[t, e] * (a @ W_down[e])
        us = x[t] @ np.asarray(Ws_up, np.float64)
        if shared_rms:
            us = us / np.sqrt(np.mean(us * us) + eps)
        out[t] += silu(us) @ np.asarray(Ws_down, np.float64)
    return out
