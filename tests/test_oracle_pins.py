"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test targets a plausible mistake: a dropped term (bias, lambda, mean term,
shared expert), a wrong sign, a wrong reduction axis, a transposed operand, a
wrong tie rule at zero, or broken bucketing/combine.  CPU only.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from synthetic import make_custom, make_layer, round_to_bf16, bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _fw(L, **over):
    x = over.pop("x", L.x)
    w = L.weights()
    w.update(over)
    return oracle.forward(x, **w, eps=L.eps)


def _rms(a):
    return float(np.sqrt(np.mean(np.asarray(a) ** 2)))


def _torch_shared(x, Ws_up, Ws_down):
    """Shared expert through torch library routines (a second, independent evaluation)."""
    xt = torch.from_numpy(np.ascontiguousarray(x))
    return (torch.nn.functional.silu(xt @ torch.from_numpy(Ws_up)) @ torch.from_numpy(Ws_down)).numpy()


# 1. brute force --------------------------------------------------------------
@pytest.mark.parametrize("case", ["c1", "c2slice", "skewed"])
def test_sparse_dispatch_equals_dense_bruteforce(case):
    if case == "c1":
        L = make_layer(1)
    elif case == "c2slice":
        # d=2048 layer of the decode workload, first 8 experts, 6 tokens
        L = make_custom(2048, 8, 128, 256, 6, "bf16", seed=3)
    else:
        L = make_custom(128, 12, 64, 96, 24, "f32", seed=5, skew_var=0.3, ratio=0.3)
    r = _fw(L)
    bf = oracle.forward_dense_bruteforce(L.x, **L.weights(), eps=L.eps)
    assert r.active.any() and not r.active.all()
    assert np.max(np.abs(r.out - bf)) <= 1e-12 * _rms(bf)


# 2./3. collapses to the shared expert ----------------------------------------
def test_all_negative_logits_give_shared_only():
    L = make_layer(1)
    r = _fw(L, b_r=np.full(L.E, -1e4))
    assert not r.active.any()
    assert np.array_equal(r.routed, np.zeros_like(r.routed))
    ref = _torch_shared(L.x, L.Ws_up, L.Ws_down)
    assert np.max(np.abs(r.out - ref)) <= 1e-13 * _rms(ref)


def test_lambda_zero_gives_shared_only_and_inactive():
    L = make_layer(1)
    r = _fw(L, lam=np.zeros(L.E))
    assert not r.active.any()
    ref = _torch_shared(L.x, L.Ws_up, L.Ws_down)
    assert np.max(np.abs(r.out - ref)) <= 1e-13 * _rms(ref)


def test_single_lambda_zero_only_drops_that_expert():
    L = make_layer(1)
    lam = L.lam.copy()
    lam[3] = 0.0
    r0 = _fw(L)
    r1 = _fw(L, lam=lam)
    assert r0.active[:, 3].any() and not r1.active[:, 3].any()
    # expert 3's contribution, rebuilt from the brute-force pieces
    m = L.x @ oracle.mean_up(L.W_up)
    S = np.nonzero(r0.active[:, 3])[0]
    y3 = oracle.expert_mlp(L.x[S], m[S], L.W_up[3], L.W_down[3], L.eps) * r0.g[S, 3][:, None]
    diff = r0.out.copy()
    diff[S] -= y3
    assert np.max(np.abs(diff - r1.out)) <= 1e-12 * _rms(r0.out)


def test_gate_is_linear_in_lambda():
    L = make_layer(1)
    r1 = _fw(L)
    r3 = _fw(L, lam=2.5 * L.lam)
    assert np.array_equal(r1.active, r3.active)
    assert np.max(np.abs(r3.routed - 2.5 * r1.routed)) <= 1e-12 * _rms(r1.routed)
    # and the gate equals lambda * logit on active entries (ReLU then scale)
    assert np.allclose(r1.g[r1.active], (L.lam[None, :] * r1.z)[r1.active], rtol=0, atol=0)


# 4./5. mean term ---------------------------------------------------------------
def test_mean_term_is_mean_of_expert_projections():
    L = make_layer(1)
    m = L.x @ oracle.mean_up(L.W_up)
    per = np.stack([L.x @ L.W_up[e] for e in range(L.E)])     # [E,T,F]
    assert np.max(np.abs(m - per.mean(axis=0))) <= 1e-12 * np.max(np.abs(per))


def test_mean_subtracted_activations_sum_to_zero_over_experts():
    # NormSiLU step 1 over the right set: sum_e (h_e - m) == 0 for every token
    L = make_custom(96, 7, 48, 32, 9, "f32", seed=11)
    m = L.x @ oracle.mean_up(L.W_up)
    ht = np.stack([L.x @ L.W_up[e] - m for e in range(L.E)])
    scale = np.max(np.abs(ht))
    assert np.max(np.abs(ht.sum(axis=0))) <= 1e-12 * scale
    # the wrong sign (adding m) would not sum to zero
    assert np.max(np.abs(np.stack([L.x @ L.W_up[e] + m for e in range(L.E)]).sum(0))) > 1e-3 * scale


def test_mean_includes_inactive_experts():
    # Wbar is fixed at load time: deactivating experts must not change the
    # routed output of the experts that stay active.
    L = make_layer(1)
    b = L.b_r.copy()
    b[[0, 5]] = -1e4
    r0 = _fw(L)
    r1 = _fw(L, b_r=b)
    keep = [e for e in range(L.E) if e not in (0, 5)]
    m = L.x @ oracle.mean_up(L.W_up)
    ref = np.zeros_like(r1.routed)
    for e in keep:
        S = np.nonzero(r0.active[:, e])[0]
        if S.size:
            ref[S] += r0.g[S, e][:, None] * oracle.expert_mlp(L.x[S], m[S], L.W_up[e], L.W_down[e], L.eps)
    assert np.max(np.abs(r1.routed - ref)) <= 1e-12 * _rms(ref)


# 6./8. RMS step -----------------------------------------------------------------
def test_up_projection_scale_invariance_at_eps0():
    L = make_layer(1)
    w = L.weights()
    a = oracle.forward(L.x, **w, eps=0.0)
    w["W_up"] = 7.25 * L.W_up
    b = oracle.forward(L.x, **w, eps=0.0)
    assert np.max(np.abs(a.out - b.out)) <= 1e-10 * _rms(a.out)


def test_pre_silu_rows_have_mean_square_ms_over_ms_plus_eps():
    rng = np.random.default_rng(0)
    h = rng.standard_normal((10, 32)) * 1e-3
    m = rng.standard_normal((10, 32)) * 1e-4
    eps = 1e-6
    ht = h - m
    ms = np.mean(ht * ht, axis=1)
    r = np.sqrt(ms + eps)
    u = ht / r[:, None]
    # invert SiLU numerically to check what normsilu fed it
    a = oracle.normsilu(h, m, eps)
    # u*sigmoid(u) is monotone for u > -1.278; check the relation on reconstructed u
    assert np.allclose(a, u / (1 + np.exp(-u)), rtol=1e-14, atol=0)
    assert np.allclose(np.mean(u * u, axis=1), ms / (ms + eps), rtol=1e-12)


def test_rms_axis_is_per_row():
    # rows with very different scales normalise independently (wrong axis fails)
    h = np.array([[1.0, -2.0, 3.0, 0.5], [100.0, 200.0, -50.0, 10.0]])
    a = oracle.normsilu(h, np.zeros_like(h), 0.0)
    a_row0 = oracle.normsilu(h[:1], np.zeros((1, 4)), 0.0)
    a_row1_scaled = oracle.normsilu(h[1:] / 100.0, np.zeros((1, 4)), 0.0)
    assert np.allclose(a[0], a_row0[0], rtol=1e-15)
    assert np.allclose(a[1], a_row1_scaled[0], rtol=1e-13)


# 7. E = 1 -----------------------------------------------------------------------
def test_single_expert_routed_contribution_vanishes():
    L = make_custom(64, 1, 32, 48, 12, "f32", seed=2, ratio=0.9)
    r = _fw(L)
    assert r.active.any()
    assert np.max(np.abs(r.routed)) <= 1e-12 * _rms(r.shared)


# 9. F = 1 closed form -------------------------------------------------------------
def test_f1_closed_form():
    with open(os.path.join(GOLDEN, "closed_forms.json")) as f:
        cf = json.load(f)
    h = np.array([[3.7], [-0.02], [1e-2]])
    a = oracle.normsilu(h, np.zeros_like(h), 1e-12)
    assert abs(a[0, 0] - cf["silu_of_plus_one"]) < 1e-6
    assert abs(a[1, 0] - cf["silu_of_minus_one"]) < 1e-6
    assert abs(a[2, 0] - cf["silu_of_plus_one"]) < 1e-6


# 10. single expert with Wbar = 0 vs torch rms_norm / silu ----------------------------
def test_single_active_expert_with_zero_mean_matches_torch_rmsnorm_silu():
    d, F, Fs, T = 64, 24, 16, 10
    L = make_custom(d, 2, F, Fs, T, "f32", seed=4)
    W_up = L.W_up.copy()
    W_up[1] = -W_up[0]                      # Wbar == 0 exactly
    b = np.array([1e4, -1e4])               # expert 0 always on, expert 1 never
    r = _fw(L, W_up=W_up, b_r=b)
    assert r.active[:, 0].all() and not r.active[:, 1].any()
    eps = L.eps
    h = torch.from_numpy(L.x @ W_up[0])
    a = torch.nn.functional.silu(torch.nn.functional.rms_norm(h, (F,), eps=eps))
    y = (a @ torch.from_numpy(L.W_down[0])).numpy() * r.g[:, :1]
    assert np.max(np.abs(r.routed - y)) <= 1e-12 * _rms(y)


# 11. token independence, expert permutation -----------------------------------------
def test_token_independence():
    L = make_layer(1)
    full = _fw(L).out
    rows = np.concatenate([_fw(L, x=L.x[t:t + 1]).out for t in range(L.T)])
    assert np.max(np.abs(full - rows)) <= 1e-12 * _rms(full)


def test_expert_permutation_equivariance():
    L = make_layer(1)
    perm = np.random.default_rng(1).permutation(L.E)
    r0 = _fw(L)
    r1 = _fw(L, W_r=L.W_r[:, perm], b_r=L.b_r[perm], lam=L.lam[perm],
             W_up=L.W_up[perm], W_down=L.W_down[perm])
    assert np.array_equal(r1.active, r0.active[:, perm])
    assert np.max(np.abs(r0.out - r1.out)) <= 1e-12 * _rms(r0.out)


def test_transposed_down_projection_is_detected():
    # non-square F != d: feeding W_down transposed would not even conform
    L = make_layer(1)
    with pytest.raises(ValueError):
        oracle.forward(L.x, L.W_r, L.b_r, L.lam, L.W_up, np.swapaxes(L.W_down, 1, 2),
                       L.Ws_up, L.Ws_down, eps=L.eps)


# zero tie ---------------------------------------------------------------------------
def test_zero_logit_is_inactive_and_positive_is_active():
    L = make_layer(1)
    x0 = np.zeros((3, L.d))
    b = np.zeros(L.E)
    b[2] = 1e-30
    b[4] = -1e-30
    r = _fw(L, x=x0, b_r=b)
    expect = np.zeros((3, L.E), bool)
    expect[:, 2] = True
    assert np.array_equal(r.active, expect)
    assert np.all(r.g[:, 2] == L.lam[2] * 1e-30)


# 12. realised ratio ---------------------------------------------------------------
@pytest.mark.parametrize("ratio", [0.05, 0.10, 0.20, 0.40])
def test_realised_activation_ratio_in_binomial_band(ratio):
    L = make_custom(512, 32, 32, 32, 512, "bf16", seed=7, ratio=ratio)
    _, active, _ = oracle.router(L.x, L.W_r, L.b_r, L.lam)
    n = active.size
    p_hat = active.mean()
    # per-token count is variable (ReLU routing), the mean is the target
    assert abs(p_hat - ratio) <= 5 * math.sqrt(ratio * (1 - ratio) / n) + 0.01
    per_tok = active.sum(axis=1)
    assert per_tok.min() < per_tok.max()


def test_generator_bf16_rounding_is_single_rne_cast():
    # halfway cases round to even; exact values stay; bits round-trip
    one = 1.0
    ulp = 2.0 ** -7
    v = np.array([one + ulp / 2, one + 3 * ulp / 2, one + ulp / 2 + 1e-12, -2.5, 0.0])
    r = round_to_bf16(v)
    assert r[0] == one and r[1] == one + 2 * ulp and r[2] == one + ulp
    assert r[3] == -2.5 and r[4] == 0.0
    bits = bf16_bits(r)
    assert bits[0] == 0x3F80 and bits[3] == 0xC020
    t = torch.tensor(v[:2], dtype=torch.float64).to(torch.bfloat16).double().numpy()
    assert np.array_equal(t, r[:2])


# TopK routing variant --------------------------------------------------------
def _fw_topk(L, k, **over):
    x = over.pop("x", L.x)
    w = L.weights()
    w.update(over)
    return oracle.forward(x, **w, eps=L.eps, top_k=k)


@pytest.mark.parametrize("k", [1, 2, 3, 5])
def test_topk_selection_equals_best_subset_and_softmax_gates(k):
    # selection pinned by enumerating every k-subset (largest logit sum) and
    # by the order statistics of the logits; gates by their defining ratios
    L = make_custom(64, 7, 32, 64, 12, "f32", seed=11)
    z, active, g = oracle.router_topk(L.x, L.W_r, L.b_r, k)
    for t in range(L.T):
        import itertools
        best = max(itertools.combinations(range(L.E), k), key=lambda s: sum(z[t, list(s)]))
        assert set(np.nonzero(active[t])[0]) == set(best)
        kept, dropped = z[t, active[t]], z[t, ~active[t]]
        assert dropped.size == 0 or kept.min() > dropped.max()
        assert math.isclose(g[t].sum(), 1.0, rel_tol=1e-12)
        assert np.all(g[t, ~active[t]] == 0.0) and np.all(g[t, active[t]] > 0.0)
        a = np.nonzero(active[t])[0]
        for i in a:
            for j in a:
                assert math.isclose(g[t, i] / g[t, j], math.exp(z[t, i] - z[t, j]), rel_tol=1e-9)


def test_topk_ties_go_to_lower_expert_index():
    x = np.eye(5)                              # token t reads row t of W_r
    W_r = np.array([[1.0, 3.0, 3.0, 0.0, 3.0]] * 5)
    z, active, g = oracle.router_topk(x, W_r, np.zeros(5), 2)
    assert np.array_equal(np.nonzero(active[0])[0], [1, 2])
    assert np.allclose(g[0, [1, 2]], 0.5)
    z, active, _ = oracle.router_topk(x, W_r, np.zeros(5), 4)
    assert np.array_equal(np.nonzero(active[0])[0], [0, 1, 2, 4])


def test_topk_k1_is_argmax_with_gate_one():
    L = make_custom(64, 8, 32, 64, 10, "f32", seed=12)
    z, active, g = oracle.router_topk(L.x, L.W_r, L.b_r, 1)
    assert np.array_equal(np.nonzero(active)[1], np.argmax(z, axis=1))
    assert np.array_equal(g[active], np.ones(L.T))


def test_topk_full_k_is_softmax_over_all_experts():
    L = make_custom(64, 8, 32, 64, 6, "f32", seed=13)
    z, active, g = oracle.router_topk(L.x, L.W_r, L.b_r, L.E)
    assert active.all()
    ref = torch.softmax(torch.from_numpy(z), dim=1).numpy()   # library routine
    assert np.max(np.abs(g - ref)) <= 1e-15


def test_topk_ignores_lambda_and_ratio_bias_sign():
    # the TopK variant has no expert-wise scale and keeps k experts whatever
    # the sign of the logits (a negative bias does not empty the selection)
    L = make_custom(64, 8, 32, 64, 6, "f32", seed=14)
    a = _fw_topk(L, 2)
    b = _fw_topk(L, 2, lam=np.zeros(L.E))
    c = _fw_topk(L, 2, b_r=L.b_r - 100.0)
    assert np.array_equal(a.out, b.out)
    assert np.all(c.active.sum(axis=1) == 2)
    assert np.max(np.abs(a.out - c.out)) <= 1e-12 * _rms(a.out)   # a shift of every logit changes nothing


@pytest.mark.parametrize("k", [1, 3])
def test_topk_sparse_forward_equals_subset_bruteforce(k):
    L = make_custom(128, 6, 64, 96, 9, "f32", seed=15)
    r = _fw_topk(L, k)
    bf = oracle.forward_dense_bruteforce(L.x, **L.weights(), eps=L.eps, top_k=k)
    assert np.all(r.active.sum(axis=1) == k)
    assert np.max(np.abs(r.out - bf)) <= 1e-12 * _rms(bf)


# gated-expert variant --------------------------------------------------------
def test_gated_sparse_forward_equals_dense_bruteforce():
    L = make_custom(128, 7, 64, 96, 10, "f32", seed=21, gated=True, ratio=0.3)
    r = oracle.forward(L.x, **L.weights(), eps=L.eps)
    bf = oracle.forward_dense_bruteforce(L.x, **L.weights(), eps=L.eps)
    assert r.active.any() and not r.active.all()
    assert np.max(np.abs(r.out - bf)) <= 1e-12 * _rms(bf)


def test_gated_with_unit_up_projection_is_the_nongated_layer_on_the_gate():
    # x carries a constant-1 feature and W_up reads only it, so x.W_up = 1:
    # the gated expert must reduce to the non-gated one whose up-projection
    # is W_gate (catches swapped gate/up roles and a mean term on the wrong
    # projection)
    L = make_custom(64, 6, 32, 64, 9, "f32", seed=22, gated=True, ratio=0.4)
    x = L.x.copy()
    x[:, -1] = 1.0
    W_one = np.zeros_like(L.W_up)
    W_one[:, -1, :] = 1.0
    w = L.weights()
    gated = oracle.forward(x, **dict(w, W_up=W_one), eps=L.eps)
    w.pop("W_gate")
    plain = oracle.forward(x, **dict(w, W_up=L.W_gate), eps=L.eps)
    assert gated.active.any()
    assert np.max(np.abs(gated.out - plain.out)) <= 1e-12 * _rms(plain.out)


def test_gated_routed_part_is_linear_in_the_up_projection():
    L = make_custom(64, 6, 32, 64, 9, "f32", seed=23, gated=True, ratio=0.4)
    a = oracle.forward(L.x, **L.weights(), eps=L.eps)
    b = oracle.forward(L.x, **dict(L.weights(), W_up=-3.0 * L.W_up), eps=L.eps)
    assert np.max(np.abs(b.routed + 3.0 * a.routed)) <= 1e-12 * _rms(a.routed)
    assert np.array_equal(a.shared, b.shared)


def test_gated_mean_term_is_the_mean_gate_projection():
    # shifting every expert's gate projection by the same matrix leaves the
    # mean-subtracted gate rows, and so the layer, unchanged
    L = make_custom(64, 6, 32, 64, 9, "f32", seed=24, gated=True, ratio=0.4)
    rng = np.random.default_rng(5)
    shift = rng.standard_normal((L.d, L.F))
    a = oracle.forward(L.x, **L.weights(), eps=L.eps)
    b = oracle.forward(L.x, **dict(L.weights(), W_gate=L.W_gate + shift[None]), eps=L.eps)
    assert np.max(np.abs(a.out - b.out)) <= 1e-10 * _rms(a.out)


# ablation switches ------------------------------------------------------------
ABL = [dict(normsilu_mean=False), dict(normsilu_rms=False), dict(normsilu_mean=False, normsilu_rms=False),
       dict(scalar_lambda=True), dict(shared_rms=True)]


@pytest.mark.parametrize("flags", ABL)
def test_ablation_sparse_forward_equals_dense_bruteforce(flags):
    L = make_custom(96, 7, 64, 80, 10, "f32", seed=31, ratio=0.35)
    r = oracle.forward(L.x, **L.weights(), eps=L.eps, **flags)
    bf = oracle.forward_dense_bruteforce(L.x, **L.weights(), eps=L.eps, **flags)
    assert r.active.any() and not r.active.all()
    assert np.max(np.abs(r.out - bf)) <= 1e-12 * _rms(bf)
    # each switch changes the result
    base = oracle.forward(L.x, **L.weights(), eps=L.eps)
    assert np.max(np.abs(r.out - base.out)) > 1e-3 * _rms(base.out)


def test_ablation_without_both_steps_is_a_vanilla_silu_mlp():
    # library check: torch's SiLU MLP per expert, gate-weighted, plus the shared expert
    L = make_custom(64, 5, 32, 48, 9, "f32", seed=32, ratio=0.4)
    r = oracle.forward(L.x, **L.weights(), eps=L.eps, normsilu_mean=False, normsilu_rms=False)
    x = torch.tensor(L.x)
    out = torch.nn.functional.silu(x @ torch.tensor(L.Ws_up)) @ torch.tensor(L.Ws_down)
    g = torch.tensor(r.g)
    for e in range(L.E):
        y = torch.nn.functional.silu(x @ torch.tensor(L.W_up[e])) @ torch.tensor(L.W_down[e])
        out = out + g[:, e:e + 1] * y
    assert np.max(np.abs(r.out - out.numpy())) <= 1e-12 * _rms(r.out)


def test_ablation_no_rms_equals_full_on_unit_rms_rows():
    # one token, two experts, F = 2: h~ = (1, -1) and (-1, 1) have RMS 1, so
    # with eps = 0 dropping step 2 changes nothing; scaling W_up by 3 then
    # changes the no-RMS layer only
    x = np.array([[1.0]])
    W_up = np.array([[[2.0, 0.0]], [[0.0, 2.0]]])
    W_down = np.array([[[0.5], [-1.5]], [[2.0], [0.25]]])
    kw = dict(W_r=np.array([[1.0, 1.0]]), b_r=np.zeros(2), lam=np.array([0.7, 1.3]), W_down=W_down,
              Ws_up=np.array([[0.3]]), Ws_down=np.array([[1.1]]), eps=0.0)
    full = oracle.forward(x, W_up=W_up, **kw).out
    norms = oracle.forward(x, W_up=W_up, **kw, normsilu_rms=False).out
    assert np.allclose(full, norms, rtol=0, atol=1e-15)
    full3 = oracle.forward(x, W_up=3 * W_up, **kw).out
    norms3 = oracle.forward(x, W_up=3 * W_up, **kw, normsilu_rms=False).out
    assert np.allclose(full3, full, rtol=0, atol=1e-15)          # RMS step: scale invariant
    assert np.max(np.abs(norms3 - full)) > 1e-2


def test_ablation_no_mean_equals_full_on_zero_mean_experts():
    L = make_custom(64, 6, 32, 48, 9, "f32", seed=33, ratio=0.4)
    W0 = L.W_up - L.W_up.mean(axis=0, keepdims=True)     # the experts' mean is zero
    w = dict(L.weights(), W_up=W0)
    a = oracle.forward(L.x, **w, eps=L.eps).out
    b = oracle.forward(L.x, **w, eps=L.eps, normsilu_mean=False).out
    assert np.max(np.abs(a - b)) <= 1e-12 * _rms(a)


def test_ablation_shared_rms_is_scale_invariant_and_plain_on_unit_rms():
    L = make_custom(64, 4, 32, 2, 1, "f32", seed=34)
    L.b_r = np.full_like(L.b_r, -1e3)                    # shared expert only
    x = np.zeros((1, 64))
    x[0, 0] = 1.0
    Ws_up = np.zeros((64, 2))
    Ws_up[0] = [1.0, -1.0]                               # u = (1, -1): RMS 1
    w = dict(L.weights(), Ws_up=Ws_up)
    plain = oracle.forward(x, **w, eps=0.0).out
    rmsv = oracle.forward(x, **w, eps=0.0, shared_rms=True).out
    assert np.allclose(plain, rmsv, rtol=0, atol=1e-15)
    rms5 = oracle.forward(x, **dict(w, Ws_up=5 * Ws_up), eps=0.0, shared_rms=True).out
    assert np.allclose(rms5, rmsv, rtol=0, atol=1e-15)


def test_ablation_scalar_lambda_is_lambda0_everywhere():
    L = make_custom(64, 6, 32, 48, 9, "f32", seed=35, ratio=0.4)
    a = oracle.forward(L.x, **L.weights(), eps=L.eps, scalar_lambda=True)
    b = oracle.forward(L.x, **dict(L.weights(), lam=np.full_like(L.lam, L.lam[0])), eps=L.eps)
    assert np.array_equal(a.out, b.out) and np.array_equal(a.g, b.g)
