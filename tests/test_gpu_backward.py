"""GPU parity of the backward pass (deco_moe_backward) against the fp64 oracle
(oracle/deco_backward.py, pinned by finite differences and autograd).

Bar, per gradient tensor G: max |G_gpu - G_oracle| <= tol * RMS(G_oracle),
tol = 1e-4 for fp32 layers and 2e-2 for bf16 layers (the forward's bar).  It
follows from the arithmetic: the fp32 intermediates that feed products (dh~,
g*a, the row dm | dz | du_s, s) are carried as bf16 high and low parts
(about 16 significant bits); what stays rounded once is the forward's own
(the mean term's bf16 Wbar) and dx's expert part (dh~ and its pair rows in
fp16), each at most 2^-9 relative per term with fp32 accumulation.  With
one rounding of dh~ or g*a to bf16 instead, dW_up and dW_down miss this bar
by 4x on the heavy-tailed gates (max |G| / RMS(G) up to 44).
Routing is compared as in the forward tests: cases are drawn so no logit
lies within 1e-5 of its decision boundary, and the call's pair count must
equal the oracle's.
"""
import numpy as np
import pytest
import torch

import oracle
from synthetic import make_custom, make_dout, make_layer
from synthetic.device import layer_tensors, to_tensor, x_tensor

pytestmark = pytest.mark.gpu

import sparse_moe_relu_amd as dm

TOL = {"bf16": 2e-2, "f32": 1e-4}
NAMES = ["dx", "dW_r", "db_r", "dlambda", "dW_up", "dW_down", "dWs_up", "dWs_down"]
ORACLE = {"dlambda": "dlam"}


def _say(msg):
    print(f"[bwd] {msg}", flush=True)


def _layer(L, max_tokens, k=0):
    return dm.Layer(**layer_tensors(L), max_tokens=max_tokens, eps=L.eps, top_k=k, backward=True)


def _margin_ok(L, k):
    z = L.x @ L.W_r + L.b_r
    if k:
        zs = -np.sort(-z, axis=1)
        return k == L.E or bool(np.all(zs[:, k - 1] - zs[:, k] > 1e-5))
    return bool(np.all(np.abs(z) > 1e-5))


def check(L, layer, *, k=0, reg=0.0, seed=1, label=""):
    assert _margin_ok(L, k), f"{label}: a logit sits on a routing boundary; pick another seed"
    dout = make_dout(L, seed)
    _say(f"{label} T={L.T} d={L.d} E={L.E} F={L.F} Fs={L.Fs} {L.dtype} k={k} reg={reg}")
    ref = oracle.backward(L.x, **L.weights(), dout=dout, eps=L.eps, reg_coef=reg, top_k=k)
    got = layer.backward(x_tensor(L), to_tensor(dout, L.dtype), reg_coef=reg)
    torch.cuda.synchronize()
    assert int(got["n_active_pairs"].item()) == ref.n_active, label
    worst = {}
    for n in NAMES:
        g = got[n].cpu().numpy().astype(np.float64)
        want = getattr(ref, ORACLE.get(n, n))
        assert g.shape == want.shape, (n, g.shape, want.shape)
        assert np.all(np.isfinite(g)), (label, n)
        rms = float(np.sqrt(np.mean(want ** 2)))
        err = float(np.max(np.abs(g - want))) if g.size else 0.0
        worst[n] = err / rms if rms > 0 else err
        assert err <= TOL[L.dtype] * rms + (1e-30 if rms == 0 else 0.0), \
            f"{label}: {n} max err {err:.3e} > {TOL[L.dtype]} * rms {rms:.3e}"
    _say("  ok: " + " ".join(f"{n}={v:.1e}" for n, v in worst.items()) + f" pairs={ref.n_active}")
    return got


def test_backward_c1_fp32():
    L = make_layer(1)
    layer = _layer(L, 64)
    check(L, layer, label="c1")
    layer.free()


def test_backward_c1_fp32_with_entropy_term():
    L = make_layer(1)
    layer = _layer(L, 64)
    check(L, layer, reg=0.3, label="c1-reg")
    layer.free()


def test_backward_bf16_decode_layer_shapes_and_determinism():
    L = make_layer(2, T=64)
    layer = _layer(L, 64)
    a = check(L, layer, label="c2-64")
    dout = to_tensor(make_dout(L, 1), L.dtype)
    b = layer.backward(x_tensor(L), dout)
    for n in NAMES:
        assert torch.equal(a[n], b[n]), n   # no atomics: bitwise repeatable
    layer.free()


def test_backward_bf16_several_tiles_ragged():
    # seed 1: no logit of the 700 x 56 within 1e-5 of zero (seed 0 has one)
    L = make_layer(3, seed=1, T=700)
    layer = _layer(L, 700)
    check(L, layer, label="c3-700", seed=2)
    layer.free()


def test_backward_c3_full_size():
    # the size and launch shapes the bench times (T = 4096, d = 2048, 56 experts);
    # seed 5: no logit of the 4096 x 56 within 1e-5 of zero (seeds 1-4 have one)
    L = make_layer(3, seed=5)
    layer = _layer(L, L.T)
    check(L, layer, label="c3-4096", seed=2)
    layer.free()


def test_backward_two_way_split_of_the_dense_weight_gradients():
    # 1024 <= T < 2048: the dense weight-gradient jobs split their K = T rows in
    # two ranges (one below, four from 2048); seed 2 keeps every logit off zero
    L = make_layer(3, seed=2, T=1500)
    layer = _layer(L, L.T)
    check(L, layer, label="c3-1500", seed=3)
    layer.free()


def test_backward_bf16_entropy_term():
    L = make_layer(2, T=200, ratio=0.3)
    layer = _layer(L, 200)
    check(L, layer, reg=0.05, label="c2-reg", seed=3)
    layer.free()


@pytest.mark.parametrize("k", [1, 11])
def test_backward_topk(k):
    L = make_layer(2, T=96)
    layer = _layer(L, 96, k)
    check(L, layer, k=k, label=f"topk{k}", seed=4)
    layer.free()


@pytest.mark.parametrize("shape", [
    (128, 5, 32, 64, "bf16"),     # E not a multiple of 16, smallest F
    (192, 70, 64, 96, "bf16"),    # two mask words, Fs not a multiple of 64
    (256, 12, 256, 32, "bf16"),   # widest F
    (128, 3, 256, 160, "f32"),
])
def test_backward_shapes(shape):
    d, E, F, Fs, dt = shape
    L = make_custom(d, E, F, Fs, 77, dt, seed=9, ratio=0.3)
    layer = _layer(L, 80)
    check(L, layer, label=f"shape{shape}", seed=5)
    layer.free()


def test_backward_no_active_expert():
    L = make_custom(256, 24, 128, 128, 13, "bf16", seed=4)
    L.b_r = np.full_like(L.b_r, -1e4)
    layer = _layer(L, 32)
    got = check(L, layer, reg=0.1, label="all-negative")
    assert int(got["n_active_pairs"].item()) == 0
    layer.free()


def test_backward_needs_the_flag_and_rejects_bad_calls():
    L = make_layer(1)
    plain = dm.Layer(**layer_tensors(L), max_tokens=16, eps=L.eps)
    dout = to_tensor(make_dout(L), L.dtype)
    with pytest.raises(dm.DecoError) as ex:
        plain.backward(x_tensor(L), dout)
    assert ex.value.status == dm.DECO_ERR_UNSUPPORTED
    plain.free()
    layer = _layer(L, 16, k=2)
    with pytest.raises(dm.DecoError) as ex:
        layer.backward(x_tensor(L), dout, reg_coef=0.5)   # the entropy term is for the ReLU routing
    assert ex.value.status == dm.DECO_ERR_INVALID_ARG
    layer.free()


@pytest.mark.parametrize("case", ["T1", "E2", "E256_sparse"])
def test_backward_edges(case):
    if case == "T1":
        L = make_layer(2, T=1)                      # a single token: one-row tiles everywhere
    elif case == "E2":
        L = make_custom(64, 2, 32, 32, 9, "bf16", seed=0, ratio=0.5)   # the fewest experts it supports
    else:
        L = make_custom(128, 256, 32, 64, 40, "bf16", seed=3, ratio=0.05)   # 4 mask words, many empty experts
    layer = _layer(L, max(L.T, 16))
    check(L, layer, label=case, seed=6)
    layer.free()
