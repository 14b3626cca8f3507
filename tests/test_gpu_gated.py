"""GPU parity of the gated-expert variant against the fp64 oracle.

The variant is "DECO (gated)", the expert design the DECO paper (Sec. 2
"Expert design") compares with its non-gated experts: NormSiLU acts on the
gate projection x.W_gate[e] (its mean term from the mean of all experts'
gate projections) and multiplies x.W_up[e] element by element before the
down-projection.  Loaded through deco_moe_load_weights_gated; both kernel
paths, with ReLU routing and with the TopK routing variant.  Same bar as
test_gpu_parity.py: excess over the output's half-ulp <= tol * RMS(out),
masks bit-exact outside the |z| < 1e-5 band (ReLU routing) or outside the
k-th/(k+1)-th near-tie band (TopK).
"""
import numpy as np
import pytest
import torch

import oracle
from synthetic import make_custom, make_layer
from synthetic.device import layer_tensors, x_tensor

pytestmark = pytest.mark.gpu

import sparse_moe_relu_amd as dm

TOL = {"bf16": 2e-2, "f32": 1e-4}
NEAR = 1e-5
DEC, PRE = dm.DECO_PATH_DECODE, dm.DECO_PATH_PREFILL


def _say(msg):
    print(f"[gated] {msg}", flush=True)


def half_ulp(v, dtype):
    _, ex = np.frexp(np.abs(v))
    bits = {"bf16": 8, "f32": 24}[dtype]
    return np.where(v == 0, 0.0, np.ldexp(1.0, ex - 1 - bits))


def _layer(L, max_tokens, k=0):
    t = layer_tensors(L)
    assert "W_gate" in t
    return dm.Layer(**t, max_tokens=max_tokens, eps=L.eps, top_k=k)


def check(L, layer, path, *, T=None, k=0, label=""):
    T = L.T if T is None else T
    _say(f"{label} T={T} k={k} path={path} d={L.d} E={L.E} F={L.F} Fs={L.Fs} {L.dtype}")
    ref = oracle.forward(L.x[:T], **L.weights(), eps=L.eps, top_k=k)
    out = layer(x_tensor(L)[:T].contiguous(), path=path)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got)), label
    act = layer.active_mask(T).numpy()
    if k == 0:
        near_tok = np.any(np.abs(ref.z) < NEAR, axis=1)
    else:
        zs = -np.sort(-ref.z, axis=1)
        near_tok = (zs[:, k - 1] - zs[:, k] < NEAR) if k < L.E else np.zeros(T, bool)
    mism = np.any(act != ref.active, axis=1)
    assert not np.any(mism & ~near_tok), f"{label}: {int(np.sum(mism & ~near_tok))} tokens routed differently"
    rows = ~near_tok
    rms = float(np.sqrt(np.mean(ref.out ** 2)))
    err = np.abs(got[rows] - ref.out[rows]) - half_ulp(got[rows], L.dtype)
    excess = float(err.max()) if err.size else 0.0
    assert excess <= TOL[L.dtype] * rms, f"{label}: excess {excess:.3e} > {TOL[L.dtype]} * rms {rms:.3e}"
    assert layer.error_flags() == 0
    _say(f"  ok: excess/rms={excess / rms:.2e} near={int(near_tok.sum())} active={ref.active.mean():.3f}")
    return got, ref


@pytest.mark.parametrize("path", [DEC, PRE])
def test_gated_c1_fp32(path):
    L = make_layer(1, gated=True)
    layer = _layer(L, 64)
    check(L, layer, path, label="c1")
    # the mean term comes from the gate projections
    wbar = layer.mean_up().cpu().numpy().astype(np.float64)
    want = oracle.mean_up(L.W_gate)
    assert np.max(np.abs(wbar - want)) <= 1e-6 * np.max(np.abs(want))
    layer.free()


def test_gated_c2_bf16_decode_and_prefill():
    L = make_layer(2, gated=True)
    layer = _layer(L, 64)
    got_d, ref = check(L, layer, DEC, label="c2")
    got_p, _ = check(L, layer, PRE, label="c2")
    rms = float(np.sqrt(np.mean(ref.out ** 2)))
    assert float(np.max(np.abs(got_d - got_p))) <= 2e-2 * rms
    # repeat: bitwise identical
    again = layer(x_tensor(L), path=DEC).float().cpu().numpy().astype(np.float64)
    assert np.array_equal(got_d, again)
    Lb = make_layer(2, T=16, gated=True)
    for T in (1, 5, 16):
        check(Lb, layer, DEC, T=T, label="c2-T")
    layer.free()


def test_gated_differs_from_nongated_layer():
    # the same router, W_up and W_down loaded without the gate give another
    # result: the gated kernels do not silently ignore W_gate
    L = make_layer(2, gated=True)
    gl = _layer(L, 16)
    t = layer_tensors(L)
    t.pop("W_gate")
    pl = dm.Layer(**t, max_tokens=16, eps=L.eps)
    a = gl(x_tensor(L), path=DEC).float()
    b = pl(x_tensor(L), path=DEC).float()
    assert float((a - b).abs().max()) > 0.1 * float(a.pow(2).mean().sqrt())
    gl.free()
    pl.free()


def test_gated_prefill_several_tiles_ragged():
    L = make_layer(3, T=700, gated=True)
    layer = _layer(L, 700)
    check(L, layer, PRE, label="c3-700")
    for T in (17, 129):
        check(L, layer, PRE, T=T, label="c3-ragged")
    layer.free()


def test_gated_prefill_full_size():
    L = make_layer(3, gated=True)
    layer = _layer(L, L.T)
    got, _ = check(L, layer, PRE, label="c3")
    again = layer(x_tensor(L), path=PRE).float().cpu().numpy().astype(np.float64)
    assert np.array_equal(got, again)
    layer.free()


@pytest.mark.parametrize("shape", [
    (128, 5, 32, 64, "bf16"),     # E not a multiple of 16, smallest F
    (192, 70, 64, 96, "bf16"),    # two mask words, F = 64
    (256, 12, 256, 32, "bf16"),   # widest F
    (128, 3, 256, 160, "f32"),
])
@pytest.mark.parametrize("path", [DEC, PRE])
def test_gated_shapes(shape, path):
    d, E, F, Fs, dt = shape
    T = 11 if path == DEC else 77
    L = make_custom(d, E, F, Fs, T, dt, seed=9, ratio=0.3, gated=True)
    layer = _layer(L, 80)
    check(L, layer, path, label=f"shape{shape}")
    layer.free()


@pytest.mark.parametrize("path", [DEC, PRE])
def test_gated_with_topk_routing(path):
    L = make_layer(2, gated=True)
    k = round(0.2 * L.E)
    layer = _layer(L, 64, k)
    check(L, layer, path, k=k, label="c2-topk")
    layer.free()


@pytest.mark.parametrize("path", [DEC, PRE])
def test_gated_no_active_expert_is_shared_only(path):
    L = make_custom(256, 24, 128, 128, 13, "bf16", seed=4, gated=True)
    L.b_r = np.full_like(L.b_r, -1e4)
    layer = _layer(L, 32)
    _, ref = check(L, layer, path, label="all-negative")
    assert not ref.active.any()
    layer.free()
