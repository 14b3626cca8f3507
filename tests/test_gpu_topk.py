"""GPU parity of the TopK routing variant (top_k > 0) against the fp64 oracle.

The variant is the baseline of the DECO paper's Sec. 4 acceleration
experiment (Table 4): conventional TopK in place of the ReLU routing, same
experts.  Where floating point decides the selection, both sides decide in
their own precision and are compared where that cannot matter:
  * the GPU keeps exactly the top_k of its own fp32 logits (ties to the lower
    expert index), bit-exact;
  * its selection equals the oracle's except on tokens whose oracle k-th and
    (k+1)-th largest logits lie within NEAR of each other (counted);
  * outputs on the other tokens meet the bar of test_gpu_parity.py
    (excess over the output's half-ulp <= tol * RMS(out_oracle)).
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


def _say(msg):
    print(f"[topk] {msg}", flush=True)


def half_ulp(v, dtype):
    _, ex = np.frexp(np.abs(v))
    bits = {"bf16": 8, "f32": 24}[dtype]
    return np.where(v == 0, 0.0, np.ldexp(1.0, ex - 1 - bits))


def run_topk(L, k, layer, path, T=None, label=""):
    T = L.T if T is None else T
    _say(f"{label} k={k} T={T} path={path} d={L.d} E={L.E} {L.dtype}")
    ref = oracle.forward(L.x[:T], **L.weights(), eps=L.eps, top_k=k)
    out = layer(x_tensor(L)[:T].contiguous(), path=path)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    act = layer.active_mask(T).numpy()
    _, logits = layer.routing(T)
    zg = logits.cpu().numpy().astype(np.float64)
    assert np.all(act.sum(axis=1) == k), f"{label}: not exactly k experts per token"
    for t in range(T):
        own = np.argsort(-zg[t], kind="stable")[:k]
        assert set(np.nonzero(act[t])[0]) == set(own), f"{label}: token {t} is not the top-k of its own logits"
    zs = -np.sort(-ref.z, axis=1)
    gap = zs[:, k - 1] - zs[:, k] if k < L.E else np.full(T, np.inf)
    near = gap < NEAR
    mism = np.any(act != ref.active, axis=1)
    assert not np.any(mism & ~near), f"{label}: {int(np.sum(mism & ~near))} tokens select differently"
    rows = ~near
    rms = float(np.sqrt(np.mean(ref.out ** 2)))
    err = np.abs(got[rows] - ref.out[rows]) - half_ulp(got[rows], L.dtype)
    excess = float(err.max()) if err.size else 0.0
    assert np.all(np.isfinite(got)), label
    assert excess <= TOL[L.dtype] * rms, f"{label}: excess {excess:.3e} > {TOL[L.dtype]} * rms {rms:.3e}"
    assert layer.error_flags() == 0
    _say(f"  ok: excess/rms={excess / rms:.2e} near_ties={int(near.sum())} mismatched_in_band={int(mism.sum())}")
    return got


def _layer(L, max_tokens, k):
    return dm.Layer(**layer_tensors(L), max_tokens=max_tokens, eps=L.eps, top_k=k)


@pytest.mark.parametrize("path", [dm.DECO_PATH_DECODE, dm.DECO_PATH_PREFILL])
@pytest.mark.parametrize("k", [1, 2, 8])
def test_topk_c1_fp32(path, k):
    L = make_layer(1)
    layer = _layer(L, 64, k)
    run_topk(L, k, layer, path, label="c1")
    layer.free()


@pytest.mark.parametrize("path", [dm.DECO_PATH_DECODE, dm.DECO_PATH_PREFILL])
def test_topk_c2_bf16_twenty_percent(path):
    L = make_layer(2)
    k = round(0.2 * L.E)
    layer = _layer(L, 64, k)
    got = run_topk(L, k, layer, path, label="c2")
    # repeat: bitwise identical
    again = layer(x_tensor(L), path=path).float().cpu().numpy().astype(np.float64)
    assert np.array_equal(got, again)
    for T in (1, 5):
        run_topk(L, k, layer, path, T=T, label="c2-T")
    layer.free()


def test_topk_c2_all_experts_and_single_expert():
    L = make_layer(2)
    for k in (L.E, 1):
        layer = _layer(L, 16, k)
        run_topk(L, k, layer, dm.DECO_PATH_DECODE, label="c2-edge")
        run_topk(L, k, layer, dm.DECO_PATH_PREFILL, label="c2-edge")
        layer.free()


def test_topk_prefill_several_tiles_ragged():
    L = make_layer(3, T=700)
    k = 11
    layer = _layer(L, 700, k)
    run_topk(L, k, layer, dm.DECO_PATH_PREFILL, label="c3-700")
    layer.free()


def test_topk_prefill_full_size():
    # the size the sweep measures the TopK baseline at (T = 4096, k = 11 of 56)
    L = make_layer(3)
    k = 11
    layer = _layer(L, L.T, k)
    run_topk(L, k, layer, dm.DECO_PATH_PREFILL, label="c3-4096")
    layer.free()


def test_topk_wide_expert_set_decode():
    # E = 200: four words of mask, router panels past 64 experts
    L = make_custom(256, 200, 32, 64, 12, "bf16", seed=41)
    layer = _layer(L, 16, 40)
    run_topk(L, 40, layer, dm.DECO_PATH_DECODE, label="E200")
    run_topk(L, 40, layer, dm.DECO_PATH_PREFILL, label="E200")
    layer.free()
