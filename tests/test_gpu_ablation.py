"""GPU parity of the ablation switches (deco_moe_config.normsilu,
scalar_lambda, shared_rms) against the fp64 oracle, both kernel paths.

The switches are the ablations the qidianchuan.cn write-up of the DECO paper
reports (section 二): NormSiLU without its mean term, without its RMS step
(both off: vanilla SiLU experts), a scalar router scale, and an RMS-only
NormSiLU shared expert.  Same bar as test_gpu_parity.py.
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
FLAGS = {
    "no_mean": dict(normsilu_mean=False),
    "no_rms": dict(normsilu_rms=False),
    "vanilla": dict(normsilu_mean=False, normsilu_rms=False),
    "scalar_lambda": dict(scalar_lambda=True),
    "shared_rms": dict(shared_rms=True),
    "all": dict(normsilu_mean=False, scalar_lambda=True, shared_rms=True),
}


def _say(msg):
    print(f"[abl] {msg}", flush=True)


def half_ulp(v, dtype):
    _, ex = np.frexp(np.abs(v))
    bits = {"bf16": 8, "f32": 24}[dtype]
    return np.where(v == 0, 0.0, np.ldexp(1.0, ex - 1 - bits))


def check(L, layer, path, flags, *, T=None, label=""):
    T = L.T if T is None else T
    _say(f"{label} T={T} path={path} {L.dtype} {flags}")
    ref = oracle.forward(L.x[:T], **L.weights(), eps=L.eps, **flags)
    out = layer(x_tensor(L)[:T].contiguous(), path=path)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got)), label
    act = layer.active_mask(T).numpy()
    near = np.any(np.abs(ref.z) < NEAR, axis=1)
    mism = np.any(act != ref.active, axis=1)
    assert not np.any(mism & ~near), f"{label}: {int(np.sum(mism & ~near))} tokens routed differently"
    rows = ~near
    rms = float(np.sqrt(np.mean(ref.out ** 2)))
    err = np.abs(got[rows] - ref.out[rows]) - half_ulp(got[rows], L.dtype)
    excess = float(err.max()) if err.size else 0.0
    assert excess <= TOL[L.dtype] * rms, f"{label}: excess {excess:.3e} > {TOL[L.dtype]} * rms {rms:.3e}"
    _say(f"  ok: excess/rms={excess / rms:.2e}")
    return got


@pytest.mark.parametrize("name", list(FLAGS))
@pytest.mark.parametrize("path", [DEC, PRE])
def test_ablation_c1_fp32(name, path):
    L = make_layer(1)
    layer = dm.Layer(**layer_tensors(L), max_tokens=64, eps=L.eps, **FLAGS[name])
    check(L, layer, path, FLAGS[name], label=f"c1-{name}")
    layer.free()


@pytest.mark.parametrize("name", list(FLAGS))
def test_ablation_bf16_decode_and_prefill(name):
    L = make_layer(2, T=16)
    layer = dm.Layer(**layer_tensors(L), max_tokens=300, eps=L.eps, **FLAGS[name])
    check(L, layer, DEC, FLAGS[name], T=8, label=f"c2-{name}")
    check(L, layer, DEC, FLAGS[name], T=1, label=f"c2-{name}")
    Lp = make_layer(2, T=300)   # the same weights (they do not depend on T), 300 tokens
    check(Lp, layer, PRE, FLAGS[name], label=f"c2-300-{name}")
    layer.free()


@pytest.mark.parametrize("name", ["vanilla", "shared_rms"])
def test_ablation_prefill_full_size(name):
    # the size the sweep measures the ablations at (c3, T = 4096)
    L = make_layer(3)
    layer = dm.Layer(**layer_tensors(L), max_tokens=L.T, eps=L.eps, **FLAGS[name])
    check(L, layer, PRE, FLAGS[name], label=f"c3-4096-{name}")
    layer.free()


def test_ablation_shapes_and_topk():
    # E not a multiple of 16, Fs not a multiple of 64, TopK routing with the switches
    L = make_custom(192, 70, 64, 96, 77, "bf16", seed=9, ratio=0.3)
    fl = dict(normsilu_rms=False, shared_rms=True)
    layer = dm.Layer(**layer_tensors(L), max_tokens=80, eps=L.eps, **fl)
    check(L, layer, DEC, fl, T=11, label="E70-dec")
    check(L, layer, PRE, fl, label="E70-pre")
    layer.free()
    k = 11
    Lk = make_layer(2, T=16)
    layer = dm.Layer(**layer_tensors(Lk), max_tokens=16, eps=Lk.eps, top_k=k, normsilu_mean=False)
    for path in (DEC, PRE):
        ref = oracle.forward(Lk.x, **Lk.weights(), eps=Lk.eps, top_k=k, normsilu_mean=False)
        got = layer(x_tensor(Lk), path=path).float().cpu().numpy().astype(np.float64)
        rms = float(np.sqrt(np.mean(ref.out ** 2)))
        assert float(np.max(np.abs(got - ref.out) - half_ulp(got, "bf16"))) <= 2e-2 * rms
    layer.free()
