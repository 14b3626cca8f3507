"""The fp16 operand range of bf16 layers (both kernel paths run the routed
down-projection on fp16 operands, and the prefill pair rows are fp16).

Heavy gates (lambda_e = 1e3 for every expert, the scale the DECO router
learns per expert reaching three orders of magnitude) must still match the
oracle at the usual bar; gates that push the fp16 operands past 65504
(lambda_e = 1e6) must raise error bit 5 on both paths instead of returning
inf silently; a W_down entry outside the fp16 range is refused at load
(DECO_ERR_UNSUPPORTED) for bf16 layers and accepted for fp32 layers.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from synthetic import make_custom, make_layer
from synthetic.device import layer_tensors, x_tensor

pytestmark = pytest.mark.gpu

import sparse_moe_relu_amd as dm

DEC, PRE = dm.DECO_PATH_DECODE, dm.DECO_PATH_PREFILL
RANGE_BIT = 32


def _say(msg):
    print(f"[fp16] {msg}", flush=True)


def half_ulp(v, dtype):
    _, ex = np.frexp(np.abs(v))
    bits = {"bf16": 8, "f32": 24}[dtype]
    return np.where(v == 0, 0.0, np.ldexp(1.0, ex - 1 - bits))


def _with_lambda(L, lam):
    return dataclasses.replace(L, lam=np.full_like(L.lam, lam))


@pytest.mark.parametrize("path,T", [(DEC, 8), (PRE, 64)])
def test_heavy_gates_match_oracle(path, T):
    L = _with_lambda(make_layer(2, T=T), 1e3)
    ref = oracle.forward(L.x, **L.weights(), eps=L.eps)
    layer = dm.Layer(**layer_tensors(L), max_tokens=64, eps=L.eps)
    layer.error_flags()
    got = layer(x_tensor(L), path=path).float().cpu().numpy().astype(np.float64)
    rms = float(np.sqrt(np.mean(ref.out ** 2)))
    excess = float(np.max(np.abs(got - ref.out) - half_ulp(got, "bf16")))
    amax = float(np.max(np.abs(ref.g)))
    _say(f"lambda=1e3 path={path} T={T}: max gate {amax:.3g}, rms(out) {rms:.3g}, excess/rms {excess / rms:.2e}")
    assert np.all(np.isfinite(got))
    assert excess <= 2e-2 * rms
    assert layer.error_flags() == 0
    layer.free()


@pytest.mark.parametrize("path,T", [(DEC, 8), (PRE, 64)])
def test_gates_past_fp16_range_raise_the_flag(path, T):
    L = _with_lambda(make_layer(2, T=T), 1e6)
    layer = dm.Layer(**layer_tensors(L), max_tokens=64, eps=L.eps)
    layer.error_flags()
    layer(x_tensor(L), path=path)
    torch.cuda.synchronize()
    flags = layer.error_flags()
    _say(f"lambda=1e6 path={path} T={T}: flags {flags}")
    assert flags & RANGE_BIT
    layer.free()


def test_w_down_past_fp16_range_refused_for_bf16_only():
    L = make_custom(128, 8, 32, 64, 4, "bf16", seed=3)
    W = L.W_down.copy()
    W[3, 5, 7] = 1.0e5   # bf16-representable, past 65504
    big = dataclasses.replace(L, W_down=W)
    with pytest.raises(dm.DecoError) as ei:
        dm.Layer(**layer_tensors(big), max_tokens=16, eps=L.eps)
    assert ei.value.status == dm.DECO_ERR_UNSUPPORTED
    W = L.W_down.copy()
    W[0, 0, 0] = np.nan
    with pytest.raises(dm.DecoError) as ei:
        dm.Layer(**layer_tensors(dataclasses.replace(L, W_down=W)), max_tokens=16, eps=L.eps)
    assert ei.value.status == dm.DECO_ERR_UNSUPPORTED
    # just inside the range: accepted
    W = L.W_down.copy()
    W[3, 5, 7] = 65280.0   # the largest bf16 value within the fp16 range
    ok = dm.Layer(**layer_tensors(dataclasses.replace(L, W_down=W)), max_tokens=16, eps=L.eps)
    ok.free()
    # fp32 layers have no fp16 operand
    Lf = make_custom(128, 8, 32, 64, 4, "f32", seed=3)
    W = Lf.W_down.copy()
    W[3, 5, 7] = 1.0e5
    f = dm.Layer(**layer_tensors(dataclasses.replace(Lf, W_down=W)), max_tokens=16, eps=Lf.eps)
    f.free()


def test_norm_input_past_half_fp16_range_refused_with_the_mean_term():
    """The decode path multiplies x by the folded NormSiLU input W_up[e] - Wbar
    in fp16: |W_up - Wbar| <= 2 max |W_up|, so bf16 layers with the mean term
    refuse max |W_up| > 32752; the mean-term ablation (plain W_up) and fp32
    layers accept it."""
    L = make_custom(128, 8, 32, 64, 4, "bf16", seed=3)
    W = L.W_up.copy()
    W[2, 9, 4] = 4.0e4   # bf16-representable, past 32752
    big = dataclasses.replace(L, W_up=W)
    with pytest.raises(dm.DecoError) as ei:
        dm.Layer(**layer_tensors(big), max_tokens=16, eps=L.eps)
    assert ei.value.status == dm.DECO_ERR_UNSUPPORTED
    W = L.W_up.copy()
    W[2, 9, 4] = 32640.0   # the largest bf16 value within the limit
    ok = dm.Layer(**layer_tensors(dataclasses.replace(L, W_up=W)), max_tokens=16, eps=L.eps)
    ok.free()
    nm = dm.Layer(**layer_tensors(big), max_tokens=16, eps=L.eps, normsilu_mean=False)
    nm.free()
    Lf = make_custom(128, 8, 32, 64, 4, "f32", seed=3)
    W = Lf.W_up.copy()
    W[2, 9, 4] = 4.0e4
    f = dm.Layer(**layer_tensors(dataclasses.replace(Lf, W_up=W)), max_tokens=16, eps=Lf.eps)
    f.free()


def test_x_past_fp16_range_raises_the_flag_on_the_decode_path():
    """x enters the decode path's NormSiLU-input product converted to fp16: a
    token value past 65504 raises error bit 5 instead of an inf product."""
    L = make_layer(2, T=8)
    x = L.x.copy()
    x[3, 100] = 1.0e5
    big = L.with_x(x)
    layer = dm.Layer(**layer_tensors(big), max_tokens=16, eps=L.eps)
    layer.error_flags()
    layer(x_tensor(big), path=DEC)
    torch.cuda.synchronize()
    flags = layer.error_flags()
    _say(f"x = 1e5 decode: flags {flags}")
    assert flags & RANGE_BIT
    # in range: no flag, and the result matches the oracle
    layer(x_tensor(L), path=DEC)
    torch.cuda.synchronize()
    assert layer.error_flags() == 0
    layer.free()
