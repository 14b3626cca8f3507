"""Layers sharing one prefill/backward workspace (deco_moe_config.shared_workspace):
their results equal those of layers with a workspace of their own, bit for
bit, also after the shared workspace grew for a larger layer (which re-points
the layers already loaded) and after a sharing layer is freed."""
import numpy as np
import pytest
import torch

from synthetic import make_custom
from synthetic.device import layer_tensors, x_tensor

pytestmark = pytest.mark.gpu

import sparse_moe_relu_amd as dm


def _say(msg):
    print(f"[ws] {msg}", flush=True)


def _run(layer, L, path, T=None):
    T = L.T if T is None else T
    out = layer(x_tensor(L)[:T].contiguous(), path=path)
    torch.cuda.synchronize()
    return out.clone()


def test_shared_workspace_matches_private():
    La = make_custom(256, 16, 64, 128, 300, "bf16", seed=21)
    Lb = make_custom(512, 24, 128, 256, 1000, "bf16", seed=22)
    a0 = dm.Layer(**layer_tensors(La), max_tokens=La.T, eps=La.eps)
    b0 = dm.Layer(**layer_tensors(Lb), max_tokens=Lb.T, eps=Lb.eps)
    a = dm.Layer(**layer_tensors(La), max_tokens=La.T, eps=La.eps, shared_workspace=True)
    ref_a = _run(a0, La, dm.DECO_PATH_PREFILL)
    assert torch.equal(_run(a, La, dm.DECO_PATH_PREFILL), ref_a)
    # a larger sharing layer: the shared workspace grows, `a` is re-pointed
    b = dm.Layer(**layer_tensors(Lb), max_tokens=Lb.T, eps=Lb.eps, shared_workspace=True)
    ref_b = _run(b0, Lb, dm.DECO_PATH_PREFILL)
    _say("prefill, two sharing layers, alternating")
    for _ in range(2):
        assert torch.equal(_run(b, Lb, dm.DECO_PATH_PREFILL), ref_b)
        assert torch.equal(_run(a, La, dm.DECO_PATH_PREFILL), ref_a)
        assert torch.equal(_run(a, La, dm.DECO_PATH_PREFILL, T=37), _run(a0, La, dm.DECO_PATH_PREFILL, T=37))
    # the decode path keeps its own state per layer
    assert torch.equal(_run(a, La, dm.DECO_PATH_DECODE, T=8), _run(a0, La, dm.DECO_PATH_DECODE, T=8))
    a.free()
    assert torch.equal(_run(b, Lb, dm.DECO_PATH_PREFILL), ref_b)
    b.free()
    # a new sharing layer after every sharer is gone
    c = dm.Layer(**layer_tensors(La), max_tokens=La.T, eps=La.eps, shared_workspace=True)
    assert torch.equal(_run(c, La, dm.DECO_PATH_PREFILL), ref_a)
    assert c.error_flags() == 0
    c.free()
    a0.free()
    b0.free()


def test_shared_workspace_backward_matches_private():
    L = make_custom(256, 16, 64, 128, 200, "bf16", seed=23)
    from synthetic import make_dout
    from synthetic.device import to_tensor
    dout = to_tensor(make_dout(L), L.dtype)
    p = dm.Layer(**layer_tensors(L), max_tokens=L.T, eps=L.eps, backward=True)
    s = dm.Layer(**layer_tensors(L), max_tokens=L.T, eps=L.eps, backward=True, shared_workspace=True)
    gp = p.backward(x_tensor(L), dout)
    gs = s.backward(x_tensor(L), dout)
    torch.cuda.synchronize()
    for k in gp:
        assert torch.equal(gp[k], gs[k]), k
    p.free()
    s.free()
