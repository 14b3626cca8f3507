"""GPU parity of the small-batch split of the prefill expert tiles against the
fp64 oracle (same bar as test_gpu_parity.py).

Small batches of a non-gated layer run each 64-row expert tile as k parts of
the up-projection (k_pre_expert_kpart: fp32 sums per pair slot) and column
blocks of the down-projection (k_pre_expert: the parts added in order, then
NormSiLU and the block's W_down panels).  Cases: one, two and four k parts;
one to eight column blocks; 16- to 256-column experts; experts with several
64-row tiles; ragged batches; the largest split batch of the d = 4096 layer
and the first batches past it; no active expert; the NormSiLU ablations; TopK
routing; fp32 layers; a bitwise repeat.  Each case also checks from the
per-kernel launch counts that the split ran (or, past its range, did not).
"""
import numpy as np
import pytest
import torch

import oracle
from synthetic import make_custom, make_layer
from synthetic.device import layer_tensors, x_tensor
from test_gpu_ablation import check as check_ablation
from test_gpu_parity import _layer_obj, _subset, check
from test_gpu_topk import run_topk

pytestmark = pytest.mark.gpu

import sparse_moe_relu_amd as dm

PRE = dm.DECO_PATH_PREFILL
KPART = "k_pre_expert_kpart"


def _run(L, ref, layer, *, T=None, label="", split=True, fn=None):
    dm.timing_enable(True)
    dm.timing_reset()
    try:
        got = fn() if fn else check(L, ref, layer, PRE, T=T, label=label)
        times = dm.timing_read()
    finally:
        dm.timing_enable(False)
    ran = KPART in times
    assert ran == split, f"{label}: split {'expected' if split else 'not expected'}, kernels {sorted(times)}"
    return got


@pytest.mark.parametrize("shape", [
    (2048, 56, 128, 1024, "bf16", 0.2),   # the d = 2048 layer's shape: 4 k parts, up to 8 column blocks
    (256, 24, 128, 128, "bf16", 0.3),     # one k part, four stages of W_down
    (512, 12, 64, 96, "bf16", 0.5),       # two k parts; experts with several 64-row tiles
    (1024, 40, 32, 64, "bf16", 0.3),      # 32-column experts
    (1024, 8, 256, 64, "bf16", 0.3),      # 256-column experts (two-panel W_down stages)
    (128, 3, 64, 160, "f32", 0.3),        # fp32
])
@pytest.mark.parametrize("T", [1, 77, 300])
def test_split_shapes(shape, T):
    d, E, F, Fs, dt, ratio = shape
    L = make_custom(d, E, F, Fs, T, dt, seed=9, ratio=ratio)
    ref = oracle.forward(L.x, **L.weights(), eps=L.eps)
    layer = _layer_obj(L, 320)
    got = _run(L, ref, layer, label=f"split{shape}")
    again = layer(x_tensor(L), path=PRE).float().cpu().numpy().astype(np.float64)
    assert np.array_equal(got, again), "the split prefill is not repeatable bitwise"
    layer.free()


def test_split_bounds_on_the_d4096_layer():
    # the split runs while its k-part units (4 per estimated 64-row expert
    # tile, a quarter of the batch per expert) fit the persistent grid in one
    # pass: on a 256-CU device (512 workgroups) up to 259 tokens of the
    # d = 4096 layer, not from 260 on
    L = make_layer(4, T=512)
    ref = oracle.forward(L.x, **L.weights(), eps=L.eps)
    layer = _layer_obj(L, 2048)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    _run(L, _subset(ref, 256), layer, T=256, label="c4-256")
    if cus == 256:
        _run(L, _subset(ref, 259), layer, T=259, label="c4-259")
        _run(L, _subset(ref, 260), layer, T=260, label="c4-260", split=False)
        _run(L, ref, layer, T=512, label="c4-512", split=False)
    layer.free()


def test_split_no_active_expert():
    L = make_custom(256, 24, 128, 128, 200, "bf16", seed=4)
    L.b_r = np.full_like(L.b_r, -1e4)
    ref = oracle.forward(L.x, **L.weights(), eps=L.eps)
    assert not ref.active.any()
    layer = _layer_obj(L, 256)
    # no expert tile: the k-part kernel has no units (it still launches)
    _run(L, ref, layer, label="split-none-active")
    layer.free()


@pytest.mark.parametrize("flags", [dict(normsilu_mean=False), dict(normsilu_rms=False),
                                   dict(normsilu_mean=False, scalar_lambda=True, shared_rms=True)])
def test_split_ablations(flags):
    L = make_custom(512, 24, 128, 256, 150, "bf16", seed=11, ratio=0.3)
    layer = dm.Layer(**layer_tensors(L), max_tokens=256, eps=L.eps, **flags)
    _run(L, None, layer, fn=lambda: check_ablation(L, layer, PRE, flags, label=f"split-{flags}"))
    layer.free()


def test_split_topk():
    L = make_custom(1024, 40, 128, 256, 130, "bf16", seed=12, ratio=0.2)
    layer = dm.Layer(**layer_tensors(L), max_tokens=256, eps=L.eps, top_k=6)
    _run(L, None, layer, fn=lambda: run_topk(L, 6, layer, PRE, label="split-topk"))
    layer.free()
