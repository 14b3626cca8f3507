"""GPU parity of the two prefill down-projection variants, each forced through
deco_moe_forward_path, against the fp64 oracle (same bar as
test_gpu_parity.py).

DECO_PATH_PREFILL_TOKEN: the expert kernel writes each pair's activation row
and k_pre_dc forms out = shared term + the token's experts in ascending order
per (256-token, 128-column) block.  Cases: fp32 and bf16 layers, one, two and
four k-blocks per expert, one to four mask words, ragged token and column
blocks, a wave with more than 32 rows on one expert (the rows past the
prefetched blocks), no active expert at all, one expert, gated experts, and a
bitwise repeat.  DECO_PATH_PREFILL_PAIRS: the per-pair output rows and the
combine kernel, at full size (what DECO_PATH_PREFILL runs).
DECO_PATH_PREFILL_FUSED: the shared expert's down-projection and the combine
in one kernel (8-, 4- and 2-panel tiles by batch size), on the same shapes,
with the split expert tiles of small batches, gated experts, no active
expert, and at full size.
"""
import numpy as np
import pytest
import torch

import oracle
from synthetic import make_custom, make_layer
from synthetic.device import layer_tensors, x_tensor
from test_gpu_parity import _layer_obj, _subset, check

pytestmark = pytest.mark.gpu

import sparse_moe_relu_amd as dm

TOKEN, PAIRS, FUSED = dm.DECO_PATH_PREFILL_TOKEN, dm.DECO_PATH_PREFILL_PAIRS, dm.DECO_PATH_PREFILL_FUSED


def test_token_variant_c1_fp32():
    L = make_layer(1)
    ref = oracle.forward(L.x, **L.weights(), eps=L.eps)
    layer = _layer_obj(L, 64)
    check(L, ref, layer, TOKEN, label="c1-token")
    layer.free()


@pytest.mark.parametrize("shape", [
    (256, 24, 128, 128, "bf16", 0.2),   # four k-blocks per expert
    (192, 70, 64, 96, "bf16", 0.3),     # two k-blocks, two mask words, a partial column block, odd Fs k-blocks
    (128, 5, 32, 64, "bf16", 0.3),      # one k-block
    (128, 3, 64, 160, "f32", 0.3),      # fp32, four k-blocks
    (128, 256, 128, 64, "bf16", 0.7),   # four mask words; up to ~64 rows of a wave on one expert
    (64, 1, 32, 32, "bf16", 0.3),       # one expert
])
@pytest.mark.parametrize("T", [1, 77, 300, 513])
def test_token_variant_shapes(shape, T):
    d, E, F, Fs, dt, ratio = shape
    L = make_custom(d, E, F, Fs, T, dt, seed=5, ratio=ratio)
    ref = oracle.forward(L.x, **L.weights(), eps=L.eps)
    layer = _layer_obj(L, 520)
    got = check(L, ref, layer, TOKEN, label=f"token{shape}")
    again = layer(x_tensor(L), path=TOKEN).float().cpu().numpy().astype(np.float64)
    assert np.array_equal(got, again), "token-major prefill is not repeatable bitwise"
    layer.free()


def test_token_variant_no_active_expert():
    L = make_custom(256, 24, 128, 128, 300, "bf16", seed=4)
    L.b_r = np.full_like(L.b_r, -1e4)
    ref = oracle.forward(L.x, **L.weights(), eps=L.eps)
    assert not ref.active.any()
    layer = _layer_obj(L, 300)
    check(L, ref, layer, TOKEN, label="token-none-active")
    layer.free()


def test_token_variant_gated():
    L = make_custom(256, 24, 128, 128, 300, "bf16", seed=6, ratio=0.3, gated=True)
    ref = oracle.forward(L.x, **L.weights(), eps=L.eps)
    layer = dm.Layer(**layer_tensors(L), max_tokens=300, eps=L.eps)
    check(L, ref, layer, TOKEN, label="token-gated")
    layer.free()


def test_token_variant_needs_at_most_four_k_blocks():
    L = make_custom(128, 4, 256, 64, 8, "bf16", seed=2)
    layer = _layer_obj(L, 16)
    x = x_tensor(L)
    out = torch.empty_like(x)
    lib = dm.load_library()
    st = lib.deco_moe_forward_path(layer.handle, x.data_ptr(), L.T, out.data_ptr(), None, TOKEN)
    assert st == dm.DECO_ERR_UNSUPPORTED
    assert lib.deco_moe_forward_path(layer.handle, x.data_ptr(), L.T, out.data_ptr(), None, 6) == \
        dm.DECO_ERR_INVALID_ARG
    layer.free()


def test_all_variants_full_size_c3():
    L = make_layer(3)
    ref = oracle.forward(L.x, **L.weights(), eps=L.eps)
    layer = _layer_obj(L, L.T)
    a = check(L, ref, layer, PAIRS, label="c3-pairs")
    check(L, ref, layer, TOKEN, label="c3-token")
    check(L, ref, layer, FUSED, label="c3-fused")
    c = check(L, ref, layer, dm.DECO_PATH_PREFILL, label="c3-prefill")
    assert np.array_equal(a, c), "DECO_PATH_PREFILL runs the pairs variant"
    for T in (257, 4001):
        check(L, _subset(ref, T), layer, PAIRS, T=T, label="c3-pairs-ragged")
        check(L, _subset(ref, T), layer, TOKEN, T=T, label="c3-token-ragged")
        check(L, _subset(ref, T), layer, FUSED, T=T, label="c3-fused-ragged")
    layer.free()


def test_fused_variant_c1_fp32():
    L = make_layer(1)
    ref = oracle.forward(L.x, **L.weights(), eps=L.eps)
    layer = _layer_obj(L, 64)
    check(L, ref, layer, FUSED, label="c1-fused")
    layer.free()


@pytest.mark.parametrize("shape", [
    (256, 24, 128, 128, "bf16", 0.2),
    (192, 70, 64, 96, "bf16", 0.3),     # a partial 8-, 4- and 2-panel column tile (d = 12 panels)
    (1024, 40, 32, 64, "bf16", 0.3),
    (128, 3, 64, 160, "f32", 0.3),
])
@pytest.mark.parametrize("T", [1, 77, 300, 1100])
def test_fused_variant_shapes(shape, T):
    d, E, F, Fs, dt, ratio = shape
    L = make_custom(d, E, F, Fs, T, dt, seed=7, ratio=ratio)
    ref = oracle.forward(L.x, **L.weights(), eps=L.eps)
    layer = _layer_obj(L, 1100)
    got = check(L, ref, layer, FUSED, label=f"fused{shape}")
    again = layer(x_tensor(L), path=FUSED).float().cpu().numpy().astype(np.float64)
    assert np.array_equal(got, again), "the fused prefill is not repeatable bitwise"
    layer.free()


def test_fused_variant_no_active_expert_and_gated():
    L = make_custom(256, 24, 128, 128, 300, "bf16", seed=4)
    L.b_r = np.full_like(L.b_r, -1e4)
    ref = oracle.forward(L.x, **L.weights(), eps=L.eps)
    layer = _layer_obj(L, 300)
    check(L, ref, layer, FUSED, label="fused-none-active")
    layer.free()
    L = make_custom(256, 24, 128, 128, 300, "bf16", seed=6, ratio=0.3, gated=True)
    ref = oracle.forward(L.x, **L.weights(), eps=L.eps)
    layer = dm.Layer(**layer_tensors(L), max_tokens=300, eps=L.eps)
    check(L, ref, layer, FUSED, label="fused-gated")
    layer.free()
