"""The allocation-free decode entry point (deco_moe_forward_decode_noalloc),
called through the C ABI, against the regular decode path
(deco_moe_forward_path with DECO_PATH_DECODE): the same kernels, so the
outputs must agree bit for bit.  Two calls in a row per layer, the second
with a smaller T, and calls alternating between layers of different launch
shapes (they share the one static scratch array)."""
import numpy as np
import pytest
import torch

import sparse_moe_relu_amd as dm
from synthetic import make_custom, make_layer
from synthetic.device import layer_tensors, x_tensor

pytestmark = pytest.mark.gpu

LIMIT = 4 << 20


def _say(msg):
    print(f"[noalloc] {msg}", flush=True)


def _compare(layer, L, T, label):
    lib = dm.load_library()
    xs = x_tensor(L)[:T].contiguous()
    ref = torch.empty_like(xs)
    got = torch.full_like(xs, float("nan"))
    _say(f"{label} T={T} d={L.d} E={L.E} {L.dtype}")
    assert lib.deco_moe_forward_path(layer.handle, xs.data_ptr(), T, ref.data_ptr(), None,
                                     dm.DECO_PATH_DECODE) == dm.DECO_OK
    assert lib.deco_moe_forward_decode_noalloc(layer.handle, xs.data_ptr(), T, got.data_ptr(), None) == dm.DECO_OK
    torch.cuda.synchronize()
    ib = torch.int16 if xs.element_size() == 2 else torch.int32
    assert torch.equal(got.view(ib), ref.view(ib)), f"{label}: outputs differ"
    assert layer.error_flags() == 0


def test_noalloc_matches_decode_path():
    Lc2 = make_layer(2, T=16)
    Lc1 = make_layer(1)
    a = dm.Layer(**layer_tensors(Lc2), max_tokens=16, eps=Lc2.eps)
    b = dm.Layer(**layer_tensors(Lc1), max_tokens=16, eps=Lc1.eps)
    assert 0 < a.decode_noalloc_bytes() <= LIMIT and 0 < b.decode_noalloc_bytes() <= LIMIT
    _compare(a, Lc2, 16, "c2")
    _compare(a, Lc2, 5, "c2")          # smaller second call
    _compare(b, Lc1, 16, "c1")          # another layer, another grid, same scratch
    _compare(b, Lc1, 3, "c1")
    _compare(a, Lc2, 8, "c2 again")
    a.free()
    b.free()


def test_noalloc_topk_and_gated():
    L = make_layer(2, T=16)
    k = dm.Layer(**layer_tensors(L), max_tokens=16, eps=L.eps, top_k=11)
    _compare(k, L, 16, "c2 top-11")
    _compare(k, L, 7, "c2 top-11")
    k.free()
    Lg = make_custom(256, 24, 64, 128, 16, "bf16", seed=4, gated=True)
    g = dm.Layer(**layer_tensors(Lg), max_tokens=16, eps=Lg.eps)
    _compare(g, Lg, 16, "gated")
    _compare(g, Lg, 2, "gated")
    g.free()


def test_noalloc_rejects_oversized_and_bad_arguments():
    # fp32, 256 experts of d_ff 256, shared d_ff 16384: the activation rows
    # alone take 4 MiB + 1 MiB, past the array
    L = make_custom(64, 256, 256, 16384, 4, "f32", seed=1)
    layer = dm.Layer(**layer_tensors(L), max_tokens=16, eps=L.eps)
    assert layer.decode_noalloc_bytes() > LIMIT
    lib = dm.load_library()
    x = x_tensor(L)[:4].contiguous()
    out = torch.empty_like(x)
    assert lib.deco_moe_forward_decode_noalloc(layer.handle, x.data_ptr(), 4, out.data_ptr(), None) \
        == dm.DECO_ERR_UNSUPPORTED
    layer.free()
    Lc1 = make_layer(1)
    small = dm.Layer(**layer_tensors(Lc1), max_tokens=32, eps=Lc1.eps)
    x = x_tensor(Lc1)
    x17 = torch.cat([x, x[:1]]).contiguous()
    out = torch.empty_like(x17)
    assert lib.deco_moe_forward_decode_noalloc(small.handle, x17.data_ptr(), 17, out.data_ptr(), None) \
        == dm.DECO_ERR_INVALID_ARG   # past the decode path's T
    assert lib.deco_moe_forward_decode_noalloc(small.handle, x.data_ptr(), 0, out.data_ptr(), None) == dm.DECO_OK
    assert lib.deco_moe_decode_noalloc_bytes(None) == dm.DECO_ERR_INVALID_ARG
    small.free()
