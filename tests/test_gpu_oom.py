"""Forced device-allocation failure at load.

A layer whose max_tokens makes its prefill workspace larger than the device
(1 Mi tokens x 257 pair slots x d = 2048 x 2 bytes, about 1.1 TB, against
288 GB of HBM) must fail with DECO_ERR_OUT_OF_MEMORY after its weight and
routing buffers were already allocated, release them (device memory back
where it was), and leave the library usable: a layer of ordinary size loads
and matches the fp64 oracle afterwards.  Both workspace modes: owned by the
layer, and the per-device shared workspace.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_moe_relu_amd as dm
from synthetic import make_custom
from synthetic.device import layer_tensors, x_tensor

pytestmark = pytest.mark.gpu


def test_forced_out_of_memory_releases_and_recovers():
    dm.load_library()
    L = make_custom(2048, 256, 32, 32, 16, "bf16", seed=3)
    W = layer_tensors(L)
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    for shared_ws in (False, True):
        print(f"[oom] load with max_tokens = 2^20, shared_workspace={shared_ws}", flush=True)
        with pytest.raises(dm.DecoError) as ei:
            dm.Layer(**W, max_tokens=1 << 20, eps=L.eps, shared_workspace=shared_ws)
        assert ei.value.status == dm.DECO_ERR_OUT_OF_MEMORY
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert abs(free1 - free0) < (64 << 20), (free0, free1)

    # the library still works: an ordinary layer of the same weights
    ref = oracle.forward(L.x, **L.weights(), eps=L.eps)
    for shared_ws in (False, True):
        layer = dm.Layer(**W, max_tokens=L.T, eps=L.eps, shared_workspace=shared_ws)
        for T in (8, 16):
            out = layer(x_tensor(L)[:T].contiguous(), path=dm.DECO_PATH_PREFILL if T == 16 else dm.DECO_PATH_DECODE)
            torch.cuda.synchronize()
            got = out.float().cpu().numpy().astype(np.float64)
            want = ref.out[:T]
            rms = float(np.sqrt(np.mean(want ** 2)))
            _, ex = np.frexp(np.abs(got))
            half_ulp = np.where(got == 0, 0.0, np.ldexp(1.0, ex - 9))
            excess = float(np.max(np.abs(got - want) - half_ulp))
            assert excess <= 2e-2 * rms, (shared_ws, T, excess / rms)
        layer.free()
