"""Move synthetic layer inputs to torch device tensors (no arithmetic beyond exact casts)."""
from __future__ import annotations

import numpy as np
import torch

from .gen import LayerInputs

_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def to_tensor(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """float64 values already representable in `dtype` -> exact device tensor."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device=device).to(_DT[dtype]).contiguous()


def layer_tensors(L: LayerInputs, device="cuda") -> dict:
    """Weights of `L` as device tensors (b_r, lam as float32), ready for the binding."""
    w = dict(W_r=to_tensor(L.W_r, L.dtype, device), b_r=to_tensor(L.b_r, "f32", device),
             lam=to_tensor(L.lam, "f32", device), W_up=to_tensor(L.W_up, L.dtype, device),
             W_down=to_tensor(L.W_down, L.dtype, device), Ws_up=to_tensor(L.Ws_up, L.dtype, device),
             Ws_down=to_tensor(L.Ws_down, L.dtype, device))
    if L.W_gate is not None:
        w["W_gate"] = to_tensor(L.W_gate, L.dtype, device)
    return w


def x_tensor(L: LayerInputs, device="cuda") -> torch.Tensor:
    return to_tensor(L.x, L.dtype, device)
