"""Python binding of libdeco_moe.so: the MI355X DECO sparse-MoE FFN layer.

Argument marshalling only: every step of the forward pass runs in the HIP
kernels of the library.  torch provides device memory and streams.  There is
no fallback: if the library is missing the import of `load_library()` fails
loudly (build it with ``python -m sparse_moe_relu_amd.build``).
"""
from __future__ import annotations

import ctypes
import os

# torch first: its HIP runtime (soname libamdhip64.so.7) must be the one the
# library binds to, so tensors and kernels share one runtime.
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# the in-tree build; load_library(path) before any other call binds another
# build instead (the first load wins)
LIB_PATH = os.path.join(_PKG, "libdeco_moe.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "deco_moe.h")

DECO_OK = 0
DECO_ERR_INVALID_ARG = -1
DECO_ERR_UNSUPPORTED = -2
DECO_ERR_OUT_OF_MEMORY = -3
DECO_ERR_HIP = -4
DECO_DT_BF16 = 0
DECO_DT_F32 = 1
DECO_PATH_AUTO = 0
DECO_PATH_DECODE = 1
DECO_PATH_PREFILL = 2
DECO_PATH_PREFILL_PAIRS = 3
DECO_PATH_PREFILL_TOKEN = 4
DECO_PATH_PREFILL_FUSED = 5
DECODE_MAX_T = 16
DECO_NORMSILU_NO_MEAN = 1
DECO_NORMSILU_NO_RMS = 2

EXPORTS = ("deco_moe_check_config", "deco_moe_load_weights", "deco_moe_load_weights_gated", "deco_moe_forward",
           "deco_moe_forward_path", "deco_moe_forward_decode_noalloc", "deco_moe_decode_noalloc_bytes",
           "deco_moe_copy_routing", "deco_moe_copy_mean_up",
           "deco_moe_free", "deco_moe_status_string", "deco_moe_read_error_flags", "deco_moe_timing_enable",
           "deco_moe_timing_reset", "deco_moe_timing_read", "deco_moe_backward",
           "deco_moe_sparsity_coef_update")


class DecoConfig(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("d_ff", ctypes.c_int32), ("d_ff_shared", ctypes.c_int32),
                ("max_tokens", ctypes.c_int32), ("dtype", ctypes.c_int),
                ("rms_eps", ctypes.c_float), ("top_k", ctypes.c_int32), ("backward", ctypes.c_int32),
                ("normsilu", ctypes.c_int32), ("scalar_lambda", ctypes.c_int32), ("shared_rms", ctypes.c_int32),
                ("shared_workspace", ctypes.c_int32)]


class DecoGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("dx", "dW_r", "db_r", "dlambda", "dW_up", "dW_down", "dWs_up",
                                                 "dWs_down", "n_active_pairs")]


class DecoError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load (once) and type the C ABI.  Raises if the library is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libdeco_moe.so not found at {path}; build it with "
                           "`python -m sparse_moe_relu_amd.build` (no fallback path exists)")
    lib = ctypes.CDLL(path)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.deco_moe_check_config.argtypes = [ctypes.POINTER(DecoConfig)]
    lib.deco_moe_check_config.restype = i32
    lib.deco_moe_load_weights.argtypes = [ctypes.POINTER(DecoConfig), vp, vp, vp, vp, vp, vp, vp, vp,
                                          ctypes.POINTER(vp)]
    lib.deco_moe_load_weights.restype = i32
    lib.deco_moe_load_weights_gated.argtypes = [ctypes.POINTER(DecoConfig), vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                                ctypes.POINTER(vp)]
    lib.deco_moe_load_weights_gated.restype = i32
    lib.deco_moe_forward.argtypes = [vp, vp, i64, vp, vp]
    lib.deco_moe_forward.restype = i32
    lib.deco_moe_forward_path.argtypes = [vp, vp, i64, vp, vp, i32]
    lib.deco_moe_forward_path.restype = i32
    lib.deco_moe_forward_decode_noalloc.argtypes = [vp, vp, i64, vp, vp]
    lib.deco_moe_forward_decode_noalloc.restype = i32
    lib.deco_moe_decode_noalloc_bytes.argtypes = [vp]
    lib.deco_moe_decode_noalloc_bytes.restype = i64
    lib.deco_moe_copy_routing.argtypes = [vp, i64, vp, vp, vp]
    lib.deco_moe_copy_routing.restype = i32
    lib.deco_moe_copy_mean_up.argtypes = [vp, vp, vp]
    lib.deco_moe_copy_mean_up.restype = i32
    lib.deco_moe_read_error_flags.argtypes = [vp, ctypes.POINTER(ctypes.c_uint32)]
    lib.deco_moe_read_error_flags.restype = i32
    lib.deco_moe_free.argtypes = [vp]
    lib.deco_moe_free.restype = None
    lib.deco_moe_status_string.argtypes = [i32]
    lib.deco_moe_status_string.restype = ctypes.c_char_p
    lib.deco_moe_timing_enable.argtypes = [i32]
    lib.deco_moe_timing_enable.restype = i32
    lib.deco_moe_timing_reset.argtypes = []
    lib.deco_moe_timing_reset.restype = i32
    lib.deco_moe_timing_read.argtypes = [i32, ctypes.POINTER(ctypes.c_char_p),
                                         ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
    lib.deco_moe_timing_read.restype = i32
    lib.deco_moe_backward.argtypes = [vp, vp, vp, i64, ctypes.c_float, ctypes.POINTER(DecoGrads), vp]
    lib.deco_moe_backward.restype = i32
    lib.deco_moe_sparsity_coef_update.argtypes = [ctypes.c_float] * 4
    lib.deco_moe_sparsity_coef_update.restype = ctypes.c_float
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().deco_moe_status_string(int(status)).decode()


def make_config(d: int, E: int, F: int, Fs: int, max_tokens: int, dtype: str = "bf16",
                eps: float = 1e-6, top_k: int = 0, backward: bool = False, *, normsilu_mean: bool = True,
                normsilu_rms: bool = True, scalar_lambda: bool = False, shared_rms: bool = False,
                shared_workspace: bool = False) -> DecoConfig:
    """top_k = 0: DECO's ReLU routing; 1..E: the TopK routing variant.
    backward: keep what deco_moe_backward needs.  The last four are the
    ablation switches of deco_moe_config; shared_workspace: one prefill/backward
    workspace per device for every layer that sets it."""
    dt = {"bf16": DECO_DT_BF16, "f32": DECO_DT_F32}[dtype]
    ns = (0 if normsilu_mean else DECO_NORMSILU_NO_MEAN) | (0 if normsilu_rms else DECO_NORMSILU_NO_RMS)
    return DecoConfig(d, E, F, Fs, max_tokens, dt, eps, top_k, 1 if backward else 0, ns,
                      1 if scalar_lambda else 0, 1 if shared_rms else 0, 1 if shared_workspace else 0)


def sparsity_coef_update(coef: float, active_ratio: float, target_ratio: float, factor: float = 1.002) -> float:
    """One step of the adaptive sparsity coefficient (deco_moe_sparsity_coef_update)."""
    return float(load_library().deco_moe_sparsity_coef_update(coef, active_ratio, target_ratio, factor))


def check_config(cfg: DecoConfig) -> int:
    return int(load_library().deco_moe_check_config(ctypes.byref(cfg)))


def _stream_handle(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


_TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


class Layer:
    """One DECO MoE FFN layer whose weights live in library-owned device buffers.

    Weights are device tensors of the layer dtype (b_r and lam: float32):
    W_r [d,E], b_r [E], lam [E], W_up [E,d,F], W_down [E,F,d], Ws_up [d,Fs],
    Ws_down [Fs,d].  They are packed at construction and may be freed after.
    W_gate [E,d,F] (optional) selects the gated-expert variant
    (deco_moe_load_weights_gated): NormSiLU acts on x.W_gate[e] and the
    result multiplies x.W_up[e].
    """

    def __init__(self, W_r, b_r, lam, W_up, W_down, Ws_up, Ws_down, *, max_tokens: int,
                 eps: float = 1e-6, top_k: int = 0, W_gate=None, backward: bool = False,
                 normsilu_mean: bool = True, normsilu_rms: bool = True, scalar_lambda: bool = False,
                 shared_rms: bool = False, shared_workspace: bool = False, stream=None):
        lib = load_library()
        dtype = {torch.bfloat16: "bf16", torch.float32: "f32"}.get(W_up.dtype)
        if dtype is None:
            raise TypeError(f"unsupported weight dtype {W_up.dtype}")
        E, d, F = W_up.shape
        Fs = Ws_up.shape[1]
        shapes = {"W_r": (W_r, (d, E)), "W_up": (W_up, (E, d, F)), "W_down": (W_down, (E, F, d)),
                  "Ws_up": (Ws_up, (d, Fs)), "Ws_down": (Ws_down, (Fs, d))}
        if W_gate is not None:
            shapes["W_gate"] = (W_gate, (E, d, F))
        for name, (t, shp) in shapes.items():
            if tuple(t.shape) != shp or t.dtype != W_up.dtype or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"{name}: expected contiguous device {shp} {W_up.dtype}, got "
                                 f"{tuple(t.shape)} {t.dtype} {t.device}")
        for name, t in (("b_r", b_r), ("lam", lam)):
            if tuple(t.shape) != (E,) or t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"{name}: expected contiguous device float32 ({E},)")
        self.cfg = make_config(d, E, F, Fs, max_tokens, dtype, eps, top_k, backward, normsilu_mean=normsilu_mean,
                               normsilu_rms=normsilu_rms, scalar_lambda=scalar_lambda, shared_rms=shared_rms,
                               shared_workspace=shared_workspace)
        self.top_k = top_k
        self.gated = W_gate is not None
        self.d, self.E, self.F, self.Fs, self.dtype = d, E, F, Fs, dtype
        self.max_tokens = max_tokens
        self.W = (E + 63) // 64
        h = ctypes.c_void_p()
        if W_gate is None:
            st = lib.deco_moe_load_weights(ctypes.byref(self.cfg), W_r.data_ptr(), b_r.data_ptr(),
                                           lam.data_ptr(), W_up.data_ptr(), W_down.data_ptr(),
                                           Ws_up.data_ptr(), Ws_down.data_ptr(), _stream_handle(stream),
                                           ctypes.byref(h))
            what = "deco_moe_load_weights"
        else:
            st = lib.deco_moe_load_weights_gated(ctypes.byref(self.cfg), W_r.data_ptr(), b_r.data_ptr(),
                                                 lam.data_ptr(), W_gate.data_ptr(), W_up.data_ptr(),
                                                 W_down.data_ptr(), Ws_up.data_ptr(), Ws_down.data_ptr(),
                                                 _stream_handle(stream), ctypes.byref(h))
            what = "deco_moe_load_weights_gated"
        if st != DECO_OK:
            raise DecoError(st, what)
        self._h = h

    @property
    def handle(self) -> ctypes.c_void_p:
        if self._h is None:
            raise RuntimeError("layer was freed")
        return self._h

    def forward(self, x: torch.Tensor, out: torch.Tensor | None = None, *, path: int = DECO_PATH_AUTO,
                stream=None) -> torch.Tensor:
        if x.dim() != 2 or x.shape[1] != self.d or x.dtype != _TORCH_DT[self.dtype] or not x.is_cuda \
                or not x.is_contiguous():
            raise ValueError(f"x: expected contiguous device [T,{self.d}] {_TORCH_DT[self.dtype]}")
        T = x.shape[0]
        if out is None:
            out = torch.empty_like(x)
        elif (tuple(out.shape) != tuple(x.shape) or out.dtype != x.dtype or out.device != x.device
              or not out.is_contiguous()):
            # the library writes T*d elements at out's address: a smaller or
            # differently typed buffer would be overrun
            raise ValueError(f"out: expected contiguous {tuple(x.shape)} {x.dtype} on {x.device}")
        st = load_library().deco_moe_forward_path(self.handle, x.data_ptr(), T, out.data_ptr(),
                                                  _stream_handle(stream), int(path))
        if st != DECO_OK:
            raise DecoError(st, "deco_moe_forward")
        return out

    __call__ = forward

    def forward_decode_noalloc(self, x: torch.Tensor, out: torch.Tensor, *, stream=None) -> torch.Tensor:
        """deco_moe_forward_decode_noalloc: the decode path with its scratch in
        the library's static device array (allocates nothing; `out` is
        required)."""
        if x.dim() != 2 or x.shape[1] != self.d or x.dtype != _TORCH_DT[self.dtype] or not x.is_cuda \
                or not x.is_contiguous():
            raise ValueError(f"x: expected contiguous device [T,{self.d}] {_TORCH_DT[self.dtype]}")
        if (tuple(out.shape) != tuple(x.shape) or out.dtype != x.dtype or out.device != x.device
                or not out.is_contiguous()):
            raise ValueError(f"out: expected contiguous {tuple(x.shape)} {x.dtype} on {x.device}")
        st = load_library().deco_moe_forward_decode_noalloc(self.handle, x.data_ptr(), x.shape[0],
                                                            out.data_ptr(), _stream_handle(stream))
        if st != DECO_OK:
            raise DecoError(st, "deco_moe_forward_decode_noalloc")
        return out

    def decode_noalloc_bytes(self) -> int:
        return int(load_library().deco_moe_decode_noalloc_bytes(self.handle))

    def backward(self, x: torch.Tensor, dout: torch.Tensor, *, reg_coef: float = 0.0, stream=None) -> dict:
        """Gradients of sum(dout * layer(x)) + reg_coef * mean router entropy
        (deco_moe_backward): float32 device tensors dx, dW_r, db_r, dlambda,
        dW_up, dW_down, dWs_up, dWs_down, and n_active_pairs (int32 [1])."""
        if x.dim() != 2:
            raise ValueError(f"x: expected contiguous device [T,{self.d}] {_TORCH_DT[self.dtype]}")
        T = x.shape[0]
        for name, t in (("x", x), ("dout", dout)):
            if t.dim() != 2 or tuple(t.shape) != (T, self.d) or t.dtype != _TORCH_DT[self.dtype] or not t.is_cuda \
                    or not t.is_contiguous():
                raise ValueError(f"{name}: expected contiguous device [T,{self.d}] {_TORCH_DT[self.dtype]}")
        f32 = dict(dtype=torch.float32, device=x.device)
        d, E, F, Fs = self.d, self.E, self.F, self.Fs
        g = dict(dx=torch.empty((T, d), **f32), dW_r=torch.empty((d, E), **f32), db_r=torch.empty(E, **f32),
                 dlambda=torch.empty(E, **f32), dW_up=torch.empty((E, d, F), **f32),
                 dW_down=torch.empty((E, F, d), **f32), dWs_up=torch.empty((d, Fs), **f32),
                 dWs_down=torch.empty((Fs, d), **f32),
                 n_active_pairs=torch.empty(1, dtype=torch.int32, device=x.device))
        gs = DecoGrads(*[g[n].data_ptr() for n, _ in DecoGrads._fields_])
        st = load_library().deco_moe_backward(self.handle, x.data_ptr(), dout.data_ptr(), T, float(reg_coef),
                                              ctypes.byref(gs), _stream_handle(stream))
        if st != DECO_OK:
            raise DecoError(st, "deco_moe_backward")
        return g

    def routing(self, T: int, stream=None):
        """(mask [T, ceil(E/64)] int64 bit words, logits [T, E] float32) of the last forward."""
        mask = torch.empty((T, self.W), dtype=torch.int64, device="cuda")
        logits = torch.empty((T, self.E), dtype=torch.float32, device="cuda")
        st = load_library().deco_moe_copy_routing(self.handle, T, mask.data_ptr(), logits.data_ptr(),
                                                  _stream_handle(stream))
        if st != DECO_OK:
            raise DecoError(st, "deco_moe_copy_routing")
        return mask, logits

    def active_mask(self, T: int, stream=None) -> torch.Tensor:
        """Boolean [T, E] active-expert mask of the last forward (on the host)."""
        mask, _ = self.routing(T, stream)
        words = mask.cpu().numpy().view("uint64")
        import numpy as np
        bits = np.unpackbits(words.view(np.uint8).reshape(T, self.W, 8), axis=2, bitorder="little")
        return torch.from_numpy(bits.reshape(T, self.W * 64)[:, :self.E].astype(bool))

    def mean_up(self, stream=None) -> torch.Tensor:
        wbar = torch.empty((self.d, self.F), dtype=torch.float32, device="cuda")
        st = load_library().deco_moe_copy_mean_up(self.handle, wbar.data_ptr(), _stream_handle(stream))
        if st != DECO_OK:
            raise DecoError(st, "deco_moe_copy_mean_up")
        return wbar

    def error_flags(self) -> int:
        """Device-side health flags (bit 0: a decode wait timed out); clears them."""
        f = ctypes.c_uint32()
        st = load_library().deco_moe_read_error_flags(self.handle, ctypes.byref(f))
        if st != DECO_OK:
            raise DecoError(st, "deco_moe_read_error_flags")
        return int(f.value)

    def free(self):
        if getattr(self, "_h", None) is not None:
            load_library().deco_moe_free(self._h)
            self._h = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def timing_enable(on: bool = True):
    load_library().deco_moe_timing_enable(1 if on else 0)


def timing_reset():
    load_library().deco_moe_timing_reset()


def timing_read() -> dict:
    """{kernel name: (total_ms, launches)} accumulated since the last reset."""
    lib = load_library()
    out = {}
    i = 0
    while True:
        name = ctypes.c_char_p()
        ms = ctypes.c_double()
        n = ctypes.c_int64()
        if lib.deco_moe_timing_read(i, ctypes.byref(name), ctypes.byref(ms), ctypes.byref(n)) != DECO_OK:
            break
        if n.value:
            out[name.value.decode()] = (ms.value, n.value)
        i += 1
    return out
