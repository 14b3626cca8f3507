"""Seeded generator for the five synthetic DECO layer workloads.

The DECO pages measure a trained model inside a decoding framework on a
speculative-decoding benchmark; neither the model nor the benchmark is
available, so synthetic layers with the distributions below stand in for them.

Recipe (shared by every workload):
  * numpy PCG64, ``SeedSequence(seed).spawn(8)`` giving independent streams in
    the fixed order x, W_r, W_up, W_down, Ws_up, Ws_down, lambda, bias-skew;
  * every value is drawn in float64 and cast ONCE, round-to-nearest-even, to
    the storage type (bf16 or fp32).  The returned float64 arrays hold exactly
    the values the GPU sees;
  * x ~ N(0, 1); W_r, W_up, Ws_up ~ N(0, 1/d); W_down ~ N(0, 1/F);
    Ws_down ~ N(0, 1/Fs)  (second argument = variance);
  * lambda_e = exp(N(0, 0.5)), or exp(0.8 N(0, 1)) for the d=4096 layer
    (heterogeneous expert output norms);
  * router bias b_e = -q * ||W_r[:, e]||_2 with q the standard-normal quantile
    of (1 - ratio): for x ~ N(0, I) the logit x.W_r[:, e] is N(0, ||W_r[:,e]||^2)
    so each expert fires for `ratio` of the tokens on average (ReLU routing
    keeps the per-token count variable);
  * the prefill workload adds a per-expert skew ~ N(0, 0.3) to b, which spreads
    the per-expert load (mean ratio Phi(-q / sqrt(1.3)) ~ 23 %).

b and lambda are float32 values.  Nothing here evaluates the layer.
"""
from __future__ import annotations

import dataclasses
import math
from statistics import NormalDist

import numpy as np

# workload table ---------------------------------------------------------------
CONFIGS = {
    1: dict(name="tiny-fp32", d=64, E=8, F=32, Fs=64, T=16, dtype="f32",
            lam="lognormal-var0.5", ratio=0.20, skew_var=0.0),
    2: dict(name="decode-bf16", d=2048, E=56, F=128, Fs=1024, T=8, dtype="bf16",
            lam="lognormal-var0.5", ratio=0.20, skew_var=0.0),
    3: dict(name="prefill-bf16", d=2048, E=56, F=128, Fs=1024, T=4096, dtype="bf16",
            lam="lognormal-var0.5", ratio=0.20, skew_var=0.3),
    4: dict(name="edge-d4096-bf16", d=4096, E=112, F=128, Fs=2048, T=16, dtype="bf16",
            lam="lognormal-sigma0.8", ratio=0.20, skew_var=0.0,
            T_sweep=(1, 16, 256, 2048)),
    5: dict(name="ratio-sweep-bf16", d=2048, E=56, F=128, Fs=1024, T=1024, dtype="bf16",
            lam="lognormal-var0.5", ratio=0.20, skew_var=0.0,
            ratio_sweep=(0.05, 0.10, 0.20, 0.40)),
}


def dense_equivalent_dff(cfg: dict) -> int:
    """d_ff of the non-gated dense FFN with the same parameter count (E*F + Fs)."""
    return cfg["E"] * cfg["F"] + cfg["Fs"]


# rounding helpers ------------------------------------------------------------
def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value (ties to even), once.

    bf16 keeps 8 significant bits; frexp gives a in [0.5, 1) * 2^e, so the
    value is rint(a * 2^8) / 2^8 * 2^e with numpy's half-to-even rint.
    Inputs here are far from bf16's overflow and subnormal ranges.
    """
    a = np.asarray(a, dtype=np.float64)
    m, e = np.frexp(a)
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


def bf16_bits(a_bf16_values: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float64 arrays that already hold bf16 values."""
    f32 = np.ascontiguousarray(a_bf16_values, dtype=np.float32)
    bits = f32.view(np.uint32)
    assert not np.any(bits & 0xFFFF), "value is not exactly representable in bf16"
    return (bits >> 16).astype(np.uint16)


def _cast(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_to_bf16(a)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


@dataclasses.dataclass
class LayerInputs:
    """One synthetic layer plus one batch of tokens, as float64 arrays whose
    values are exactly representable in `dtype` (b_r and lam: float32)."""
    d: int
    E: int
    F: int
    Fs: int
    T: int
    dtype: str
    eps: float
    x: np.ndarray        # [T, d]
    W_r: np.ndarray      # [d, E]
    b_r: np.ndarray      # [E]
    lam: np.ndarray      # [E]
    W_up: np.ndarray     # [E, d, F]
    W_down: np.ndarray   # [E, F, d]
    Ws_up: np.ndarray    # [d, Fs]
    Ws_down: np.ndarray  # [Fs, d]
    name: str = ""
    W_gate: np.ndarray | None = None   # [E, d, F], gated-expert layers only

    def weights(self) -> dict:
        w = dict(W_r=self.W_r, b_r=self.b_r, lam=self.lam, W_up=self.W_up,
                 W_down=self.W_down, Ws_up=self.Ws_up, Ws_down=self.Ws_down)
        if self.W_gate is not None:
            w["W_gate"] = self.W_gate
        return w

    def with_x(self, x: np.ndarray) -> "LayerInputs":
        return dataclasses.replace(self, x=np.asarray(x, dtype=np.float64), T=int(x.shape[0]))


def make_custom(d: int, E: int, F: int, Fs: int, T: int, dtype: str = "bf16", *,
                seed: int = 0, ratio: float = 0.20, lam: str = "lognormal-var0.5",
                skew_var: float = 0.0, eps: float = 1e-6, name: str = "custom",
                gated: bool = False) -> LayerInputs:
    """Draw one layer of the given shape with the recipe in the module docstring.
    gated: also a gate projection W_gate [E,d,F] ~ N(0, 1/d) from a ninth
    sub-stream (the first eight, and so the other weights, are unchanged)."""
    ss = np.random.SeedSequence(seed).spawn(9 if gated else 8)
    rng = [np.random.Generator(np.random.PCG64(s)) for s in ss]
    x = _cast(rng[0].standard_normal((T, d)), dtype)
    W_r = _cast(rng[1].standard_normal((d, E)) / math.sqrt(d), dtype)
    W_up = _cast(rng[2].standard_normal((E, d, F)) / math.sqrt(d), dtype)
    W_down = _cast(rng[3].standard_normal((E, F, d)) / math.sqrt(F), dtype)
    Ws_up = _cast(rng[4].standard_normal((d, Fs)) / math.sqrt(d), dtype)
    Ws_down = _cast(rng[5].standard_normal((Fs, d)) / math.sqrt(Fs), dtype)
    if lam == "lognormal-var0.5":
        lam_v = np.exp(math.sqrt(0.5) * rng[6].standard_normal(E))
    elif lam == "lognormal-sigma0.8":
        lam_v = np.exp(0.8 * rng[6].standard_normal(E))
    elif lam == "ones":
        lam_v = np.ones(E)
    else:
        raise ValueError(lam)
    q = NormalDist().inv_cdf(1.0 - ratio)
    b = -q * np.sqrt(np.sum(W_r * W_r, axis=0))
    if skew_var > 0.0:
        b = b + math.sqrt(skew_var) * rng[7].standard_normal(E)
    f32 = lambda a: np.asarray(a, dtype=np.float32).astype(np.float64)
    W_gate = None
    if gated:
        W_gate = _cast(np.random.Generator(np.random.PCG64(ss[8])).standard_normal((E, d, F)) / math.sqrt(d), dtype)
    return LayerInputs(d=d, E=E, F=F, Fs=Fs, T=T, dtype=dtype, eps=eps, x=x, W_r=W_r,
                       b_r=f32(b), lam=f32(lam_v), W_up=W_up, W_down=W_down,
                       Ws_up=Ws_up, Ws_down=Ws_down, name=name, W_gate=W_gate)


def make_layer(cfg_id: int, seed: int = 0, *, T: int | None = None,
               ratio: float | None = None, gated: bool = False) -> LayerInputs:
    """The synthetic workload `cfg_id` (1..5).  `T` overrides the token count
    (the d=4096 layer is swept over T), `ratio` the target activation ratio
    (the ratio-sweep workload)."""
    c = CONFIGS[cfg_id]
    return make_custom(c["d"], c["E"], c["F"], c["Fs"], c["T"] if T is None else T,
                       c["dtype"], seed=seed, ratio=c["ratio"] if ratio is None else ratio,
                       lam=c["lam"], skew_var=c["skew_var"], name=c["name"], gated=gated)


def make_dout(L: LayerInputs, seed: int = 1) -> np.ndarray:
    """An upstream gradient of the layer output for the backward pass:
    [T, d] ~ N(0, 1), cast once to the layer dtype (float64 values)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 0xD0])))
    return _cast(rng.standard_normal((L.T, L.d)), L.dtype)
