"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Bar: the layer's arithmetic agrees with the oracle to 2e-2 * RMS(out_oracle)
for bf16 and 1e-4 * RMS(out_oracle) for fp32 (RMS over all T*d entries),
before the single final rounding of `out` to its dtype: elementwise
    |out_gpu - out_oracle| - ulp(out_gpu) / 2  <=  tol * RMS(out_oracle).
(The workloads' outputs are heavy-tailed, max|out| / RMS up to ~24, so the
half-ulp of the bf16 output format alone reaches 5 % of RMS on some of them.)
The literal max|out_gpu - out_oracle| / RMS is printed for every case.
Active-expert masks: bit-exact except entries whose oracle logit has
|z| < 1e-5 (counted and printed).
Inputs: the seeded synthetic workloads of `synthetic` (full sizes, in the
launch configuration the benchmark times), plus edge cases.
"""
import functools
import sys

import numpy as np
import pytest
import torch

import oracle
from synthetic import make_custom, make_layer
from synthetic.gen import round_to_bf16
from synthetic.device import layer_tensors, x_tensor

pytestmark = pytest.mark.gpu

import sparse_moe_relu_amd as dm

TOL = {"bf16": 2e-2, "f32": 1e-4}
NEAR = 1e-5


def _say(msg):
    print(f"[parity] {msg}", flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=None)
def _workload(cfg_id, T=None, ratio=None):
    return make_layer(cfg_id, T=T, ratio=ratio)


def _layer_obj(L, max_tokens):
    return dm.Layer(**layer_tensors(L), max_tokens=max_tokens, eps=L.eps)


def half_ulp(v: np.ndarray, dtype: str) -> np.ndarray:
    """Half a unit in the last place of the dtype at each (already rounded) value."""
    _, ex = np.frexp(np.abs(v))
    bits = {"bf16": 8, "f32": 24}[dtype]
    return np.where(v == 0, 0.0, np.ldexp(1.0, ex - 1 - bits))


def check(L, ref, layer, path=None, *, T=None, label=""):
    """Run the GPU layer on L.x[:T] and compare with ref (oracle on the same rows)."""
    T = L.T if T is None else T
    x = x_tensor(L)[:T].contiguous()
    _say(f"{label} T={T} path={path} d={L.d} E={L.E} F={L.F} Fs={L.Fs} {L.dtype}")
    out = layer(x, path=dm.DECO_PATH_AUTO if path is None else path)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    want = ref.out[:T]
    rms = float(np.sqrt(np.mean(want ** 2)))
    assert np.all(np.isfinite(got)), label
    err = float(np.max(np.abs(got - want)))
    excess = float(np.max(np.abs(got - want) - half_ulp(got, L.dtype)))
    assert excess <= TOL[L.dtype] * rms, \
        f"{label}: max err beyond output rounding {excess:.3e} > {TOL[L.dtype]} * rms {rms:.3e} (literal {err:.3e})"
    act = layer.active_mask(T).numpy()
    mism = act != ref.active[:T]
    near = np.abs(ref.z[:T]) < NEAR
    assert not np.any(mism & ~near), f"{label}: {int(np.sum(mism & ~near))} mask mismatches outside band"
    assert layer.error_flags() == 0, f"{label}: a device-side wait timed out"
    _, logits = layer.routing(T)
    zabs = np.abs(logits.cpu().numpy().astype(np.float64) - ref.z[:T])
    zerr = float(np.max(zabs))
    # logits are fp32 sums of d exact (bf16) or once-rounded (fp32) products
    # plus the bias: whatever the summation order, |error| <= (d + 2) u
    # sum_k |x_k W_r[k, e]| + u |z| with u = 2^-24
    u = 2.0 ** -24
    zbound = (L.d + 2) * u * (np.abs(L.x[:T]) @ np.abs(L.W_r)) + u * np.abs(ref.z[:T]) + 1e-30
    assert np.all(zabs <= zbound), f"{label}: logit error {zerr:.3e} beyond the fp32 summation bound"
    _say(f"  ok: excess/rms={excess / rms:.2e} literal err/rms={err / rms:.2e} mask_mismatch_in_band={int(mism.sum())} near_zero={int(near.sum())} "
         f"zerr={zerr:.2e} zerr/bound={float(np.max(zabs / zbound)):.2f} active={ref.active[:T].mean():.3f}")
    return got


def _subset(ref, T):
    return oracle.OracleResult(out=ref.out[:T], z=ref.z[:T], active=ref.active[:T], g=ref.g[:T],
                               routed=ref.routed[:T], shared=ref.shared[:T])


# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def c1():
    L = _workload(1)
    ref = oracle.forward(L.x, **L.weights(), eps=L.eps)
    return L, ref, _layer_obj(L, 64)


@pytest.mark.parametrize("path", ["decode", "prefill"])
def test_c1_tiny_fp32(c1, path):
    L, ref, layer = c1
    check(L, ref, layer, dm.DECO_PATH_DECODE if path == "decode" else dm.DECO_PATH_PREFILL, label="c1")


def test_c1_mean_up_matches_oracle(c1):
    L, _, layer = c1
    wbar = layer.mean_up().cpu().numpy().astype(np.float64)
    want = oracle.mean_up(L.W_up)
    assert np.max(np.abs(wbar - want)) <= 1e-6 * np.max(np.abs(want))


@pytest.fixture(scope="module")
def c2():
    L = _workload(2)
    ref = oracle.forward(L.x, **L.weights(), eps=L.eps)
    return L, ref, _layer_obj(L, 64)


@pytest.mark.parametrize("path", ["decode", "prefill"])
def test_c2_decode_bf16(c2, path):
    L, ref, layer = c2
    check(L, ref, layer, dm.DECO_PATH_DECODE if path == "decode" else dm.DECO_PATH_PREFILL, label="c2")


def test_c2_mean_up_matches_oracle(c2):
    L, _, layer = c2
    wbar = layer.mean_up().cpu().numpy().astype(np.float64)
    want = oracle.mean_up(L.W_up)
    assert np.max(np.abs(wbar - want)) <= 1e-5 * np.max(np.abs(want))


@pytest.mark.parametrize("T", [1, 2, 5, 16])
def test_c2_decode_token_counts(c2, T):
    L, ref, layer = c2
    Lb = make_layer(2, T=16)
    refb = oracle.forward(Lb.x, **Lb.weights(), eps=Lb.eps)
    check(Lb, _subset(refb, T), layer, dm.DECO_PATH_DECODE, T=T, label="c2-T")


def test_c2_decode_and_prefill_agree_and_repeat_bitwise(c2):
    L, ref, layer = c2
    x = x_tensor(L)
    a = layer(x, path=dm.DECO_PATH_DECODE).clone()
    b = layer(x, path=dm.DECO_PATH_DECODE).clone()
    c = layer(x, path=dm.DECO_PATH_PREFILL).clone()
    torch.cuda.synchronize()
    assert torch.equal(a, b), "decode path is not deterministic"
    rms = float(np.sqrt(np.mean(ref.out ** 2)))
    an = a.float().cpu().numpy().astype(np.float64)
    cn = c.float().cpu().numpy().astype(np.float64)
    # both are rounded once to bf16: allow half an ulp each on top of the bar
    gap = np.abs(an - cn) - half_ulp(an, "bf16") - half_ulp(cn, "bf16")
    assert float(gap.max()) <= 2e-2 * rms


def test_decode_and_prefill_replay_from_a_hip_graph(c2):
    """Both forward paths are kernel launches only (no allocation, copy,
    memset or host wait per call), so a serving loop can capture them in a
    HIP graph.  Every replay must equal the eager result bitwise, also with
    eager calls on other inputs between the replays (they rewrite the
    layer's workspace)."""
    L, ref, layer = c2
    x = x_tensor(L)
    x_other = torch.flip(x, dims=[0]).contiguous()
    want_dec = layer(x, path=dm.DECO_PATH_DECODE).clone()
    want_pre = layer(x, path=dm.DECO_PATH_PREFILL).clone()
    out_dec, out_pre = torch.empty_like(x), torch.empty_like(x)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer(x, out_dec, path=dm.DECO_PATH_DECODE)
        layer(x, out_pre, path=dm.DECO_PATH_PREFILL)
    torch.cuda.synchronize()
    for rep in range(3):
        other = layer(x_other, path=dm.DECO_PATH_DECODE if rep % 2 else dm.DECO_PATH_PREFILL).clone()
        out_dec.zero_()
        out_pre.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_dec, want_dec), f"decode replay {rep} differs from the eager call"
        assert torch.equal(out_pre, want_pre), f"prefill replay {rep} differs from the eager call"
        assert not torch.equal(other, want_dec)
    del g
    torch.cuda.synchronize()


def test_c3_prefill_full_size():
    L = _workload(3)
    ref = oracle.forward(L.x, **L.weights(), eps=L.eps)
    layer = _layer_obj(L, L.T)
    got = check(L, ref, layer, label="c3")
    # repeat: bitwise identical (no atomics in the combine)
    got2 = layer(x_tensor(L)).float().cpu().numpy()
    assert np.array_equal(got, got2.astype(np.float64))
    # ragged tails of the same layer through the prefill tiles, including a
    # ragged last tile of the 64-row router launch (T = 4001), repeated
    # bitwise
    for T in (17, 100, 1000, 4001):
        g1 = check(L, _subset(ref, T), layer, T=T, label="c3-ragged")
        if T == 4001:
            g2 = layer(x_tensor(L)[:T].contiguous()).float().cpu().numpy().astype(np.float64)
            assert np.array_equal(g1, g2)
    layer.free()


@pytest.fixture(scope="module")
def c4():
    L = _workload(4, T=2048)
    ref = oracle.forward(L.x, **L.weights(), eps=L.eps)
    return L, ref, _layer_obj(L, 2048)


@pytest.mark.parametrize("T", [1, 16, 256, 2047, 2048])
def test_c4_edge_model_T_sweep(c4, T):
    L, ref, layer = c4
    got = check(L, _subset(ref, T), layer, T=T, label="c4")
    if T == 2047:   # ragged last tile of the 64-row router launch, repeated bitwise
        again = layer(x_tensor(L)[:T].contiguous()).float().cpu().numpy().astype(np.float64)
        assert np.array_equal(got, again)


@pytest.mark.parametrize("ratio", [0.05, 0.10, 0.20, 0.40])
def test_c5_ratio_sweep(ratio):
    L = _workload(5, ratio=ratio)
    ref = oracle.forward(L.x, **L.weights(), eps=L.eps)
    layer = _layer_obj(L, L.T)
    check(L, ref, layer, label=f"c5-{ratio}")
    layer.free()


# edge cases --------------------------------------------------------------------
@pytest.mark.parametrize("shape", [
    (128, 5, 32, 64, "bf16"),     # E not a multiple of 16, smallest F
    (192, 70, 64, 96, "bf16"),    # two mask words, F = 64, Fs not a multiple of 64
    (256, 12, 256, 32, "bf16"),   # widest F, narrowest Fs
    (128, 3, 256, 160, "f32"),
    (64, 1, 32, 32, "bf16"),      # E = 1: routed part vanishes
    (128, 256, 256, 64, "bf16"),  # decode: routed units past one chunk per wave (the reload loop), 4 mask words
    (4096, 4, 32, 4096, "bf16"),  # decode: 16 shared k-blocks per down workgroup (more than one per wave)
])
@pytest.mark.parametrize("path", ["decode", "prefill"])
def test_shapes(shape, path):
    d, E, F, Fs, dt = shape
    T = 11 if path == "decode" else 77
    L = make_custom(d, E, F, Fs, T, dt, seed=9, ratio=0.3)
    ref = oracle.forward(L.x, **L.weights(), eps=L.eps)
    layer = _layer_obj(L, 80)
    check(L, ref, layer, dm.DECO_PATH_DECODE if path == "decode" else dm.DECO_PATH_PREFILL,
          label=f"shape{shape}")
    layer.free()


def test_changing_inputs_between_calls():
    """Alternate different batches (and sizes) through one layer on both paths:
    each call must match the oracle on its own input, so no value a kernel
    hands from one workgroup to another can be left over from an earlier call
    (the benchmark repeats one input, which would hide that)."""
    base = make_custom(512, 24, 128, 256, 16, "bf16", seed=31, ratio=0.3)
    rng = np.random.default_rng(77)
    xb = round_to_bf16(rng.standard_normal((16, base.d)))
    layer = _layer_obj(base, 64)
    plan = [(base.x, 16, dm.DECO_PATH_DECODE), (xb, 9, dm.DECO_PATH_DECODE), (base.x, 16, dm.DECO_PATH_DECODE),
            (xb, 16, dm.DECO_PATH_PREFILL), (base.x, 5, dm.DECO_PATH_PREFILL), (xb, 3, dm.DECO_PATH_DECODE),
            (base.x, 16, dm.DECO_PATH_PREFILL)]
    for k, (x, T, path) in enumerate(plan):
        L = base.with_x(x[:T])
        ref = oracle.forward(L.x, **L.weights(), eps=L.eps)
        check(L, ref, layer, path, label=f"alternate-{k}")
    layer.free()


# T = 16 also runs the decode up kernel that requests W_up before the routing
# decision: every expert's slice has loads in flight when it finds no token
@pytest.mark.parametrize("T", [13, 16])
@pytest.mark.parametrize("case", ["all_negative", "lambda_zero", "some_lambda_zero"])
@pytest.mark.parametrize("path", ["decode", "prefill"])
def test_degenerate_routing(case, path, T):
    L = make_custom(256, 24, 128, 128, T, "bf16", seed=4)
    b, lam = L.b_r.copy(), L.lam.copy()
    if case == "all_negative":
        b[:] = -1e4
    elif case == "lambda_zero":
        lam[:] = 0.0
    else:
        lam[::3] = 0.0
    L2 = make_custom(256, 24, 128, 128, T, "bf16", seed=4)
    L2.b_r, L2.lam = b, lam
    ref = oracle.forward(L2.x, **L2.weights(), eps=L2.eps)
    layer = _layer_obj(L2, 32)
    got = check(L2, ref, layer, dm.DECO_PATH_DECODE if path == "decode" else dm.DECO_PATH_PREFILL,
                label=case)
    if case != "some_lambda_zero":
        assert not ref.active.any()
    layer.free()


def test_zero_tokens_is_a_noop(c2):
    L, ref, layer = c2
    x = x_tensor(L)
    out = torch.full_like(x, 3.0)
    st = dm.load_library().deco_moe_forward(layer.handle, x.data_ptr(), 0, out.data_ptr(), None)
    torch.cuda.synchronize()
    assert st == dm.DECO_OK
    assert bool((out == 3.0).all())


def test_invalid_T_rejected_and_out_untouched(c2):
    L, ref, layer = c2
    x = torch.zeros((65, L.d), dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(x, 5.0)
    lib = dm.load_library()
    assert lib.deco_moe_forward(layer.handle, x.data_ptr(), 65, out.data_ptr(), None) == dm.DECO_ERR_INVALID_ARG
    assert lib.deco_moe_forward_path(layer.handle, x.data_ptr(), 17, out.data_ptr(), None,
                                     dm.DECO_PATH_DECODE) == dm.DECO_ERR_INVALID_ARG
    assert lib.deco_moe_forward(layer.handle, x.data_ptr(), 8, x.data_ptr(), None) == dm.DECO_ERR_INVALID_ARG
    assert lib.deco_moe_forward(layer.handle, x.data_ptr() + 2, 8, out.data_ptr(), None) == dm.DECO_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert bool((out == 5.0).all())


def test_binding_rejects_a_mismatched_out_buffer(c2):
    # the library writes T*d elements at out's address, so the binding checks
    # out before any launch: too few rows, another dtype, a strided view
    L, ref, layer = c2
    x = x_tensor(L)[:8].contiguous()
    good = torch.full_like(x, 5.0)
    bad = [torch.empty((4, L.d), dtype=x.dtype, device="cuda"),
           torch.empty((8, L.d), dtype=torch.float32, device="cuda"),
           torch.empty((8, 2 * L.d), dtype=x.dtype, device="cuda")[:, :L.d]]
    for out in bad:
        with pytest.raises(ValueError):
            layer(x, out)
    torch.cuda.synchronize()
    assert bool((good == 5.0).all())
    got = layer(x, good)
    assert got.data_ptr() == good.data_ptr()
    assert torch.equal(got, layer(x))


def test_max_tokens_boundary():
    L = make_custom(128, 9, 64, 64, 40, "bf16", seed=21)
    ref = oracle.forward(L.x, **L.weights(), eps=L.eps)
    layer = _layer_obj(L, 40)
    check(L, ref, layer, label="T=max_tokens")
    layer.free()
