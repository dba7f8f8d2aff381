"""Seeded random configurations, checked in full against the oracle: group
sizes 1-8 (odd ones included), head dims 32/64/128, sequence lengths next to
every tile boundary the kernels use (32, 64 and 128 rows or keys), both mask
modes and a spread of scales, for bf16 and (forward and backward) fp32.  The draw is fixed (numpy seed 20261203), so
every run checks the same cases; they complement the hand-picked shapes of
the other parity tests."""
import math
import sys

import numpy as np
import pytest

import inputs
import oracle
from tests import parity

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
import reduced_query_head_amd as sqa  # noqa: E402
from tests import gpu_util  # noqa: E402
from tests.test_gpu_backward import _check_grad, dk_allowance, dq_allowance  # noqa: E402

LSE_MAX = 2.5e-3


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _draw(n, seed):
    rng = np.random.default_rng(seed)
    edges = [1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 383, 384, 385, 511, 512, 513]
    cases = []
    for i in range(n):
        R = int(rng.choice([1, 1, 2, 3, 4, 5, 6, 7, 8]))
        H_kv = int(rng.integers(1, 4))
        H_q = R * H_kv
        d = int(rng.choice([32, 64, 128]))
        S = int(rng.choice(edges)) + (int(rng.integers(0, 64)) * 8 if i % 3 == 0 else 0)
        B = int(rng.integers(1, 3))
        causal = bool(rng.integers(0, 2))
        scale = float(rng.choice([1 / math.sqrt(d), 0.05, 0.3, -0.15]))
        cases.append((B, S, H_q, H_kv, d, causal, scale))
    return cases


FWD = _draw(28, 20261203)
BWD = _draw(12, 20261204)
DEC = _draw(12, 20261205)
F32_FWD = _draw(12, 20261206)
F32_BWD = _draw(8, 20261207)
F32_LSE_MAX, F32_LSE_MEAN = 2e-5, 2e-6


@pytest.mark.parametrize("B,S,H_q,H_kv,d,causal,scale", FWD)
def test_random_forward_and_lse(B, S, H_q, H_kv, d, causal, scale):
    _say(f"fwd B={B} S={S} H={H_q}/{H_kv} d={d} causal={causal} scale={scale:.4g}")
    seed = 12000 + S + 7 * H_q + d
    q = inputs.normal(seed, 0, (B, S, H_q, d), "bf16", 0.5)
    k = inputs.normal(seed, 1, (B, S, H_kv, d), "bf16", 0.5)
    v = inputs.normal(seed, 2, (B, S, H_kv, d), "bf16", 0.5)
    dq, dk, dv = (gpu_util.to_device(a) for a in (q, k, v))
    o, lse = sqa.attn_fwd(dq, dk, dv, scale=scale, causal=causal, return_lse=True)
    torch.cuda.synchronize()
    sc = float(np.float32(scale))
    parity.check(gpu_util.to_host_f64(o), oracle.attention(q, k, v, sc, causal=causal), "bf16", "random forward")
    err = np.abs(lse.double().cpu().numpy() - oracle.lse(q, k, sc, causal=causal))
    assert err.max() <= LSE_MAX, f"lse {err.max()}"


@pytest.mark.parametrize("B,S,H_q,H_kv,d,causal,scale", BWD)
def test_random_backward(B, S, H_q, H_kv, d, causal, scale):
    _say(f"bwd B={B} S={S} H={H_q}/{H_kv} d={d} causal={causal} scale={scale:.4g}")
    seed = 13000 + S + 7 * H_q + d
    q = inputs.normal(seed, 0, (B, S, H_q, d), "bf16", 0.5)
    k = inputs.normal(seed, 1, (B, S, H_kv, d), "bf16", 0.5)
    v = inputs.normal(seed, 2, (B, S, H_kv, d), "bf16", 0.5)
    g = inputs.normal(seed, 5, (B, S, H_q, d), "bf16", 1.0)
    dq_, dk_, dv_, dg = (gpu_util.to_device(a) for a in (q, k, v, g))
    o, lse = sqa.attn_fwd(dq_, dk_, dv_, scale=scale, causal=causal, return_lse=True)
    gq, gk, gv = sqa.attn_bwd(dq_, dk_, dv_, o, dg, lse, scale=scale, causal=causal)
    torch.cuda.synchronize()
    sc = float(np.float32(scale))
    rq, rk, rv = oracle.attention_grad(q, k, v, g, sc, causal=causal)
    allow = {"dq": dq_allowance(q, k, v, g, sc, causal), "dk": dk_allowance(q, k, v, g, sc, causal), "dv": None}
    for name, got, ref in (("dq", gq, rq), ("dk", gk, rk), ("dv", gv, rv)):
        _check_grad(gpu_util.to_host_f64(got), ref, "bf16", f"random {name}", allow[name])


@pytest.mark.parametrize("B,S,H_q,H_kv,d,causal,scale", F32_FWD)
def test_random_forward_and_lse_f32(B, S, H_q, H_kv, d, causal, scale):
    """The fp32 matrix-core forward on the same kind of draw."""
    _say(f"f32 fwd B={B} S={S} H={H_q}/{H_kv} d={d} causal={causal} scale={scale:.4g}")
    seed = 15000 + S + 7 * H_q + d
    q = inputs.normal(seed, 0, (B, S, H_q, d), "f32", 0.5)
    k = inputs.normal(seed, 1, (B, S, H_kv, d), "f32", 0.5)
    v = inputs.normal(seed, 2, (B, S, H_kv, d), "f32", 0.5)
    dq, dk, dv = (gpu_util.to_device(a) for a in (q, k, v))
    o, lse = sqa.attn_fwd(dq, dk, dv, scale=scale, causal=causal, return_lse=True)
    torch.cuda.synchronize()
    sc = float(np.float32(scale))
    parity.check(gpu_util.to_host_f64(o), oracle.attention(q, k, v, sc, causal=causal), "f32", "random f32 forward")
    err = np.abs(lse.double().cpu().numpy() - oracle.lse(q, k, sc, causal=causal))
    assert err.max() <= F32_LSE_MAX and err.mean() <= F32_LSE_MEAN, f"lse max {err.max()} mean {err.mean()}"


@pytest.mark.parametrize("B,S,H_q,H_kv,d,causal,scale", F32_BWD)
def test_random_backward_f32(B, S, H_q, H_kv, d, causal, scale):
    """The fp32 matrix-core backward on the same kind of draw."""
    _say(f"f32 bwd B={B} S={S} H={H_q}/{H_kv} d={d} causal={causal} scale={scale:.4g}")
    seed = 16000 + S + 7 * H_q + d
    q = inputs.normal(seed, 0, (B, S, H_q, d), "f32", 0.5)
    k = inputs.normal(seed, 1, (B, S, H_kv, d), "f32", 0.5)
    v = inputs.normal(seed, 2, (B, S, H_kv, d), "f32", 0.5)
    g = inputs.normal(seed, 5, (B, S, H_q, d), "f32", 1.0)
    dq_, dk_, dv_, dg = (gpu_util.to_device(a) for a in (q, k, v, g))
    o, lse = sqa.attn_fwd(dq_, dk_, dv_, scale=scale, causal=causal, return_lse=True)
    gq, gk, gv = sqa.attn_bwd(dq_, dk_, dv_, o, dg, lse, scale=scale, causal=causal)
    torch.cuda.synchronize()
    sc = float(np.float32(scale))
    rq, rk, rv = oracle.attention_grad(q, k, v, g, sc, causal=causal)
    allow = {"dq": dq_allowance(q, k, v, g, sc, causal, dtype="f32"),
             "dk": dk_allowance(q, k, v, g, sc, causal, dtype="f32"), "dv": None}
    for name, got, ref in (("dq", gq, rq), ("dk", gk, rk), ("dv", gv, rv)):
        _check_grad(gpu_util.to_host_f64(got), ref, "f32", f"random f32 {name}", allow[name])


@pytest.mark.parametrize("B,S,H_q,H_kv,d,causal,scale", DEC)
def test_random_decode(B, S, H_q, H_kv, d, causal, scale):
    # causal picks ragged lengths (seeded, 0 allowed) instead of full caches
    rng = np.random.default_rng(S + H_q + d)
    lens = [int(x) for x in rng.integers(0, S + 1, B)] if causal else None
    _say(f"decode B={B} S_max={S} H={H_q}/{H_kv} d={d} lens={lens} scale={scale:.4g}")
    seed = 14000 + S + 7 * H_q + d
    q = inputs.normal(seed, 0, (B, H_q, d), "bf16", 0.5)
    k = inputs.normal(seed, 1, (B, S, H_kv, d), "bf16", 0.5)
    v = inputs.normal(seed, 2, (B, S, H_kv, d), "bf16", 0.5)
    dq, dk, dv = (gpu_util.to_device(a) for a in (q, k, v))
    dl = None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda")
    out, lse = sqa.attn_decode(dq, dk, dv, seqlens=dl, scale=scale, return_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.decode(q, k, v, float(np.float32(scale)), seqlens=lens)
    got = gpu_util.to_host_f64(out)
    got_lse = lse.double().cpu().numpy()
    empty = np.zeros(B, dtype=bool) if lens is None else np.asarray(lens) <= 0
    assert (got[empty] == 0).all() and np.isneginf(got_lse[empty]).all()
    if (~empty).any():
        parity.check(got[~empty], ref[~empty], "bf16", "random decode")
        assert np.abs(got_lse[~empty] - ref_lse[~empty]).max() <= LSE_MAX


# Shapes whose grid takes the 8-wave kernel of their head dim (at least 512
# workgroups of 8 query blocks at d = 128 and 32, 256 at d = 64), checked in
# full: ragged tails (S mod 128 = 1, 4, 55, 56, 63, 104, 127), odd group
# sizes, both masks, each head dim.
LARGE = [
    (2, 4097, 16, 16, 64, False),
    (1, 4200, 32, 8, 128, True),
    (2, 3000, 48, 16, 64, True),
    (4, 2111, 24, 8, 128, False),
    (1, 8191, 16, 2, 128, True),
    (2, 4100, 12, 4, 64, True),
    (2, 4097, 16, 16, 32, False),
    (2, 3000, 24, 8, 32, True),
]


@pytest.mark.parametrize("B,S,H_q,H_kv,d,causal", LARGE)
def test_large_grid_forward_full(B, S, H_q, H_kv, d, causal):
    items = (H_q // H_kv) * ((S + 31) // 32)
    need = 256 if d == 64 else 512
    assert B * H_kv * ((items + 7) // 8) >= need, "shape does not reach the 8-wave kernel"
    _say(f"fwd (8-wave) B={B} S={S} H={H_q}/{H_kv} d={d} causal={causal}")
    seed = 15000 + S + 7 * H_q + d
    q = inputs.normal(seed, 0, (B, S, H_q, d), "bf16", 0.5)
    k = inputs.normal(seed, 1, (B, S, H_kv, d), "bf16", 0.5)
    v = inputs.normal(seed, 2, (B, S, H_kv, d), "bf16", 0.5)
    dq, dk, dv = (gpu_util.to_device(a) for a in (q, k, v))
    scale = 1 / math.sqrt(d)
    o, lse = sqa.attn_fwd(dq, dk, dv, scale=scale, causal=causal, return_lse=True)
    torch.cuda.synchronize()
    sc = float(np.float32(scale))
    st = parity.check(gpu_util.to_host_f64(o), oracle.attention(q, k, v, sc, causal=causal), "bf16", "8-wave forward")
    err = np.abs(lse.double().cpu().numpy() - oracle.lse(q, k, sc, causal=causal))
    assert err.max() <= LSE_MAX, f"lse {err.max()}"
    _say(f"  {st}")
