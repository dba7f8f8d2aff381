"""GPU parity of the attention backward (dq, dk, dv) against the fp64 oracle
gradient on identical inputs.

Error model for bf16 (fp32 accumulation; P and dS rounded to bf16 before the
products; outputs rounded to bf16):
  * every gradient element is a sum of terms with relative rounding <= 2^-9
    and random signs: a few 1e-3 relative L2 expected;
  * D_i = <dout_i, out_i> is formed from the forward kernel's bf16 output,
    as the backward receives it.  That output carries the forward's own
    rounding (P rounded to bf16 before P.V, output rounded to bf16), at most
    2^-8 sum_j p_ij |v_je| per element, so D_i is off by up to 2^-8 a_i with
    a_i = sum_e |dout_ie| (P|V|)_ie.  That shifts every dS_ij of row i by
    p_ij times this amount: an absolute error of up to |scale| 2^-8 a_i
    max_j |k_j| on dq_i and of up to |scale| 2^-8 max_i(a_i |q_i|) sum_i p_ij
    on dk_j.
    Rows whose gradient is a small difference of large terms (few visible
    keys) feel it most; where the exact gradient is 0 (one visible key) the
    GPU value is this rounding alone.
Bounds: per row |err| <= 6e-2 |ref| + 2 * allowance (the D_i term above,
0 for dv, built from oracle values only); whole tensor relative L2 <= 2e-2
and max |err| <= 2e-2 max |ref| unless the allowance outweighs the
reference (an exactly-zero gradient), where |err| <= 2 |allowance|.
fp32: the same with 2e-5 / 1e-4 and the allowance's unit 2^-23.  At full
workload sizes dq is compared on sampled rows; dk and dv (sums over every
query) are checked through identities that hold at any size:
sum_j dk_j = 0 and sum_j dv_j = the group's summed dout.
"""
import math
import sys

import numpy as np
import pytest

import inputs
import oracle
from inputs.configs import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
import reduced_query_head_amd as sqa  # noqa: E402
from tests import gpu_util  # noqa: E402

BWD_BOUNDS = {"bf16": dict(rel=2e-2, row=6e-2, mx=2e-2, unit=2.0 ** -8),
              "f32": dict(rel=2e-5, row=1e-4, mx=2e-5, unit=2.0 ** -23)}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _f64(a):
    return inputs.bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


def _abs(a):
    """|x| elementwise in the array's own encoding (bf16 bits: clear the sign bit)."""
    return (a & np.uint16(0x7FFF)) if a.dtype == np.uint16 else np.abs(a)


def _delta_bound(q, k, v, dout, scale, causal, rows, dtype):
    """Bound of |D_i - exact D_i|: unit * sum_e |dout_ie| (P|V|)_ie."""
    pv = oracle.attention(q, k, _abs(v), scale, causal=causal, rows=rows)        # P|V|, fp64
    g = _f64(dout) if rows is None else _f64(dout)[:, rows]
    return BWD_BOUNDS[dtype]["unit"] * (np.abs(g) * pv).sum(-1)                 # [B, n, H_q]


def dq_allowance(q, k, v, dout, scale, causal, rows=None, dtype="bf16"):
    """Per (b, row, h) size of the dq error a shift of D_i by its bound causes:
    |scale| * bound_i * |sum_j p_ij k_j| (the shift moves every dS_ij of the
    row by p_ij times the same amount)."""
    pk = oracle.attention(q, k, k, scale, causal=causal, rows=rows)             # sum_j p_ij k_j
    return abs(scale) * _delta_bound(q, k, v, dout, scale, causal, rows, dtype) * np.linalg.norm(pk, axis=-1)


def dk_allowance(q, k, v, dout, scale, causal, dtype="bf16"):
    """Per (b, key, g) bound of the dk error the D_i shifts cause:
    |scale| * sum over the group's heads and rows of p_ij bound_i |q_i|,
    computed as the dv the oracle gives for an upstream gradient that holds
    bound_i |q_i| in its first channel."""
    w = _delta_bound(q, k, v, dout, scale, causal, None, dtype) * np.linalg.norm(_f64(q), axis=-1)
    up = np.zeros(q.shape, dtype=np.float64)
    up[..., 0] = w
    _, _, dvw = oracle.attention_grad(_f64(q), _f64(k), _f64(v), up, scale, causal=causal)
    return abs(scale) * dvw[..., 0]                                              # [B, S, H_kv]


def _check_grad(got, ref, dtype, what, allow=None):
    """Per row: |err| <= row*|ref| + 2*allowance.  Whole tensor: when the
    reference outweighs the allowance, relative L2 <= rel and max|err| <=
    mx*max|ref|; otherwise (a gradient that is exactly zero, e.g. one visible
    key) |err| <= 2*|allowance|."""
    got = np.asarray(got, dtype=np.float64)
    diff = got - ref
    d = ref.shape[-1]
    b = BWD_BOUNDS[dtype]
    rn = np.linalg.norm(diff.reshape(-1, d), axis=1)
    rr = np.linalg.norm(ref.reshape(-1, d), axis=1)
    al = np.zeros_like(rr) if allow is None else 2.0 * np.asarray(allow, dtype=np.float64).reshape(-1)
    assert al.shape == rr.shape
    n_diff, n_ref, n_al = np.linalg.norm(diff), np.linalg.norm(ref), np.linalg.norm(al)
    st = dict(rel_l2=float(n_diff / max(n_ref, 1e-300)),
              worst_row=float((rn / np.maximum(b["row"] * rr + al, 1e-300)).max()),
              max_rel=float(np.abs(diff).max() / max(np.abs(ref).max(), 1e-300)),
              allow_frac=float(n_al / max(n_ref, 1e-300)))
    assert np.isfinite(got).all(), f"{what}: non-finite"
    assert (rn <= b["row"] * rr + al).all() or (rn == 0).all(), f"{what}: row bound {st}"
    if n_ref > n_al:
        assert n_diff <= b["rel"] * n_ref, f"{what}: l2 {st}"
        assert np.abs(diff).max() <= b["mx"] * np.abs(ref).max(), f"{what}: max {st}"
    else:
        assert n_diff <= n_al, f"{what}: degenerate l2 {st}"
    return st


def _run(q, k, v, dout, scale, causal):
    dq_, dk_, dv_, dg = (gpu_util.to_device(a) for a in (q, k, v, dout))
    o, lse = sqa.attn_fwd(dq_, dk_, dv_, scale=scale, causal=causal, return_lse=True)
    gq, gk, gv = sqa.attn_bwd(dq_, dk_, dv_, o, dg, lse, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return gq, gk, gv


SMALL = [
    # B, S, H_q, H_kv, d, causal
    (1, 1, 1, 1, 128, False), (1, 2, 2, 1, 64, True), (1, 33, 4, 4, 128, False), (1, 65, 8, 2, 128, True),
    (2, 130, 4, 1, 64, True), (1, 200, 6, 2, 32, False), (1, 257, 16, 4, 128, True), (2, 300, 8, 8, 128, False),
    (1, 513, 4, 4, 64, True), (1, 1000, 8, 2, 128, True),
    (1, 300, 32, 1, 128, False),   # 32 query heads summed into one K/V head's dK/dV
    (1, 700, 64, 2, 64, True),     # 32 heads per group, causal, d = 64
]


# Sequences of 64 key blocks (128 keys each) or more, where the dK/dV grid
# deals 32-block chunks of a group to the XCDs: partial last chunks (67, 65
# and 65 blocks), one and three groups (idle padding workgroups), a group of
# two query heads, both masks.
CHUNKED = [
    (1, 8492, 2, 1, 32, True),
    (1, 8250, 3, 3, 32, True),
    (1, 8200, 1, 1, 32, False),
]
# d = 64 grids of 512 or more dK/dV workgroups, which take the 4-waves-per-
# SIMD build of that kernel: ragged S, both masks.
WIDE = [
    (4, 1000, 16, 16, 64, False),
    (8, 1000, 8, 8, 64, True),
]
# The chunked dK/dV grid at the head sizes of the long workloads: d = 128
# with a group of two query heads and a ragged last key block (65 blocks,
# the last one 108 keys long), both masks; and d = 64 with 8 groups of 64
# key blocks (512 workgroups, so the 4-waves-per-SIMD build runs chunked).
# dq, dk and dv are compared element by element in full.
CHUNKED_LARGE = [
    (1, 8300, 2, 1, 128, True),
    (1, 8300, 2, 1, 128, False),
    (1, 8100, 8, 8, 64, True),
]


@pytest.mark.parametrize("B,S,H_q,H_kv,d,causal", SMALL + CHUNKED + WIDE + CHUNKED_LARGE)
def test_backward_small_shapes(B, S, H_q, H_kv, d, causal):
    _say(f"bwd B={B} S={S} H={H_q}/{H_kv} d={d} causal={causal}")
    seed = 9000 + S * 7 + H_q + d
    q = inputs.normal(seed, 0, (B, S, H_q, d), "bf16", 0.5)
    k = inputs.normal(seed, 1, (B, S, H_kv, d), "bf16", 0.5)
    v = inputs.normal(seed, 2, (B, S, H_kv, d), "bf16", 0.5)
    dout = inputs.normal(seed, 5, (B, S, H_q, d), "bf16", 1.0)
    scale = 1.0 / math.sqrt(d)
    gq, gk, gv = _run(q, k, v, dout, scale, causal)
    sc = float(np.float32(scale))
    rq, rk, rv = oracle.attention_grad(q, k, v, dout, sc, causal=causal)
    allow = {"dq": dq_allowance(q, k, v, dout, sc, causal), "dk": dk_allowance(q, k, v, dout, sc, causal), "dv": None}
    for name, got, ref in (("dq", gq, rq), ("dk", gk, rk), ("dv", gv, rv)):
        st = _check_grad(gpu_util.to_host_f64(got), ref, "bf16", f"{name} S={S} H={H_q}/{H_kv} d={d} c={causal}",
                         allow[name])
        _say(f"  {name} {st}")


@pytest.mark.parametrize("causal", [False, True])
def test_backward_sharp_softmax(causal):
    """N(0,1) inputs with scale 0.7 at d = 128: each row's softmax is dominated
    by a few keys (scaled scores with a standard deviation near 8), so the
    gradients rest on a few large probabilities and their exact scores."""
    B, S, H_q, H_kv, d = 1, 512, 4, 2, 128
    q = inputs.normal(94, 0, (B, S, H_q, d), "bf16", 1.0)
    k = inputs.normal(94, 1, (B, S, H_kv, d), "bf16", 1.0)
    v = inputs.normal(94, 2, (B, S, H_kv, d), "bf16", 1.0)
    dout = inputs.normal(94, 5, (B, S, H_q, d), "bf16", 1.0)
    gq, gk, gv = _run(q, k, v, dout, 0.7, causal)
    sc = float(np.float32(0.7))
    rq, rk, rv = oracle.attention_grad(q, k, v, dout, sc, causal=causal)
    allow = {"dq": dq_allowance(q, k, v, dout, sc, causal), "dk": dk_allowance(q, k, v, dout, sc, causal), "dv": None}
    for name, got, ref in (("dq", gq, rq), ("dk", gk, rk), ("dv", gv, rv)):
        st = _check_grad(gpu_util.to_host_f64(got), ref, "bf16", f"{name} sharp c={causal}", allow[name])
        _say(f"  {name} {st}")


@pytest.mark.parametrize("scale", [-0.2, 0.0])
def test_backward_scale_values(scale):
    B, S, H_q, H_kv, d = 1, 150, 4, 2, 128
    q = inputs.normal(91, 0, (B, S, H_q, d), "bf16", 0.5)
    k = inputs.normal(91, 1, (B, S, H_kv, d), "bf16", 0.5)
    v = inputs.normal(91, 2, (B, S, H_kv, d), "bf16", 0.5)
    dout = inputs.normal(91, 5, (B, S, H_q, d), "bf16", 1.0)
    for causal in (False, True):
        gq, gk, gv = _run(q, k, v, dout, scale, causal)
        sc = float(np.float32(scale))
        rq, rk, rv = oracle.attention_grad(q, k, v, dout, sc, causal=causal)
        _check_grad(gpu_util.to_host_f64(gv), rv, "bf16", f"dv scale={scale}")
        if scale != 0.0:  # with scale 0 the score gradients are exactly zero
            _check_grad(gpu_util.to_host_f64(gq), rq, "bf16", f"dq scale={scale}",
                        dq_allowance(q, k, v, dout, sc, causal))
            _check_grad(gpu_util.to_host_f64(gk), rk, "bf16", f"dk scale={scale}",
                        dk_allowance(q, k, v, dout, sc, causal))
        else:
            assert float(gpu_util.to_host_f64(gq).__abs__().max()) == 0.0
            assert float(gpu_util.to_host_f64(gk).__abs__().max()) == 0.0


@pytest.mark.parametrize("B,S,H_q,H_kv,d,causal", [(4, 1000, 16, 16, 64, True), (2, 640, 8, 2, 32, False)])
def test_backward_negative_scale_other_builds(B, S, H_q, H_kv, d, causal):
    """A negative scale (folded into K's sign when the dK/dV kernel stages its
    rows) on the d = 64 4-waves-per-SIMD dK/dV build (512 workgroups) and on
    the d = 32 build, whose query tiles are copied by 4 of its 8 waves."""
    _say(f"bwd negative scale B={B} S={S} H={H_q}/{H_kv} d={d} causal={causal}")
    scale = -0.6 / math.sqrt(d)
    seed = 9500 + S + H_q + d
    q = inputs.normal(seed, 0, (B, S, H_q, d), "bf16", 0.5)
    k = inputs.normal(seed, 1, (B, S, H_kv, d), "bf16", 0.5)
    v = inputs.normal(seed, 2, (B, S, H_kv, d), "bf16", 0.5)
    dout = inputs.normal(seed, 5, (B, S, H_q, d), "bf16", 1.0)
    gq, gk, gv = _run(q, k, v, dout, scale, causal)
    sc = float(np.float32(scale))
    rq, rk, rv = oracle.attention_grad(q, k, v, dout, sc, causal=causal)
    allow = {"dq": dq_allowance(q, k, v, dout, sc, causal), "dk": dk_allowance(q, k, v, dout, sc, causal), "dv": None}
    for name, got, ref in (("dq", gq, rq), ("dk", gk, rk), ("dv", gv, rv)):
        st = _check_grad(gpu_util.to_host_f64(got), ref, "bf16", f"{name} scale={scale:.3g} d={d}", allow[name])
        _say(f"  {name} {st}")


@pytest.mark.parametrize("d", [32, 64, 128])
def test_backward_f32(d):
    B, S, H_q, H_kv = 1, 100, 4, 2
    q = inputs.normal(92, 0, (B, S, H_q, d), "f32")
    k = inputs.normal(92, 1, (B, S, H_kv, d), "f32")
    v = inputs.normal(92, 2, (B, S, H_kv, d), "f32")
    dout = inputs.normal(92, 5, (B, S, H_q, d), "f32")
    for causal in (False, True):
        gq, gk, gv = _run(q, k, v, dout, 1 / math.sqrt(d), causal)
        sc = float(np.float32(1 / math.sqrt(d)))
        rq, rk, rv = oracle.attention_grad(q, k, v, dout, sc, causal=causal)
        allow = {"dq": dq_allowance(q, k, v, dout, sc, causal, dtype="f32"),
                 "dk": dk_allowance(q, k, v, dout, sc, causal, dtype="f32"), "dv": None}
        for name, got, ref in (("dq", gq, rq), ("dk", gk, rk), ("dv", gv, rv)):
            _check_grad(gpu_util.to_host_f64(got), ref, "f32", f"f32 {name} d={d} c={causal}", allow[name])


# fp32 on the matrix cores: several 128-key dk/dv workgroups and 32-row
# query tiles over two heads per group, a 257-position sequence (a one-row
# tail) at d = 128, and eight heads on one K/V head with a 33-position
# sequence; a positive and a negative scale, causal and not.
F32_BWD = [(2, 300, 6, 3, 64), (1, 257, 4, 4, 128), (1, 33, 8, 1, 32)]


@pytest.mark.parametrize("B,S,H_q,H_kv,d", F32_BWD)
def test_backward_f32_tiles(B, S, H_q, H_kv, d):
    _say(f"f32 backward B={B} S={S} H={H_q}/{H_kv} d={d}")
    seed = 9400 + S + d
    q = inputs.normal(seed, 0, (B, S, H_q, d), "f32")
    k = inputs.normal(seed, 1, (B, S, H_kv, d), "f32")
    v = inputs.normal(seed, 2, (B, S, H_kv, d), "f32")
    dout = inputs.normal(seed, 5, (B, S, H_q, d), "f32")
    for causal in (False, True):
        for scale in (1 / math.sqrt(d), -0.2):
            gq, gk, gv = _run(q, k, v, dout, scale, causal)
            sc = float(np.float32(scale))
            rq, rk, rv = oracle.attention_grad(q, k, v, dout, sc, causal=causal)
            allow = {"dq": dq_allowance(q, k, v, dout, sc, causal, dtype="f32"),
                     "dk": dk_allowance(q, k, v, dout, sc, causal, dtype="f32"), "dv": None}
            for name, got, ref in (("dq", gq, rq), ("dk", gk, rk), ("dv", gv, rv)):
                st = _check_grad(gpu_util.to_host_f64(got), ref, "f32", f"f32 {name} c={causal} scale={scale:.3g}",
                                 allow[name])
                _say(f"  {name} causal={causal} scale={scale:.3g} {st}")


def test_backward_grouped_equals_mha_on_repeated_kv():
    """dq equal bit for bit; dk/dv of the grouped call equal the per-head MHA
    gradients summed over each group (to fp32/bf16 rounding)."""
    B, S, H_q, H_kv, d = 1, 300, 8, 2, 128
    q = inputs.normal(93, 0, (B, S, H_q, d), "bf16", 0.5)
    k = inputs.normal(93, 1, (B, S, H_kv, d), "bf16", 0.5)
    v = inputs.normal(93, 2, (B, S, H_kv, d), "bf16", 0.5)
    dout = inputs.normal(93, 5, (B, S, H_q, d), "bf16", 1.0)
    gq, gk, gv = _run(q, k, v, dout, 0.09, True)
    mq, mk, mv = _run(q, np.repeat(k, 4, axis=2), np.repeat(v, 4, axis=2), dout, 0.09, True)
    assert torch.equal(gq.view(torch.int16), mq.view(torch.int16))
    mk_sum = gpu_util.to_host_f64(mk).reshape(B, S, H_kv, 4, d).sum(axis=3)
    mv_sum = gpu_util.to_host_f64(mv).reshape(B, S, H_kv, 4, d).sum(axis=3)
    assert np.linalg.norm(gpu_util.to_host_f64(gk) - mk_sum) <= 1e-2 * np.linalg.norm(mk_sum)
    assert np.linalg.norm(gpu_util.to_host_f64(gv) - mv_sum) <= 1e-2 * np.linalg.norm(mv_sum)


def test_backward_deterministic():
    B, S, H_q, H_kv, d = 1, 2048, 8, 2, 128
    q = inputs.normal(94, 0, (B, S, H_q, d), "bf16", 0.5)
    k = inputs.normal(94, 1, (B, S, H_kv, d), "bf16", 0.5)
    v = inputs.normal(94, 2, (B, S, H_kv, d), "bf16", 0.5)
    dout = inputs.normal(94, 5, (B, S, H_q, d), "bf16", 1.0)
    a = _run(q, k, v, dout, 0.088, True)
    b = _run(q, k, v, dout, 0.088, True)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("name,variant", [("sweep_s4096", "gqa"), ("encoder_s32k", "sqa"), ("causal_s131k", "sqa"),
                                          ("ragged_s200k", "sqa")])
def test_backward_full_size(name, variant):
    w = WORKLOADS[name]
    vv = w.variant(variant)
    _say(f"bwd workload {name}/{variant}")
    q, k, v, _ = make_inputs(w, variant)
    dout = inputs.normal(w.seed(variant), 5, q.shape, "bf16", 1.0)
    gq, gk, gv = _run(q, k, v, dout, w.scale, w.causal)
    rng = np.random.default_rng(w.seed(variant))
    rows = np.unique(np.concatenate([np.arange(4), np.arange(w.S - 4, w.S), rng.integers(0, w.S, 24)]))
    got = gpu_util.to_host_f64(gq[:, torch.from_numpy(rows).to(gq.device)])
    sc = float(np.float32(w.scale))
    ref = oracle.attention_grad_dq_rows(q, k, v, dout, sc, rows, causal=w.causal)
    st = _check_grad(got, ref, "bf16", f"{name} dq rows", dq_allowance(q, k, v, dout, sc, w.causal, rows=rows))
    _say(f"  dq rows {st}")
    # identities at full size (fp64 sums of the bf16 outputs)
    R = vv.H_q // vv.H_kv
    dk_sum = gk.double().sum(dim=1)                                       # [B, H_kv, d]
    dk_scale = gk.double().abs().sum(dim=1)
    assert float((dk_sum.abs() / dk_scale.clamp_min(1e-30)).max()) < 2e-2, "sum_j dk_j != 0"
    dv_sum = gv.double().sum(dim=1)
    g_sum = torch.from_numpy(inputs.bf16_bits_to_f32(dout).astype(np.float64)).to(gv.device)
    g_sum = g_sum.reshape(w.B, w.S, vv.H_kv, R, w.d).sum(dim=(1, 3))
    err = float((dv_sum - g_sum).norm() / g_sum.norm())
    assert err < 2e-2, f"sum_j dv_j vs summed dout: {err}"
    _say(f"  identities ok (dv rel {err:.2e})")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_autograd_attention_matches_attn_bwd_and_oracle(dtype):
    """sqa.attention under torch.autograd: the gradients equal those of a
    direct attn_bwd call on the same forward outputs (bit for bit; the same
    kernels), and the oracle's within the parity bounds."""
    B, S, H_q, H_kv, d = 1, 200, 4, 2, 64
    mul = 0.5 if dtype == "bf16" else 1.0
    q = inputs.normal(95, 0, (B, S, H_q, d), dtype, mul)
    k = inputs.normal(95, 1, (B, S, H_kv, d), dtype, mul)
    v = inputs.normal(95, 2, (B, S, H_kv, d), dtype, mul)
    g = inputs.normal(95, 5, (B, S, H_q, d), dtype, 1.0)
    scale = 0.11
    tq, tk, tv, tg = (gpu_util.to_device(a) for a in (q, k, v, g))
    for t in (tq, tk, tv):
        t.requires_grad_(True)
    out = sqa.attention(tq, tk, tv, scale=scale, causal=True)
    out.backward(tg)
    torch.cuda.synchronize()
    with torch.no_grad():
        o2, lse = sqa.attn_fwd(tq.detach(), tk.detach(), tv.detach(), scale=scale, causal=True, return_lse=True)
        dq, dk, dv = sqa.attn_bwd(tq.detach(), tk.detach(), tv.detach(), o2, tg, lse, scale=scale, causal=True)
    torch.cuda.synchronize()
    for a, b in ((out.detach(), o2), (tq.grad, dq), (tk.grad, dk), (tv.grad, dv)):
        assert torch.equal(a, b)
    sc = float(np.float32(scale))
    rq, rk, rv = oracle.attention_grad(q, k, v, g, sc, causal=True)
    allow = {"dq": dq_allowance(q, k, v, g, sc, True, dtype=dtype), "dk": dk_allowance(q, k, v, g, sc, True, dtype=dtype),
             "dv": None}
    for name, got, ref in (("dq", tq.grad, rq), ("dk", tk.grad, rk), ("dv", tv.grad, rv)):
        _check_grad(gpu_util.to_host_f64(got), ref, dtype, f"autograd {dtype} {name}", allow[name])
