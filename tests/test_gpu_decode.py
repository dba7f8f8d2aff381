"""GPU parity of the decode attention (one query token per sequence against
its key/value cache) with the fp64 oracle on identical inputs.

Bounds are the forward's (tests/parity.py): the same arithmetic (bf16 MFMA
products, fp32 accumulation, probabilities rounded to bf16, output rounded to
bf16) plus the split merge, which only rescales fp32 partial sums by exact
powers of two and adds a few of them.  The log-normaliser uses the forward's
LSE bounds.  Cache positions at or past a sequence's length are filled with
NaN in several cases: any read of them would poison the output.
"""
import math
import sys

import numpy as np
import pytest

import inputs
import oracle
from inputs.configs import DECODE_WORKLOADS, make_decode_inputs
from tests import parity

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
import reduced_query_head_amd as sqa  # noqa: E402
from tests import gpu_util  # noqa: E402

LSE_BOUNDS = dict(max_abs=2.5e-3, mean_abs=1e-3)
BF16_NAN = np.uint16(0x7FC0)


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _run(q, k, v, lens, scale):
    dq, dk, dv = gpu_util.to_device(q), gpu_util.to_device(k), gpu_util.to_device(v)
    dl = None if lens is None else torch.from_numpy(np.asarray(lens, dtype=np.int32)).cuda()
    out, lse = sqa.attn_decode(dq, dk, dv, seqlens=dl, scale=scale, return_lse=True)
    torch.cuda.synchronize()
    return out, lse


def _poison_tail(k, v, lens):
    """NaN in every cache position at or past the sequence's length."""
    S_max = k.shape[1]
    for b, n in enumerate(lens):
        n = max(0, min(int(n), S_max))
        k[b, n:] = BF16_NAN
        v[b, n:] = BF16_NAN


def _check(out, lse, q, k, v, lens, scale, what):
    ref, ref_lse = oracle.decode(q, k, v, float(np.float32(scale)), seqlens=lens)
    got = gpu_util.to_host_f64(out)
    got_lse = lse.double().cpu().numpy()
    empty = np.zeros(q.shape[0], dtype=bool) if lens is None else (np.asarray(lens) <= 0)
    if empty.any():
        assert (got[empty] == 0).all(), f"{what}: empty cache must give zeros"
        assert np.isneginf(got_lse[empty]).all(), f"{what}: empty cache must give lse = -inf"
    full = ~empty
    if full.any():
        st = parity.check(got[full], ref[full], "bf16", what)
        dl = np.abs(got_lse[full] - ref_lse[full])
        assert np.isfinite(got_lse[full]).all()
        assert dl.max() <= LSE_BOUNDS["max_abs"] and dl.mean() <= LSE_BOUNDS["mean_abs"], f"{what}: lse {dl.max()}"
        return st
    return None


CASES = [
    # B, S_max, H_q, H_kv, d, lens
    (1, 1, 1, 1, 128, [1]),
    (2, 40, 4, 4, 128, [40, 33]),
    (3, 100, 8, 2, 64, [100, 1, 32]),
    (2, 257, 32, 8, 128, [257, 200]),
    (2, 300, 32, 1, 128, [300, 64]),          # MQA, 32 heads per group
    (1, 500, 64, 1, 64, [500]),               # 64 heads per group: two head blocks
    (2, 1000, 40, 8, 32, [999, 0]),           # 5 heads per group, one empty cache
    (4, 2048, 16, 4, 128, [2048, 5000, 31, 1500]),   # a length above S_max counts as S_max
    (1, 9000, 8, 8, 128, None),               # no length array: S_max everywhere
    (3, 33000, 32, 8, 128, [33000, 20001, 65]),
    # many short sequences: seeded lengths in [0, 600] with 0, 1 and over-long entries
    (64, 512, 32, 8, 128, [0, 1, 600] + [int(x) for x in np.random.default_rng(64).integers(0, 601, 61)]),
    (2, 1000, 128, 1, 64, [1000, 517]),      # 128 heads per group: four head blocks
    # shared splits (fewer than 4 K/V heads) over long caches: many splits,
    # lengths ending inside a split and inside a wave's quarter of one
    (3, 40000, 32, 1, 128, [40000, 12345, 257]),
    (2, 70001, 8, 2, 64, [70001, 33333]),
]


@pytest.mark.parametrize("B,S_max,H_q,H_kv,d,lens", CASES)
def test_decode_small_shapes(B, S_max, H_q, H_kv, d, lens):
    _say(f"decode B={B} S_max={S_max} H={H_q}/{H_kv} d={d} lens={lens}")
    seed = 7000 + S_max + H_q * 3 + d
    q = inputs.normal(seed, 0, (B, H_q, d), "bf16", 0.5)
    k = inputs.normal(seed, 1, (B, S_max, H_kv, d), "bf16", 0.5)
    v = inputs.normal(seed, 2, (B, S_max, H_kv, d), "bf16", 0.5)
    if lens is not None:
        _poison_tail(k, v, lens)
    out, lse = _run(q, k, v, lens, 1 / math.sqrt(d))
    st = _check(out, lse, q, k, v, lens, 1 / math.sqrt(d), f"decode {B}x{S_max} {H_q}/{H_kv} d={d}")
    _say(f"  {st}")


@pytest.mark.parametrize("scale", [-0.3, 0.0, 0.7])
def test_decode_scale_values(scale):
    B, S_max, H_q, H_kv, d = 2, 700, 8, 2, 128
    q = inputs.normal(71, 0, (B, H_q, d), "bf16", 0.5)
    k = inputs.normal(71, 1, (B, S_max, H_kv, d), "bf16", 0.5)
    v = inputs.normal(71, 2, (B, S_max, H_kv, d), "bf16", 0.5)
    out, lse = _run(q, k, v, [700, 333], scale)
    _check(out, lse, q, k, v, [700, 333], scale, f"decode scale={scale}")


def test_decode_peaked_scores():
    """Large scores (a few keys times 8, scale 1): the running maximum moves
    and the splits carry very different maxima into the merge."""
    B, S_max, H_q, H_kv, d = 2, 5000, 16, 4, 128
    q = inputs.normal(72, 0, (B, H_q, d), "bf16", 0.5)
    k = inputs.normal(72, 1, (B, S_max, H_kv, d), "bf16", 0.5)
    v = inputs.normal(72, 2, (B, S_max, H_kv, d), "bf16", 0.5)
    pos = inputs.select_positions(72, 3, S_max, 50)
    inputs.scale_positions_bf16(k, pos, 8.0)
    out, lse = _run(q, k, v, [5000, 4321], 0.25)
    _check(out, lse, q, k, v, [5000, 4321], 0.25, "decode peaked")


def test_decode_deterministic_and_matches_forward_last_row():
    B, S_max, H_q, H_kv, d = 2, 3000, 16, 4, 128
    q = inputs.normal(73, 0, (B, H_q, d), "bf16", 0.5)
    k = inputs.normal(73, 1, (B, S_max, H_kv, d), "bf16", 0.5)
    v = inputs.normal(73, 2, (B, S_max, H_kv, d), "bf16", 0.5)
    a, la = _run(q, k, v, None, 0.088)
    b, lb = _run(q, k, v, None, 0.088)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)) and torch.equal(la, lb)
    # the GPU forward's causal last row sees the same keys: both within the bound of each other
    qf = np.zeros((B, S_max, H_q, d), dtype=np.uint16)
    qf[:, -1] = q
    fo = gpu_util.run(qf, k, v, 0.088, True)
    last = gpu_util.to_host_f64(fo[:, -1])
    st = parity.error_stats(gpu_util.to_host_f64(a), last)
    assert st["rel_l2"] < 1e-2 and st["max_abs"] < 2e-2, st


def test_decode_grouped_equals_mha_on_repeated_cache():
    B, S_max, H_q, H_kv, d = 2, 1500, 16, 2, 64
    q = inputs.normal(74, 0, (B, H_q, d), "bf16", 0.5)
    k = inputs.normal(74, 1, (B, S_max, H_kv, d), "bf16", 0.5)
    v = inputs.normal(74, 2, (B, S_max, H_kv, d), "bf16", 0.5)
    a, _ = _run(q, k, v, [1500, 777], 0.125)
    b, _ = _run(q, np.repeat(k, 8, axis=2), np.repeat(v, 8, axis=2), [1500, 777], 0.125)
    st = parity.error_stats(gpu_util.to_host_f64(a), gpu_util.to_host_f64(b))
    assert st["rel_l2"] < 1e-2 and st["max_abs"] < 2e-2, st


@pytest.mark.parametrize("variant", ["gqa", "mha", "mqa", "sqa"])
def test_decode_full_size(variant):
    w = DECODE_WORKLOADS["decode_s128k"]
    _say(f"decode workload {w.name}/{variant}")
    q, k, v, lens = make_decode_inputs(w, variant)
    out, lse = _run(q, k, v, lens, w.scale)
    st = _check(out, lse, q, k, v, lens, w.scale, f"{w.name}/{variant}")
    _say(f"  {st}")


@pytest.mark.parametrize("d", [32, 64, 128])
def test_decode_f32(d):
    """fp32 path against the oracle at the fp32 bounds (max 1e-4, relative L2 1e-5)."""
    B, S_max, H_q, H_kv = 3, 300, 8, 2
    q = inputs.normal(80 + d, 0, (B, H_q, d), "f32")
    k = inputs.normal(80 + d, 1, (B, S_max, H_kv, d), "f32")
    v = inputs.normal(80 + d, 2, (B, S_max, H_kv, d), "f32")
    lens = [300, 1, 0]
    dq, dk, dv = gpu_util.to_device(q), gpu_util.to_device(k), gpu_util.to_device(v)
    dl = torch.from_numpy(np.asarray(lens, dtype=np.int32)).cuda()
    out, lse = sqa.attn_decode(dq, dk, dv, seqlens=dl, scale=-1 / math.sqrt(d), return_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.decode(q, k, v, float(np.float32(-1 / math.sqrt(d))), seqlens=lens)
    got = out.double().cpu().numpy()
    assert (got[2] == 0).all() and np.isneginf(lse[2].cpu().numpy()).all()
    parity.check(got[:2], ref[:2], "f32", f"decode f32 d={d}")
    assert np.abs(lse[:2].double().cpu().numpy() - ref_lse[:2]).max() < 2e-5
# fp32 on the matrix cores at longer caches: independent waves (eight K/V
# heads), the shared four-wave splits (one K/V head), ragged lengths.
F32_LONG = [(2, 3000, 32, 8, 128, [3000, 1777]), (1, 5000, 32, 1, 64, [4999]), (3, 2100, 6, 2, 32, [2100, 64, 65])]


@pytest.mark.parametrize("B,S_max,H_q,H_kv,d,lens", F32_LONG)
def test_decode_f32_long(B, S_max, H_q, H_kv, d, lens):
    _say(f"decode f32 B={B} S_max={S_max} H={H_q}/{H_kv} d={d} lens={lens}")
    seed = 8300 + S_max + d
    q = inputs.normal(seed, 0, (B, H_q, d), "f32")
    k = inputs.normal(seed, 1, (B, S_max, H_kv, d), "f32")
    v = inputs.normal(seed, 2, (B, S_max, H_kv, d), "f32")
    dq, dk, dv = gpu_util.to_device(q), gpu_util.to_device(k), gpu_util.to_device(v)
    dl = torch.from_numpy(np.asarray(lens, dtype=np.int32)).cuda()
    for scale in (1 / math.sqrt(d), -0.3):
        out, lse = sqa.attn_decode(dq, dk, dv, seqlens=dl, scale=scale, return_lse=True)
        torch.cuda.synchronize()
        ref, ref_lse = oracle.decode(q, k, v, float(np.float32(scale)), seqlens=lens)
        parity.check(out.double().cpu().numpy(), ref, "f32", f"decode f32 scale={scale}")
        assert np.abs(lse.double().cpu().numpy() - ref_lse).max() < 2e-5


