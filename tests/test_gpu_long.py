"""Sizes past the workloads, checked against the oracle on sampled rows: a
2^20-token causal sequence (five times the longest workload; key and tile
offsets, causal chunk order and the log-normaliser at the far end), a batch
of 96 sequences, and decode against a 2^20-position cache."""
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

LSE_MAX = 2.5e-3


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_forward_million_tokens_causal():
    B, S, H_q, H_kv, d = 1, 1 << 20, 2, 1, 64
    _say(f"forward B={B} S={S} H={H_q}/{H_kv} d={d} causal")
    q = inputs.normal(95, 0, (B, S, H_q, d), "bf16", 0.5)
    k = inputs.normal(95, 1, (B, S, H_kv, d), "bf16", 0.5)
    v = inputs.normal(95, 2, (B, S, H_kv, d), "bf16", 0.5)
    dq, dk, dv = (gpu_util.to_device(a) for a in (q, k, v))
    o, lse = sqa.attn_fwd(dq, dk, dv, scale=1 / math.sqrt(d), causal=True, return_lse=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(95)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, (1 << 19) - 1, 1 << 19], np.arange(S - 8, S),
                                     rng.integers(0, S, 8)]))
    idx = torch.from_numpy(rows).to(o.device)
    got = gpu_util.to_host_f64(o[:, idx])
    got_lse = lse[:, idx].double().cpu().numpy()
    del o, lse, dq, dk, dv
    sc = float(np.float32(1 / math.sqrt(d)))
    ref = oracle.attention(q, k, v, sc, causal=True, rows=rows)
    ref_lse = oracle.lse(q, k, sc, causal=True, rows=rows)
    st = parity.check(got, ref, "bf16", "S=2^20 causal rows")
    assert np.abs(got_lse - ref_lse).max() <= LSE_MAX
    _say(f"  rows={rows.size} {st}")


def test_forward_wide_batch():
    B, S, H_q, H_kv, d = 96, 1000, 8, 2, 128
    _say(f"forward B={B} S={S} H={H_q}/{H_kv} d={d}")
    q = inputs.normal(96, 0, (B, S, H_q, d), "bf16", 0.5)
    k = inputs.normal(96, 1, (B, S, H_kv, d), "bf16", 0.5)
    v = inputs.normal(96, 2, (B, S, H_kv, d), "bf16", 0.5)
    o = gpu_util.run(q, k, v, 1 / math.sqrt(d), False)
    bsel = [0, 1, 47, 95]
    rows = np.array([0, 31, 32, 511, 999])
    got = gpu_util.to_host_f64(o[bsel][:, torch.from_numpy(rows).to(o.device)])
    ref = oracle.attention(q[bsel], k[bsel], v[bsel], float(np.float32(1 / math.sqrt(d))), causal=False, rows=rows)
    st = parity.check(got, ref, "bf16", "B=96 rows")
    _say(f"  {st}")


def test_decode_million_position_cache():
    B, S_max, H_q, H_kv, d = 2, 1 << 20, 16, 2, 128
    _say(f"decode B={B} S_max={S_max} H={H_q}/{H_kv} d={d}")
    q = inputs.normal(97, 0, (B, H_q, d), "bf16", 0.5)
    k = inputs.normal(97, 1, (B, S_max, H_kv, d), "bf16", 0.5)
    v = inputs.normal(97, 2, (B, S_max, H_kv, d), "bf16", 0.5)
    lens = [S_max, 700001]
    dq, dk, dv = (gpu_util.to_device(a) for a in (q, k, v))
    dl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    out, lse = sqa.attn_decode(dq, dk, dv, seqlens=dl, scale=0.088, return_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.decode(q, k, v, float(np.float32(0.088)), seqlens=lens)
    st = parity.check(gpu_util.to_host_f64(out), ref, "bf16", "decode S_max=2^20")
    assert np.abs(lse.double().cpu().numpy() - ref_lse).max() <= LSE_MAX
    _say(f"  {st}")


def test_forward_tensors_past_4_gib():
    """q and out of 2^19 x 32 x 128 bf16 elements (4 GiB each, element
    offsets up to 2^31): the rows at the far end need 64-bit addressing.
    Inputs are a seeded 4096-row block repeated along the sequence (the
    causal mask still makes every row's softmax different)."""
    B, S, H_q, H_kv, d, blk = 1, 1 << 19, 32, 8, 128, 4096
    _say(f"forward B={B} S={S} H={H_q}/{H_kv} d={d} causal, q = 4 GiB")
    reps = S // blk
    q = np.tile(inputs.normal(98, 0, (B, blk, H_q, d), "bf16", 0.5), (1, reps, 1, 1))
    k = np.tile(inputs.normal(98, 1, (B, blk, H_kv, d), "bf16", 0.5), (1, reps, 1, 1))
    v = np.tile(inputs.normal(98, 2, (B, blk, H_kv, d), "bf16", 0.5), (1, reps, 1, 1))
    dq, dk, dv = (gpu_util.to_device(a) for a in (q, k, v))
    o, lse = sqa.attn_fwd(dq, dk, dv, scale=1 / math.sqrt(d), causal=True, return_lse=True)
    torch.cuda.synchronize()
    rows = np.array([0, 4095, 4096, (1 << 18) + 7, S - 33, S - 1])
    idx = torch.from_numpy(rows).to(o.device)
    got = gpu_util.to_host_f64(o[:, idx])
    got_lse = lse[:, idx].double().cpu().numpy()
    del o, lse, dq, dk, dv
    torch.cuda.empty_cache()
    sc = float(np.float32(1 / math.sqrt(d)))
    ref = oracle.attention(q, k, v, sc, causal=True, rows=rows)
    ref_lse = oracle.lse(q, k, sc, causal=True, rows=rows)
    st = parity.check(got, ref, "bf16", "q, out = 4 GiB")
    assert np.abs(got_lse - ref_lse).max() <= LSE_MAX
    _say(f"  {st}")


def test_backward_tensors_past_4_gib():
    """The backward at the same 4 GiB shape: dq at rows across the sequence
    against the oracle, and the two identities that hold at any size
    (sum_j dk_j = 0 since every row of dS sums to zero; sum_j dv_j = the
    summed dout of the group's query heads since every row of P sums to one)."""
    from tests.test_gpu_backward import _check_grad, dq_allowance
    B, S, H_q, H_kv, d, blk = 1, 1 << 19, 32, 8, 128, 4096
    _say(f"backward B={B} S={S} H={H_q}/{H_kv} d={d} causal, q = 4 GiB")
    reps = S // blk
    q = np.tile(inputs.normal(99, 0, (B, blk, H_q, d), "bf16", 0.5), (1, reps, 1, 1))
    k = np.tile(inputs.normal(99, 1, (B, blk, H_kv, d), "bf16", 0.5), (1, reps, 1, 1))
    v = np.tile(inputs.normal(99, 2, (B, blk, H_kv, d), "bf16", 0.5), (1, reps, 1, 1))
    g = np.tile(inputs.normal(99, 5, (B, blk, H_q, d), "bf16", 1.0), (1, reps, 1, 1))
    scale = 1 / math.sqrt(d)
    dq_, dk_, dv_, dg = (gpu_util.to_device(a) for a in (q, k, v, g))
    o, lse = sqa.attn_fwd(dq_, dk_, dv_, scale=scale, causal=True, return_lse=True)
    gq, gk, gv = sqa.attn_bwd(dq_, dk_, dv_, o, dg, lse, scale=scale, causal=True)
    torch.cuda.synchronize()
    del o, lse, dq_, dk_, dv_
    rows = np.array([0, 4095, 4096, (1 << 18) + 7, S - 33, S - 1])
    got = gpu_util.to_host_f64(gq[:, torch.from_numpy(rows).to(gq.device)])
    sc = float(np.float32(scale))
    ref = oracle.attention_grad_dq_rows(q, k, v, g, sc, rows, causal=True)
    st = _check_grad(got, ref, "bf16", "dq rows, 4 GiB", dq_allowance(q, k, v, g, sc, True, rows=rows))
    _say(f"  dq rows {st}")
    R = H_q // H_kv
    dk_sum = gk.double().sum(dim=1)
    dk_scale = gk.double().abs().sum(dim=1)
    assert float((dk_sum.abs() / dk_scale.clamp_min(1e-30)).max()) < 2e-2, "sum_j dk_j != 0"
    dv_sum = gv.double().sum(dim=1)
    g_sum = dg.double().reshape(B, S, H_kv, R, d).sum(dim=(1, 3))
    err = float((dv_sum - g_sum).norm() / g_sum.norm())
    assert err < 2e-2, f"sum_j dv_j vs summed dout: {err}"
    _say(f"  identities ok (dv rel {err:.2e})")
