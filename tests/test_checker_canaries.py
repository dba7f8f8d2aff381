"""The parity checker must reject plausible wrong outputs.

Each wrong output is made on the CPU from the oracle itself (zeros, swapped
heads, the interleaved head map, a non-causal result for a causal request,
one 64-key-tile's worth of rows left unwritten) and compared against the
correct oracle output at a sequence length where |o| is small.
"""
import numpy as np
import pytest

import inputs
import oracle
from tests.parity import check, error_stats


@pytest.fixture(scope="module")
def case():
    B, S, H_q, H_kv, d = 1, 2048, 4, 2, 64
    q = inputs.normal(77, 0, (B, S, H_q, d), "bf16", 0.5)
    k = inputs.normal(77, 1, (B, S, H_kv, d), "bf16", 0.5)
    v = inputs.normal(77, 2, (B, S, H_kv, d), "bf16", 0.5)
    rows = np.unique(np.concatenate([np.arange(0, 64), np.arange(S - 64, S),
                                     np.random.default_rng(3).integers(0, S, 128)]))
    ref_nc = oracle.attention(q, k, v, 0.125, causal=False, rows=rows)
    ref_c = oracle.attention(q, k, v, 0.125, causal=True, rows=rows)
    return dict(q=q, k=k, v=v, rows=rows, ref_nc=ref_nc, ref_c=ref_c)


def _must_fail(got, ref):
    with pytest.raises(AssertionError):
        check(got, ref, "bf16")


def test_correct_output_passes_after_bf16_rounding(case):
    ref = case["ref_nc"]
    got = inputs.bf16_bits_to_f32(inputs.f32_to_bf16_bits(ref.astype(np.float32)))
    check(got, ref, "bf16")


def test_zero_output_fails(case):
    _must_fail(np.zeros_like(case["ref_nc"]), case["ref_nc"])
    # zeros also fail the relative check on their own
    assert error_stats(np.zeros_like(case["ref_nc"]), case["ref_nc"])["rel_l2"] == 1.0


def test_swapped_heads_fail(case):
    _must_fail(case["ref_nc"][:, :, [1, 0, 2, 3], :], case["ref_nc"])


def test_interleaved_head_map_fails(case):
    q, k, v = case["q"], case["k"], case["v"]
    wrong = oracle.attention(q, np.tile(k, (1, 1, 2, 1)), np.tile(v, (1, 1, 2, 1)), 0.125, rows=case["rows"])
    _must_fail(wrong, case["ref_nc"])


def test_noncausal_for_causal_fails(case):
    _must_fail(case["ref_nc"], case["ref_c"])


def test_one_tile_unwritten_fails(case):
    got = case["ref_nc"].copy()
    got[:, -64:] = 0.0
    _must_fail(got, case["ref_nc"])
