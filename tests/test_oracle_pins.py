"""Pins for the oracle: facts fixed by the pages or by mathematics.

None of these re-types the oracle's loop.  They check it against hand-derived
closed forms (tests/golden), a library routine (torch's CPU
scaled_dot_product_attention in fp64, the call the GQA explainer's PyTorch
module makes), algebraic invariants of softmax attention, and the special
cases the pages name (G = H is MHA, G = 1 is MQA).  Each is chosen so that a
plausible slip in the oracle (a wrong head map, a transposed score, a causal
mask off by one, a dropped scale, a missing max shift, bad bf16 decoding)
fails at least one of them.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import inputs
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.txt")


def _num(tok):
    val = 1.0
    for factor in tok.split("*"):
        if factor == "ln2":
            val *= math.log(2.0)
        else:
            val *= float(Fraction(factor))
    return val


def _golden_cases():
    cases, cur, key = [], None, None
    with open(GOLDEN) as f:
        for raw in f:
            line = raw.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            if parts[0] == "case":
                cur = {"name": parts[1]}
            elif parts[0] == "shape":
                cur["shape"] = tuple(int(x) for x in parts[1:])
            elif parts[0] in ("scale", "causal"):
                cur[parts[0]] = _num(parts[1])
            elif parts[0] in ("q", "k", "v", "out"):
                key = parts[0]
            elif parts[0] == "end":
                cases.append(cur)
            else:
                cur[key] = np.array([_num(t) for t in parts], dtype=np.float64)
    return cases


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_hand_derived_cases(case):
    B, S, H_q, H_kv, d = case["shape"]
    q = case["q"].reshape(B, S, H_q, d)
    k = case["k"].reshape(B, S, H_kv, d)
    v = case["v"].reshape(B, S, H_kv, d)
    out = oracle.attention(q, k, v, case["scale"], causal=bool(case["causal"]))
    np.testing.assert_allclose(out.ravel(), case["out"], rtol=1e-14, atol=1e-14)


def _rand(rng, B, S, H, d, std=1.0):
    return rng.standard_normal((B, S, H, d)) * std


def _torch_sdpa(q, k, v, scale, causal):
    """torch CPU fp64 SDPA on K/V expanded to the query heads (BHSD)."""
    R = q.shape[2] // k.shape[2]
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(R, dim=1)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(R, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(
        tq.contiguous(), tk.contiguous(), tv.contiguous(), is_causal=causal, scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,S,H_q,H_kv,d", [(1, 7, 4, 2, 8), (2, 13, 6, 3, 5), (1, 33, 8, 1, 16),
                                             (2, 9, 3, 3, 4)])
def test_matches_torch_sdpa_fp64(B, S, H_q, H_kv, d, causal):
    rng = np.random.default_rng(1000 + S * 7 + H_q)
    q, k, v = _rand(rng, B, S, H_q, d), _rand(rng, B, S, H_kv, d), _rand(rng, B, S, H_kv, d)
    scale = 0.37
    ours = oracle.attention(q, k, v, scale, causal=causal)
    ref = _torch_sdpa(q, k, v, scale, causal)
    np.testing.assert_allclose(ours, ref, rtol=1e-12, atol=1e-13)


def test_textbook_row_normalised_form_without_shift():
    """o = D(A)^-1 A V with A = exp(scale Q K^T), masked entries 0, no max shift."""
    rng = np.random.default_rng(7)
    for causal in (False, True):
        q, k, v = _rand(rng, 1, 11, 2, 6), _rand(rng, 1, 11, 2, 6), _rand(rng, 1, 11, 2, 6)
        ours = oracle.attention(q, k, v, 0.5, causal=causal)
        for h in range(2):
            A = np.exp(0.5 * (q[0, :, h, :] @ k[0, :, h, :].T))
            if causal:
                A = np.tril(A)
            O = np.diag(1.0 / A.sum(axis=1)) @ A @ v[0, :, h, :]
            np.testing.assert_allclose(ours[0, :, h, :], O, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_grouped_equals_mha_on_repeated_kv(causal):
    """GQA(q, k, v) == MHA(q, expand(k), expand(v)), expand as in the page's module."""
    rng = np.random.default_rng(11)
    B, S, H_q, H_kv, d = 2, 17, 8, 2, 8
    q, k, v = _rand(rng, B, S, H_q, d), _rand(rng, B, S, H_kv, d), _rand(rng, B, S, H_kv, d)
    R = H_q // H_kv
    # unsqueeze/expand/reshape along the head axis: K/V head g -> heads gR..gR+R-1
    k_rep = np.repeat(k, R, axis=2)
    v_rep = np.repeat(v, R, axis=2)
    grouped = oracle.attention(q, k, v, 0.3, causal=causal)
    mha = oracle.attention(q, k_rep, v_rep, 0.3, causal=causal)
    assert np.array_equal(grouped, mha)
    # the interleaved map (h -> h mod H_kv) is a different function
    inter = oracle.attention(q, np.tile(k, (1, 1, R, 1)), np.tile(v, (1, 1, R, 1)), 0.3, causal=causal)
    assert np.abs(inter - grouped).max() > 1e-3


def test_mqa_every_head_reads_the_single_kv_head():
    rng = np.random.default_rng(12)
    B, S, H_q, d = 1, 10, 5, 4
    q, k, v = _rand(rng, B, S, H_q, d), _rand(rng, B, S, 1, d), _rand(rng, B, S, 1, d)
    full = oracle.attention(q, k, v, 0.7)
    for h in range(H_q):
        single = oracle.attention(q[:, :, h:h + 1, :].copy(), k, v, 0.7)
        assert np.array_equal(full[:, :, h:h + 1, :], single)


@pytest.mark.parametrize("causal", [False, True])
def test_constant_scores_give_mean_of_v(causal):
    rng = np.random.default_rng(13)
    B, S, H_q, H_kv, d = 2, 9, 4, 2, 3
    q = np.zeros((B, S, H_q, d))
    k, v = _rand(rng, B, S, H_kv, d), _rand(rng, B, S, H_kv, d)
    out = oracle.attention(q, k, v, 1.3, causal=causal)
    for h in range(H_q):
        g = h // (H_q // H_kv)
        if causal:
            expect = np.cumsum(v[:, :, g, :], axis=1) / np.arange(1, S + 1)[None, :, None]
        else:
            expect = np.broadcast_to(v[:, :, g, :].mean(axis=1, keepdims=True), (B, S, d))
        np.testing.assert_allclose(out[:, :, h, :], expect, rtol=1e-13, atol=1e-14)


def test_causal_row_zero_is_v0():
    rng = np.random.default_rng(14)
    B, S, H_q, H_kv, d = 2, 6, 6, 3, 5
    q, k, v = _rand(rng, B, S, H_q, d, 5.0), _rand(rng, B, S, H_kv, d, 5.0), _rand(rng, B, S, H_kv, d)
    out = oracle.attention(q, k, v, 1.0, causal=True)
    for h in range(H_q):
        assert np.array_equal(out[:, 0, h, :], v[:, 0, h // 2, :])


def test_causal_row_equals_noncausal_on_prefix():
    """Row i of the causal result is the non-causal result on positions 0..i."""
    rng = np.random.default_rng(15)
    B, S, H_q, H_kv, d = 1, 12, 2, 1, 4
    q, k, v = _rand(rng, B, S, H_q, d), _rand(rng, B, S, H_kv, d), _rand(rng, B, S, H_kv, d)
    causal = oracle.attention(q, k, v, 0.9, causal=True)
    for i in range(S):
        pre = oracle.attention(q[:, :i + 1].copy(), k[:, :i + 1].copy(), v[:, :i + 1].copy(), 0.9)
        np.testing.assert_allclose(causal[:, i], pre[:, i], rtol=1e-14, atol=1e-15)


def test_key_shift_invariance_forces_max_subtraction():
    """Adding u to every key adds the same q.u to each score of a row: no change.

    With |scale * q.u| near 1000, exp() overflows fp64 unless the row maximum
    is subtracted first, so this also pins the stabilisation.
    """
    rng = np.random.default_rng(16)
    B, S, H, d = 1, 8, 2, 4
    q = np.abs(_rand(rng, B, S, H, d)) + 1.0
    k, v = _rand(rng, B, S, H, d), _rand(rng, B, S, H, d)
    base = oracle.attention(q, k, v, 1.0)
    shifted = oracle.attention(q, k + 300.0, v, 1.0)
    assert np.isfinite(shifted).all()
    np.testing.assert_allclose(shifted, base, rtol=1e-9, atol=1e-9)


def test_affine_values():
    rng = np.random.default_rng(17)
    q, k, v = _rand(rng, 1, 10, 4, 3), _rand(rng, 1, 10, 2, 3), _rand(rng, 1, 10, 2, 3)
    for causal in (False, True):
        a = oracle.attention(q, k, v, 0.8, causal=causal)
        b = oracle.attention(q, k, 2.5 * v - 1.75, 0.8, causal=causal)
        np.testing.assert_allclose(b, 2.5 * a - 1.75, rtol=1e-12, atol=1e-12)


def test_permutations_noncausal():
    rng = np.random.default_rng(18)
    q, k, v = _rand(rng, 1, 15, 2, 4), _rand(rng, 1, 15, 1, 4), _rand(rng, 1, 15, 1, 4)
    base = oracle.attention(q, k, v, 0.6)
    perm = rng.permutation(15)
    keys_permuted = oracle.attention(q, k[:, perm].copy(), v[:, perm].copy(), 0.6)
    np.testing.assert_allclose(keys_permuted, base, rtol=1e-13, atol=1e-14)
    rows_permuted = oracle.attention(q[:, perm].copy(), k, v, 0.6)
    np.testing.assert_allclose(rows_permuted, base[:, perm], rtol=1e-13, atol=1e-14)


def test_single_key_and_two_key_closed_forms():
    rng = np.random.default_rng(19)
    q, k, v = _rand(rng, 1, 1, 3, 4), _rand(rng, 1, 1, 3, 4), _rand(rng, 1, 1, 3, 4)
    assert np.array_equal(oracle.attention(q, k, v, 2.0), v)
    q, k, v = _rand(rng, 1, 2, 1, 3), _rand(rng, 1, 2, 1, 3), _rand(rng, 1, 2, 1, 3)
    out = oracle.attention(q, k, v, 0.25)
    for i in range(2):
        s0 = 0.25 * float(q[0, i, 0] @ k[0, 0, 0])
        s1 = 0.25 * float(q[0, i, 0] @ k[0, 1, 0])
        w1 = 1.0 / (1.0 + math.exp(s0 - s1))
        expect = (1.0 - w1) * v[0, 0, 0] + w1 * v[0, 1, 0]
        np.testing.assert_allclose(out[0, i, 0], expect, rtol=1e-13, atol=1e-14)


def test_peaked_row_picks_its_value():
    """One key far above the rest: the output tends to that key's value."""
    rng = np.random.default_rng(20)
    q = np.ones((1, 4, 1, 2))
    k = _rand(rng, 1, 4, 1, 2) * 0.01
    k[0, 2, 0, :] = 40.0
    v = _rand(rng, 1, 4, 1, 2)
    out = oracle.attention(q, k, v, 1.0)
    np.testing.assert_allclose(out[0, :, 0, :], np.broadcast_to(v[0, 2, 0, :], (4, 2)), atol=1e-30, rtol=1e-30)


def test_batches_are_independent():
    rng = np.random.default_rng(21)
    q, k, v = _rand(rng, 3, 6, 2, 4), _rand(rng, 3, 6, 2, 4), _rand(rng, 3, 6, 2, 4)
    full = oracle.attention(q, k, v, 0.5, causal=True)
    for b in range(3):
        one = oracle.attention(q[b:b + 1].copy(), k[b:b + 1].copy(), v[b:b + 1].copy(), 0.5, causal=True)
        assert np.array_equal(full[b:b + 1], one)


def test_row_subset_equals_full_rows():
    rng = np.random.default_rng(22)
    q, k, v = _rand(rng, 2, 20, 4, 4), _rand(rng, 2, 20, 2, 4), _rand(rng, 2, 20, 2, 4)
    rows = np.array([0, 5, 19, 7])
    for causal in (False, True):
        full = oracle.attention(q, k, v, 0.5, causal=causal)
        sub = oracle.attention(q, k, v, 0.5, causal=causal, rows=rows)
        assert np.array_equal(sub, full[:, rows])


def test_bf16_inputs_decode_exactly():
    """bf16 bits give the same result as their exact fp32 widening."""
    bits_q = inputs.normal(5, 0, (1, 9, 4, 8), "bf16", 0.5)
    bits_k = inputs.normal(5, 1, (1, 9, 2, 8), "bf16", 0.5)
    bits_v = inputs.normal(5, 2, (1, 9, 2, 8), "bf16", 0.5)
    # decode by hand: sign, exponent and mantissa of each bf16 value
    def decode(bits):
        b = bits.astype(np.int64)
        sign = np.where(b >> 15, -1.0, 1.0)
        exp = (b >> 7) & 0xFF
        man = b & 0x7F
        return sign * np.where(exp == 0, man / 128.0 * 2.0 ** -126, (1 + man / 128.0) * 2.0 ** (exp - 127))
    a = oracle.attention(bits_q, bits_k, bits_v, 0.35, causal=True)
    b = oracle.attention(decode(bits_q), decode(bits_k), decode(bits_v), 0.35, causal=True)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("causal", [False, True])
def test_pair_count_is_the_flop_model(causal):
    rng = np.random.default_rng(23)
    B, S, H_q, H_kv, d = 2, 11, 6, 2, 3
    q, k, v = _rand(rng, B, S, H_q, d), _rand(rng, B, S, H_kv, d), _rand(rng, B, S, H_kv, d)
    _, pairs = oracle.attention(q, k, v, 1.0, causal=causal, return_pairs=True)
    expect = B * H_q * (S * (S + 1) // 2 if causal else S * S)
    assert pairs == expect


def test_rejects_non_divisible_heads():
    q = np.zeros((1, 2, 3, 4))
    k = np.zeros((1, 2, 2, 4))
    with pytest.raises(ValueError):
        oracle.attention(q, k, k, 1.0)


def test_thread_count_does_not_change_result():
    rng = np.random.default_rng(24)
    q, k, v = _rand(rng, 1, 40, 4, 8), _rand(rng, 1, 40, 2, 8), _rand(rng, 1, 40, 2, 8)
    a = oracle.attention(q, k, v, 0.5, causal=True, n_threads=1)
    b = oracle.attention(q, k, v, 0.5, causal=True, n_threads=4)
    assert np.array_equal(a, b)


# ---- row log-normaliser (log-sum-exp of the scaled scores) ------------------

def test_lse_matches_torch_logsumexp():
    rng = np.random.default_rng(30)
    B, S, H_q, H_kv, d = 2, 13, 6, 2, 5
    q, k = _rand(rng, B, S, H_q, d), _rand(rng, B, S, H_kv, d)
    for causal in (False, True):
        ours = oracle.lse(q, k, 0.41, causal=causal)
        kk = np.repeat(k, H_q // H_kv, axis=2)
        sc = 0.41 * torch.einsum("bihe,bjhe->bhij", torch.from_numpy(q), torch.from_numpy(kk))
        if causal:
            sc = sc.masked_fill(torch.ones(S, S, dtype=torch.bool).triu(1), float("-inf"))
        ref = torch.logsumexp(sc, dim=-1).permute(0, 2, 1).numpy()
        np.testing.assert_allclose(ours, ref, rtol=1e-13, atol=1e-13)


def test_lse_closed_forms():
    rng = np.random.default_rng(31)
    # one key: lse = scale * q.k
    q, k = _rand(rng, 1, 1, 2, 3), _rand(rng, 1, 1, 2, 3)
    np.testing.assert_allclose(oracle.lse(q, k, 0.7)[0, 0], 0.7 * (q[0, 0] * k[0, 0]).sum(-1), rtol=1e-14)
    # zero queries: lse = log(number of visible keys)
    S = 9
    q0 = np.zeros((1, S, 2, 4))
    k = _rand(rng, 1, S, 1, 4)
    np.testing.assert_allclose(oracle.lse(q0, k, 1.0)[0, :, 0], np.full(S, math.log(S)), rtol=1e-15)
    np.testing.assert_allclose(oracle.lse(q0, k, 1.0, causal=True)[0, :, 0], np.log(np.arange(1, S + 1)), rtol=1e-15)


def test_lse_key_shift_adds_q_dot_u():
    rng = np.random.default_rng(32)
    q, k = np.abs(_rand(rng, 1, 6, 2, 3)) + 1.0, _rand(rng, 1, 6, 2, 3)
    u = np.full(3, 250.0)
    base = oracle.lse(q, k, 0.5)
    shifted = oracle.lse(q, k + u, 0.5)
    np.testing.assert_allclose(shifted - base, 0.5 * (q @ u), rtol=1e-12)


def test_lse_consistent_with_forward():
    """exp(s_j - lse) are the weights: sum_j exp(s_j - lse) v_j reproduces the output."""
    rng = np.random.default_rng(33)
    B, S, H, d = 1, 7, 2, 3
    q, k, v = _rand(rng, B, S, H, d), _rand(rng, B, S, H, d), _rand(rng, B, S, H, d)
    out = oracle.attention(q, k, v, 0.6, causal=True)
    L = oracle.lse(q, k, 0.6, causal=True)
    for h in range(H):
        s = 0.6 * q[0, :, h] @ k[0, :, h].T
        w = np.tril(np.exp(s - L[0, :, h, None]))
        np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-13)
        np.testing.assert_allclose(w @ v[0, :, h], out[0, :, h], rtol=1e-12, atol=1e-13)


# ---- gradients ---------------------------------------------------------------

def _loss(q, k, v, dout, scale, causal):
    return float((oracle.attention(q, k, v, scale, causal=causal) * dout).sum())


@pytest.mark.parametrize("causal", [False, True])
def test_grad_matches_central_differences_of_the_forward(causal):
    """dL/dx for L = sum(out * dout), by central differences of the (pinned)
    forward oracle, element by element."""
    rng = np.random.default_rng(40)
    B, S, H_q, H_kv, d = 1, 5, 4, 2, 3
    q, k, v = _rand(rng, B, S, H_q, d), _rand(rng, B, S, H_kv, d), _rand(rng, B, S, H_kv, d)
    dout = _rand(rng, B, S, H_q, d)
    scale = 0.7
    dq, dk, dv = oracle.attention_grad(q, k, v, dout, scale, causal=causal)
    eps = 1e-5
    for arr, grad in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + eps
            lp = _loss(q, k, v, dout, scale, causal)
            arr[idx] = old - eps
            lm = _loss(q, k, v, dout, scale, causal)
            arr[idx] = old
            num[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-8)


@pytest.mark.parametrize("causal", [False, True])
def test_grad_matches_torch_autograd_fp64(causal):
    rng = np.random.default_rng(41)
    B, S, H_q, H_kv, d = 2, 11, 6, 3, 8
    q, k, v = _rand(rng, B, S, H_q, d), _rand(rng, B, S, H_kv, d), _rand(rng, B, S, H_kv, d)
    dout = _rand(rng, B, S, H_q, d)
    dq, dk, dv = oracle.attention_grad(q, k, v, dout, 0.35, causal=causal)
    R = H_q // H_kv
    tq = torch.from_numpy(q).requires_grad_()
    tk = torch.from_numpy(k).requires_grad_()
    tv = torch.from_numpy(v).requires_grad_()
    o = torch.nn.functional.scaled_dot_product_attention(
        tq.permute(0, 2, 1, 3), tk.permute(0, 2, 1, 3).repeat_interleave(R, dim=1),
        tv.permute(0, 2, 1, 3).repeat_interleave(R, dim=1), is_causal=causal, scale=0.35)
    o.permute(0, 2, 1, 3).backward(torch.from_numpy(dout))
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_grad_sum_invariants():
    """Softmax rows sum to one, so the key gradients of a group sum to zero and
    the value gradients sum to the group's summed upstream gradient."""
    rng = np.random.default_rng(42)
    B, S, H_q, H_kv, d = 2, 9, 4, 2, 5
    q, k, v = _rand(rng, B, S, H_q, d), _rand(rng, B, S, H_kv, d), _rand(rng, B, S, H_kv, d)
    dout = _rand(rng, B, S, H_q, d)
    for causal in (False, True):
        dq, dk, dv = oracle.attention_grad(q, k, v, dout, 0.5, causal=causal)
        np.testing.assert_allclose(dk.sum(axis=1), 0.0, atol=1e-12)
        group_dout = dout.reshape(B, S, H_kv, H_q // H_kv, d).sum(axis=3).sum(axis=1)
        np.testing.assert_allclose(dv.sum(axis=1), group_dout, rtol=1e-12, atol=1e-12)


def test_grad_zero_queries_closed_form():
    """q = 0: uniform weights; dq_i = scale * sum_j p_j (dp_j - D_i) k_j with p = 1/n."""
    rng = np.random.default_rng(43)
    B, S, H, d = 1, 6, 1, 3
    q = np.zeros((B, S, H, d))
    k, v, dout = _rand(rng, B, S, H, d), _rand(rng, B, S, H, d), _rand(rng, B, S, H, d)
    dq, dk, dv = oracle.attention_grad(q, k, v, dout, 0.9)
    dp = dout[0, :, 0] @ v[0, :, 0].T                     # [i, j]
    D = dp.mean(axis=1, keepdims=True)
    expect = 0.9 * ((dp - D) / S) @ k[0, :, 0]
    np.testing.assert_allclose(dq[0, :, 0], expect, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dk, 0.0, atol=1e-15)       # ds_ij * q_i with q = 0
    # p = 1/S for every pair, so every dv_j is the mean of the upstream rows
    np.testing.assert_allclose(dv[0, :, 0], np.tile(dout[0, :, 0].mean(axis=0), (S, 1)), rtol=1e-12)


def test_grad_dq_rows_equal_full_gradient_rows():
    rng = np.random.default_rng(44)
    B, S, H_q, H_kv, d = 2, 12, 4, 2, 5
    q, k, v = _rand(rng, B, S, H_q, d), _rand(rng, B, S, H_kv, d), _rand(rng, B, S, H_kv, d)
    dout = _rand(rng, B, S, H_q, d)
    rows = np.array([11, 0, 5])
    for causal in (False, True):
        dq, _, _ = oracle.attention_grad(q, k, v, dout, 0.45, causal=causal)
        sub = oracle.attention_grad_dq_rows(q, k, v, dout, 0.45, rows, causal=causal)
        np.testing.assert_allclose(sub, dq[:, rows], rtol=1e-14, atol=1e-15)


# ---------------------------------------------------------------------------
# decode: one query token against a key/value cache of per-sequence length


def _decode_case(seed, B, S_max, H_q, H_kv, d):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, H_q, d)), rng.standard_normal((B, S_max, H_kv, d)),
            rng.standard_normal((B, S_max, H_kv, d)))


def test_decode_equals_causal_forward_row():
    """The token at position len-1 of a causal forward sees exactly the cache
    prefix 0..len-1: decode must equal that row of the (separately pinned)
    forward oracle, output and log-normaliser."""
    B, S_max, H_q, H_kv, d = 3, 37, 8, 2, 16
    q, k, v = _decode_case(11, B, S_max, H_q, H_kv, d)
    lens = np.array([37, 1, 20])
    out, lse = oracle.decode(q, k, v, 0.3, seqlens=lens)
    rng = np.random.default_rng(12)
    for b, n in enumerate(lens):
        qf = rng.standard_normal((1, n, H_q, d))
        qf[0, n - 1] = q[b]
        kk, vv = np.ascontiguousarray(k[b:b + 1, :n]), np.ascontiguousarray(v[b:b + 1, :n])
        row = oracle.attention(qf, kk, vv, 0.3, causal=True, rows=[n - 1])
        np.testing.assert_allclose(out[b], row[0, 0], rtol=1e-12, atol=1e-13)
        lrow = oracle.lse(qf, kk, 0.3, causal=True, rows=[n - 1])
        np.testing.assert_allclose(lse[b], lrow[0, 0], rtol=1e-12, atol=1e-13)


def test_decode_matches_torch_sdpa_with_length_mask():
    B, S_max, H_q, H_kv, d = 4, 29, 6, 3, 8
    q, k, v = _decode_case(13, B, S_max, H_q, H_kv, d)
    lens = np.array([29, 5, 17, 2])
    out, lse = oracle.decode(q, k, v, 0.41, seqlens=lens)
    R = H_q // H_kv
    tq = torch.from_numpy(q)[:, :, None, :]                                     # [B, H_q, 1, d]
    tk = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(R, dim=1)   # [B, H_q, S, d]
    tv = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(R, dim=1)
    mask = (torch.arange(S_max)[None, :] < torch.from_numpy(lens)[:, None])[:, None, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(tq.contiguous(), tk.contiguous(), tv.contiguous(),
                                                           attn_mask=mask, scale=0.41)[:, :, 0, :]
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-13)
    scores = 0.41 * (tq @ tk.transpose(-1, -2))[:, :, 0, :]
    scores = scores.masked_fill(~mask[:, :, 0, :], float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(scores, dim=-1).numpy(), rtol=1e-12, atol=1e-13)


def test_decode_closed_forms():
    B, S_max, H_q, H_kv, d = 3, 16, 4, 2, 8
    _, k, v = _decode_case(14, B, S_max, H_q, H_kv, d)
    lens = np.array([16, 1, 0])
    out, lse = oracle.decode(np.zeros((B, H_q, d)), k, v, 0.5, seqlens=lens)
    for h in range(H_q):
        g = h // (H_q // H_kv)
        # constant scores: the mean of the valid values, lse = log(len)
        np.testing.assert_allclose(out[0, h], v[0, :16, g].mean(axis=0), rtol=1e-13, atol=1e-14)
        assert abs(lse[0, h] - math.log(16)) < 1e-13
        # one valid key: its value, lse = its score (0 here)
        np.testing.assert_array_equal(out[1, h], v[1, 0, g])
        assert lse[1, h] == 0.0
        # empty cache: the empty sum
        np.testing.assert_array_equal(out[2, h], np.zeros(d))
        assert lse[2, h] == -math.inf


def test_decode_length_above_cache_is_clamped_and_default_is_full():
    q, k, v = _decode_case(15, 2, 12, 4, 4, 8)
    a = oracle.decode(q, k, v, 0.2, seqlens=[12, 12])
    b = oracle.decode(q, k, v, 0.2, seqlens=[40, 1 << 40])
    c = oracle.decode(q, k, v, 0.2)
    for x, y in ((a, b), (a, c)):
        np.testing.assert_array_equal(x[0], y[0])
        np.testing.assert_array_equal(x[1], y[1])


def test_decode_grouped_equals_mha_on_repeated_cache():
    q, k, v = _decode_case(16, 2, 21, 8, 2, 8)
    lens = [21, 9]
    a = oracle.decode(q, k, v, 0.3, seqlens=lens)
    b = oracle.decode(q, np.repeat(k, 4, axis=2), np.repeat(v, 4, axis=2), 0.3, seqlens=lens)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_decode_bf16_inputs_decode_exactly():
    seed = 17
    q = inputs.normal(seed, 0, (2, 4, 32), "bf16", 0.5)
    k = inputs.normal(seed, 1, (2, 50, 2, 32), "bf16", 0.5)
    v = inputs.normal(seed, 2, (2, 50, 2, 32), "bf16", 0.5)
    f = lambda a: inputs.bf16_bits_to_f32(a).astype(np.float64)
    a = oracle.decode(q, k, v, 0.17, seqlens=[50, 31])
    b = oracle.decode(f(q), f(k), f(v), 0.17, seqlens=[50, 31])
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


# ---------------------------------------------------------------------------
# full layer: projections around the attention


def _layer_per_head_fp64(x, w_qkv, w_o, H_q, H_kv, d, scale, causal):
    """The layer written out head by head in numpy fp64, independently of the
    oracle: query head h projects x with its own d rows of the q block, reads
    the K/V projection of group g = h // (H_q / H_kv), weighs the visible
    positions by exp(scale * score) normalised to sum 1, and the concatenated
    head outputs go through the output projection."""
    x = np.asarray(x, dtype=np.float64)
    B, T, _ = x.shape
    R = H_q // H_kv
    wq = w_qkv[:H_q * d]
    wk = w_qkv[H_q * d:(H_q + H_kv) * d]
    wv = w_qkv[(H_q + H_kv) * d:]
    out = np.zeros((B, T, w_o.shape[0]))
    for b in range(B):
        for t in range(T):
            heads = []
            for h in range(H_q):
                g = h // R
                qh = wq[h * d:(h + 1) * d] @ x[b, t]
                n = t + 1 if causal else T
                keys = x[b, :n] @ wk[g * d:(g + 1) * d].T          # [n, d]
                vals = x[b, :n] @ wv[g * d:(g + 1) * d].T
                a = np.exp(scale * (keys @ qh))
                heads.append((a / a.sum()) @ vals)
            out[b, t] = w_o @ np.concatenate(heads)
    return out


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("H_q,H_kv", [(4, 4), (8, 2), (2, 2), (4, 1)])
def test_layer_matches_per_head_fp64(H_q, H_kv, causal):
    rng = np.random.default_rng(300 + H_q * 10 + H_kv)
    B, T, dm, d = 2, 19, 24, 8
    x = rng.standard_normal((B, T, dm))
    w_qkv = rng.standard_normal(((H_q + 2 * H_kv) * d, dm)) / math.sqrt(dm)
    w_o = rng.standard_normal((dm, H_q * d)) / math.sqrt(H_q * d)
    ours = oracle.layer(x, w_qkv, w_o, H_q, H_kv, d, 0.33, causal=causal)
    ref = _layer_per_head_fp64(x, w_qkv, w_o, H_q, H_kv, d, 0.33, causal)
    np.testing.assert_allclose(ours, ref, rtol=1e-11, atol=1e-12)


def test_layer_with_selection_weights_is_plain_attention():
    """W_qkv selecting slices of x and W_o = I reduce the layer to the
    attention of those slices (pinned separately)."""
    rng = np.random.default_rng(310)
    B, T, H_q, H_kv, d = 1, 23, 4, 2, 6
    nq, nkv = H_q * d, H_kv * d
    dm = nq + 2 * nkv
    x = rng.standard_normal((B, T, dm))
    out = oracle.layer(x, np.eye(dm), np.eye(dm, nq), H_q, H_kv, d, 0.4, causal=True)
    q = x[..., :nq].reshape(B, T, H_q, d)
    k = x[..., nq:nq + nkv].reshape(B, T, H_kv, d)
    v = x[..., nq + nkv:].reshape(B, T, H_kv, d)
    att = oracle.attention(q, k, v, 0.4, causal=True).reshape(B, T, nq)
    np.testing.assert_allclose(out, att @ np.eye(dm, nq).T, rtol=1e-13, atol=1e-14)


def test_layer_rows_equal_full_and_bf16_decodes_exactly():
    from inputs.configs import LAYER_WORKLOADS, make_layer_inputs
    w = LAYER_WORKLOADS["layer_s32k"]
    x, wq, wo = make_layer_inputs(w, "gqa", S=40, d_model=64)
    v = w.variant("gqa")
    full = oracle.layer(x, wq, wo, v.H_q, v.H_kv, w.d, w.scale, causal=True)
    rows = [0, 7, 39]
    sub = oracle.layer(x, wq, wo, v.H_q, v.H_kv, w.d, w.scale, causal=True, rows=rows)
    np.testing.assert_allclose(sub, full[:, rows], rtol=1e-12, atol=1e-13)
    f = lambda a: inputs.bf16_bits_to_f32(a).astype(np.float64)
    np.testing.assert_array_equal(full, oracle.layer(f(x), f(wq), f(wo), v.H_q, v.H_kv, w.d, w.scale, causal=True))
