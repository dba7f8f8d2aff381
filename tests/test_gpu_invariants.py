"""Properties of the GPU kernel that hold exactly or nearly, independent of
the oracle: causal row 0 is V[0], the grouped kernel equals the MHA kernel on
repeated K/V bit for bit, runs are deterministic, and constant scores give
the mean of V."""
import math

import numpy as np
import pytest

import inputs
from tests.parity import check

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
from tests import gpu_util  # noqa: E402


def _inputs(seed, B, S, H_q, H_kv, d):
    return (inputs.normal(seed, 0, (B, S, H_q, d), "bf16", 0.5),
            inputs.normal(seed, 1, (B, S, H_kv, d), "bf16", 0.5),
            inputs.normal(seed, 2, (B, S, H_kv, d), "bf16", 0.5))


@pytest.mark.parametrize("d", [64, 128])
def test_causal_row_zero_is_v0_bitwise(d):
    q, k, v = _inputs(5, 2, 300, 8, 2, d)
    out = gpu_util.to_host_bits(gpu_util.run(q, k, v, 1 / math.sqrt(d), True))
    for h in range(8):
        assert np.array_equal(out[:, 0, h, :], v[:, 0, h // 4, :]), h


@pytest.mark.parametrize("causal", [False, True])
def test_grouped_equals_mha_on_repeated_kv_bitwise(causal):
    q, k, v = _inputs(6, 1, 777, 8, 2, 128)
    grouped = gpu_util.to_host_bits(gpu_util.run(q, k, v, 0.09, causal))
    mha = gpu_util.to_host_bits(gpu_util.run(q, np.repeat(k, 4, axis=2), np.repeat(v, 4, axis=2), 0.09, causal))
    assert np.array_equal(grouped, mha)


def test_deterministic():
    q, k, v = _inputs(7, 1, 4096, 8, 4, 128)
    a = gpu_util.to_host_bits(gpu_util.run(q, k, v, 0.088, True))
    b = gpu_util.to_host_bits(gpu_util.run(q, k, v, 0.088, True))
    assert np.array_equal(a, b)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_queries_give_mean_of_v(causal):
    B, S, H_q, H_kv, d = 1, 1000, 4, 2, 64
    _, k, v = _inputs(8, B, S, H_q, H_kv, d)
    q = np.zeros((B, S, H_q, d), dtype=np.uint16)
    got = gpu_util.to_host_f64(gpu_util.run(q, k, v, 0.125, causal))
    vf = inputs.bf16_bits_to_f32(v).astype(np.float64)
    ref = np.empty((B, S, H_q, d))
    for h in range(H_q):
        g = h // 2
        if causal:
            ref[:, :, h] = np.cumsum(vf[:, :, g], axis=1) / np.arange(1, S + 1)[None, :, None]
        else:
            ref[:, :, h] = vf[:, :, g].mean(axis=1, keepdims=True)
    check(got, ref, "bf16", f"q=0 causal={causal}")
