"""GPU parity of the full attention layer (fused q/k/v projection, attention,
output projection) with the fp64 oracle layer on identical inputs.

Error model: the GPU rounds q, k and v to bf16 after the projection (<= 2^-9
relative each), runs the bf16 attention (~2e-3 relative L2 against exact),
rounds the attention output to bf16 before the output projection and the
result to bf16; the GEMMs accumulate in fp32.  Expected relative L2 about
3-5e-3.  Bounds, relative because the output's scale follows the weights:
relative L2 <= 1e-2, worst per-row relative L2 <= 3e-2, max |err| <= 2e-2 max |ref|.
"""
import math
import sys

import numpy as np
import pytest

import oracle
from inputs.configs import LAYER_WORKLOADS, make_layer_inputs

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
import reduced_query_head_amd as sqa  # noqa: E402
from tests import gpu_util  # noqa: E402

BOUNDS = dict(rel_l2=1e-2, row_rel_l2=3e-2, max_rel=2e-2)


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _check(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    diff = got - ref
    d = ref.shape[-1]
    rn = np.linalg.norm(diff.reshape(-1, d), axis=1)
    rr = np.linalg.norm(ref.reshape(-1, d), axis=1)
    st = dict(rel_l2=float(np.linalg.norm(diff) / np.linalg.norm(ref)),
              row_rel_l2=float((rn / np.maximum(rr, 1e-300)).max()),
              max_rel=float(np.abs(diff).max() / np.abs(ref).max()))
    assert np.isfinite(got).all(), f"{what}: non-finite"
    bad = [k for k, lim in BOUNDS.items() if not st[k] <= lim]
    assert not bad, f"{what}: {bad} {st}"
    return st


def _run(x, wq, wo, H_q, H_kv, scale, causal):
    dx, dwq, dwo = gpu_util.to_device(x), gpu_util.to_device(wq), gpu_util.to_device(wo)
    out = sqa.layer_fwd(dx, dwq, dwo, H_q, H_kv, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return out


SMALL = [
    # B, S, d_model, H_q, H_kv, d, causal
    (1, 64, 256, 4, 4, 64, False),
    (2, 130, 512, 8, 2, 64, True),
    (1, 300, 1024, 8, 8, 128, False),
    (1, 257, 768, 4, 1, 128, True),
    (2, 100, 128, 2, 2, 32, False),
    (1, 1100, 2048, 16, 4, 128, True),
]


@pytest.mark.parametrize("B,S,d_model,H_q,H_kv,d,causal", SMALL)
def test_layer_small_shapes(B, S, d_model, H_q, H_kv, d, causal):
    _say(f"layer B={B} S={S} d_model={d_model} H={H_q}/{H_kv} d={d} causal={causal}")
    w = LAYER_WORKLOADS["layer_s32k"]
    from inputs.configs import LayerWorkload, Variant
    lw = LayerWorkload(w.number, w.name, B=B, S=S, d_model=d_model, d=d, causal=causal,
                       variants=(Variant("t", H_q, H_kv),))
    x, wq, wo = make_layer_inputs(lw, "t")
    scale = 1 / math.sqrt(d)
    out = _run(x, wq, wo, H_q, H_kv, scale, causal)
    ref = oracle.layer(x, wq, wo, H_q, H_kv, d, float(np.float32(scale)), causal=causal)
    st = _check(gpu_util.to_host_f64(out), ref, f"layer {B}x{S} {H_q}/{H_kv} d={d}")
    _say(f"  {st}")


def test_layer_deterministic_and_negative_scale():
    w = LAYER_WORKLOADS["layer_s32k"]
    x, wq, wo = make_layer_inputs(w, "gqa", S=700, d_model=512)
    a = _run(x, wq, wo, 16, 4, -0.1, True)
    b = _run(x, wq, wo, 16, 4, -0.1, True)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    ref = oracle.layer(x, wq, wo, 16, 4, w.d, float(np.float32(-0.1)), causal=True)
    _check(gpu_util.to_host_f64(a), ref, "layer scale=-0.1")


@pytest.mark.parametrize("variant", ["sqa", "mha", "xsqa", "gqa"])
def test_layer_full_size_sampled_rows(variant):
    w = LAYER_WORKLOADS["layer_s32k"]
    v = w.variant(variant)
    _say(f"layer workload {w.name}/{variant}")
    x, wq, wo = make_layer_inputs(w, variant)
    out = _run(x, wq, wo, v.H_q, v.H_kv, w.scale, w.causal)
    rng = np.random.default_rng(w.seed(variant))
    rows = np.unique(np.concatenate([[0, 1, w.S - 1], rng.integers(0, w.S, 29)]))
    got = gpu_util.to_host_f64(out[:, torch.from_numpy(rows).to(out.device)])
    ref = oracle.layer(x, wq, wo, v.H_q, v.H_kv, w.d, float(np.float32(w.scale)), causal=w.causal, rows=rows)
    st = _check(got, ref, f"{w.name}/{variant} rows")
    _say(f"  {st}")
