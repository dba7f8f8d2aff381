"""Every entry point enqueues its work on the stream it is given: results on
a side stream equal those on the default stream bit for bit, and two streams
running the forward concurrently on different inputs each get their own
result (the library keeps no state shared between calls; workspaces are the
caller's)."""
import math
import sys

import numpy as np
import pytest

import inputs
from inputs.configs import LAYER_WORKLOADS, LayerWorkload, Variant, make_layer_inputs

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
import reduced_query_head_amd as sqa  # noqa: E402
from tests import gpu_util  # noqa: E402


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _same(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a, b)


def _all_entry_points(dq, dk, dv, dg, kc, vc, lens, x, wq, wo):
    o, lse = sqa.attn_fwd(dq, dk, dv, scale=0.1, causal=True, return_lse=True)
    g = sqa.attn_bwd(dq, dk, dv, o, dg, lse, scale=0.1, causal=True)
    do, dl = sqa.attn_decode(dq[:, -1].contiguous(), kc, vc, seqlens=lens, scale=0.1, return_lse=True)
    lo = sqa.layer_fwd(x, wq, wo, 8, 2, scale=1 / math.sqrt(64), causal=False)
    return [o, lse, *g, do, dl, lo]


def test_side_stream_matches_default_stream():
    _say("entry points on a side stream")
    B, S, H_q, H_kv, d = 2, 700, 8, 2, 128
    q = inputs.normal(91, 0, (B, S, H_q, d), "bf16", 0.5)
    k = inputs.normal(91, 1, (B, S, H_kv, d), "bf16", 0.5)
    v = inputs.normal(91, 2, (B, S, H_kv, d), "bf16", 0.5)
    g = inputs.normal(91, 3, (B, S, H_q, d), "bf16", 1.0)
    dq, dk, dv, dg = (gpu_util.to_device(a) for a in (q, k, v, g))
    lens = torch.tensor([700, 313], dtype=torch.int32, device="cuda")
    w = LAYER_WORKLOADS["layer_s32k"]
    lw = LayerWorkload(w.number, w.name, B=1, S=300, d_model=512, d=64, causal=False,
                       variants=(Variant("t", 8, 2),))
    x, wq, wo = (gpu_util.to_device(a) for a in make_layer_inputs(lw, "t"))

    ref = _all_entry_points(dq, dk, dv, dg, dk, dv, lens, x, wq, wo)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        got = _all_entry_points(dq, dk, dv, dg, dk, dv, lens, x, wq, wo)
    side.synchronize()
    names = ["out", "lse", "dq", "dk", "dv", "decode out", "decode lse", "layer out"]
    for n, a, b in zip(names, got, ref):
        assert _same(a, b), f"{n}: side-stream result differs from the default stream's"


def test_two_streams_concurrently():
    _say("two streams, different inputs, concurrent forwards")
    B, S, H_q, H_kv, d = 1, 4096, 16, 4, 128
    xs = []
    for seed in (92, 93):
        q = inputs.normal(seed, 0, (B, S, H_q, d), "bf16", 0.5)
        k = inputs.normal(seed, 1, (B, S, H_kv, d), "bf16", 0.5)
        v = inputs.normal(seed, 2, (B, S, H_kv, d), "bf16", 0.5)
        xs.append([gpu_util.to_device(a) for a in (q, k, v)])
    refs = [sqa.attn_fwd(*t, scale=0.088, causal=False) for t in xs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    outs = []
    for rep in range(3):
        for s, t in zip(streams, xs):
            with torch.cuda.stream(s):
                outs.append(sqa.attn_fwd(*t, scale=0.088, causal=False))
    for s in streams:
        s.synchronize()
    for i, o in enumerate(outs):
        assert _same(o, refs[i % 2]), f"launch {i}: concurrent result differs"
