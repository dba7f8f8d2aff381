"""Every entry point can be captured in a HIP graph (torch.cuda.graph) and
replayed: the library allocates nothing, clears nothing and synchronises
nothing inside a call, and enqueues all its work on the caller's stream.
Each graph is replayed several times, with fresh inputs copied into the
captured buffers, eager work and synchronisations between replays, and every
replay must equal an eager call on the same inputs bit for bit."""
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

REPLAYS = 3


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _same(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a, b)


def _capture(fn):
    """Warm fn up on a side stream (first calls may create library handles),
    then capture one call; returns the graph and the captured outputs."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = fn()
    torch.cuda.synchronize()
    return g, outs


def _replay_and_check(name, g, outs, fn, static_inputs, make_inputs):
    for rep in range(REPLAYS):
        for dst, src in zip(static_inputs, make_inputs(rep)):
            dst.copy_(src)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = fn()                       # eager call on the same inputs
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, ref)):
            assert _same(a, b), f"{name}: replay {rep}, output {i} differs from the eager call"
        _say(f"  {name} replay {rep} ok")


def _bf16(seed, stream, shape, mul):
    return gpu_util.to_device(inputs.normal(seed, stream, shape, "bf16", mul))


def test_graph_forward_and_backward():
    B, S, H_q, H_kv, d = 1, 1500, 8, 2, 128
    _say(f"graph forward+backward B={B} S={S} H={H_q}/{H_kv} d={d}")
    q = _bf16(70, 0, (B, S, H_q, d), 0.5)
    k = _bf16(70, 1, (B, S, H_kv, d), 0.5)
    v = _bf16(70, 2, (B, S, H_kv, d), 0.5)
    g_out = _bf16(70, 3, (B, S, H_q, d), 1.0)

    def fwd_bwd():
        o, lse = sqa.attn_fwd(q, k, v, scale=0.09, causal=True, return_lse=True)
        gq, gk, gv = sqa.attn_bwd(q, k, v, o, g_out, lse, scale=0.09, causal=True)
        return o, lse, gq, gk, gv

    g, outs = _capture(fwd_bwd)

    def fresh(rep):
        s = 71 + rep
        return [_bf16(s, 0, tuple(q.shape), 0.5), _bf16(s, 1, tuple(k.shape), 0.5), _bf16(s, 2, tuple(v.shape), 0.5),
                _bf16(s, 3, tuple(g_out.shape), 1.0)]

    _replay_and_check("forward+backward", g, outs, fwd_bwd, [q, k, v, g_out], fresh)


def test_graph_decode():
    B, S_max, H_q, H_kv, d = 3, 5000, 16, 4, 128
    _say(f"graph decode B={B} S_max={S_max} H={H_q}/{H_kv} d={d}")
    q = _bf16(80, 0, (B, H_q, d), 0.5)
    kc = _bf16(80, 1, (B, S_max, H_kv, d), 0.5)
    vc = _bf16(80, 2, (B, S_max, H_kv, d), 0.5)
    lens = torch.tensor([5000, 1234, 0], dtype=torch.int32, device="cuda")

    def dec():
        return sqa.attn_decode(q, kc, vc, seqlens=lens, scale=0.1, return_lse=True)

    g, outs = _capture(dec)
    rng = np.random.default_rng(81)

    def fresh(rep):
        s = 82 + rep
        new_lens = torch.tensor([int(x) for x in rng.integers(0, S_max + 1, B)], dtype=torch.int32, device="cuda")
        return [_bf16(s, 0, tuple(q.shape), 0.5), _bf16(s, 1, tuple(kc.shape), 0.5),
                _bf16(s, 2, tuple(vc.shape), 0.5), new_lens]

    _replay_and_check("decode", g, outs, dec, [q, kc, vc, lens], fresh)


def test_graph_layer():
    w = LAYER_WORKLOADS["layer_s32k"]
    lw = LayerWorkload(w.number, w.name, B=1, S=700, d_model=512, d=64, causal=True,
                       variants=(Variant("t", 8, 2),))
    _say("graph layer B=1 S=700 d_model=512 H=8/2 d=64 causal")
    x, wq, wo = (gpu_util.to_device(a) for a in make_layer_inputs(lw, "t"))

    def layer():
        return (sqa.layer_fwd(x, wq, wo, 8, 2, scale=1 / math.sqrt(64), causal=True),)

    g, outs = _capture(layer)

    def fresh(rep):
        return [_bf16(90 + rep, 0, tuple(x.shape), 1.0)]

    _replay_and_check("layer", g, outs, layer, [x], fresh)
