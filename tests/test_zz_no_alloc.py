"""The allocation-free decode entry point (sqa_attn_decode_noalloc) against
the decode entry point that takes a caller workspace (sqa_attn_decode), both
called through the C ABI on the same device inputs.

Calls come in a row on one GPU, so the second reads a scratch array that
still holds the first call's partial results; the second call is smaller
(fewer sequences, heads and positions).  Where the split plan of the
allocation-free call equals the workspace call's (its partial results fit
the 16 MiB scratch) the outputs must be bitwise equal; where the plan had to
take longer splits to fit, the two differ in rounding only and are compared
with the forward's parity bounds, and both are checked against the fp64
oracle.
"""
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


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _case(seed, B, S_max, H_q, H_kv, d, lens, dtype="bf16"):
    q = inputs.normal(seed, 0, (B, H_q, d), dtype, 0.5)
    k = inputs.normal(seed, 1, (B, S_max, H_kv, d), dtype, 0.5)
    v = inputs.normal(seed, 2, (B, S_max, H_kv, d), dtype, 0.5)
    return q, k, v, np.asarray(lens, dtype=np.int32)


def _both(q, k, v, lens, scale, stream):
    """(workspace output, workspace lse, no-alloc output, no-alloc lse) on the
    same device inputs, the no-alloc call enqueued right after the other."""
    dq, dk, dv = (gpu_util.to_device(a) for a in (q, k, v))
    dl = torch.from_numpy(lens).cuda()
    B, H_q, d = dq.shape
    S_max, H_kv = dk.shape[1], dk.shape[2]
    dt = sqa.SQA_BF16 if dq.dtype == torch.bfloat16 else sqa.SQA_FP32
    handle = stream.cuda_stream if stream is not None else 0
    out_ws, out_na = torch.empty_like(dq), torch.empty_like(dq)
    lse_ws = torch.empty((B, H_q), dtype=torch.float32, device="cuda")
    lse_na = torch.empty_like(lse_ws)
    need = sqa.attn_decode_workspace_size(B, S_max, H_q, H_kv, d)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()   # inputs and outputs exist before a side stream uses them
    st = sqa.attn_decode_raw(dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), dl.data_ptr(), out_ws.data_ptr(),
                             lse_ws.data_ptr(), ws.data_ptr(), need, B, S_max, H_q, H_kv, d, dt, scale, handle)
    assert st == sqa.SQA_OK, sqa.status_string(st)
    st = sqa.attn_decode_noalloc_raw(dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), dl.data_ptr(),
                                     out_na.data_ptr(), lse_na.data_ptr(), B, S_max, H_q, H_kv, d, dt, scale,
                                     handle)
    assert st == sqa.SQA_OK, sqa.status_string(st)
    torch.cuda.synchronize()
    return out_ws, lse_ws, out_na, lse_na


def _bits(t):
    return gpu_util.to_host_bits(t)


def test_noalloc_equals_workspace_decode_two_calls():
    """Two calls in a row, the second smaller; both plans fit the scratch,
    so the outputs and log-normalisers match the workspace call bitwise."""
    cases = [(8101, 4, 4096, 32, 8, 128, [4096, 3000, 17, 2222]),
             (8102, 2, 1000, 8, 2, 64, [1000, 431])]
    for i, (seed, B, S_max, H_q, H_kv, d, lens) in enumerate(cases):
        _say(f"no-alloc call {i}: B={B} S_max={S_max} H={H_q}/{H_kv} d={d}")
        q, k, v, ln = _case(seed, B, S_max, H_q, H_kv, d, lens)
        stream = None if i == 0 else torch.cuda.Stream()
        ow, lw, on, lnn = _both(q, k, v, ln, 1 / math.sqrt(d), stream)
        assert np.array_equal(_bits(ow), _bits(on)), "outputs differ"
        assert np.array_equal(lw.cpu().numpy().view(np.uint32), lnn.cpu().numpy().view(np.uint32)), "lse differ"
        ref, _ = oracle.decode(q, k, v, float(np.float32(1 / math.sqrt(d))), seqlens=ln)
        _say(f"  vs oracle {parity.check(gpu_util.to_host_f64(on), ref, 'bf16', 'no-alloc decode')}")


def test_noalloc_longer_splits_then_smaller_call():
    """Eight 32/4 caches of 128K positions: the workspace call's plan needs
    more than the 16 MiB scratch, so the allocation-free call takes longer
    splits (same sum, other rounding).  Then a smaller call reuses the
    scratch."""
    B, S_max, H_q, H_kv, d = 8, 131072, 32, 4, 128
    need = sqa.attn_decode_workspace_size(B, S_max, H_q, H_kv, d)
    assert need > (16 << 20), need
    lens = [131072, 70000, 1, 0, 513, 4096, 99999, 32]
    _say(f"no-alloc long: B={B} S_max={S_max} H={H_q}/{H_kv} workspace plan {need} bytes")
    q, k, v, ln = _case(8103, B, S_max, H_q, H_kv, d, lens)
    ow, lw, on, lnn = _both(q, k, v, ln, 1 / math.sqrt(d), None)
    nz = ln > 0
    st = parity.check(gpu_util.to_host_f64(on)[nz], gpu_util.to_host_f64(ow)[nz], "bf16", "no-alloc vs workspace")
    _say(f"  vs workspace call {st}")
    assert np.array_equal(_bits(on)[~nz], _bits(ow)[~nz])
    dl = np.abs(lnn.double().cpu().numpy()[nz] - lw.double().cpu().numpy()[nz])
    assert dl.max() <= 2.5e-3, dl.max()
    ref, ref_lse = oracle.decode(q, k, v, float(np.float32(1 / math.sqrt(d))), seqlens=ln)
    full = ln > 0
    got = gpu_util.to_host_f64(on)
    _say(f"  vs oracle {parity.check(got[full], ref[full], 'bf16', 'no-alloc long vs oracle')}")
    assert (got[~full] == 0).all() and np.isneginf(lnn.cpu().numpy()[~full]).all()
    assert np.abs(lnn.double().cpu().numpy()[full] - ref_lse[full]).max() <= 2.5e-3

    _say("no-alloc after it: B=1 S_max=300 H=4/4 d=32")
    q, k, v, ln = _case(8104, 1, 300, 4, 4, 32, [300])
    ow, lw, on, lnn = _both(q, k, v, ln, 1 / math.sqrt(32), torch.cuda.Stream())
    assert np.array_equal(_bits(ow), _bits(on)), "outputs differ"
    assert np.array_equal(lw.cpu().numpy().view(np.uint32), lnn.cpu().numpy().view(np.uint32)), "lse differ"


def test_noalloc_fp32_and_empty_caches():
    q, k, v, ln = _case(8105, 3, 200, 8, 4, 32, [200, 0, 5], dtype="f32")
    ow, lw, on, lnn = _both(q, k, v, ln, 0.2, None)
    assert np.array_equal(ow.cpu().numpy(), on.cpu().numpy())
    q, k, v, ln = _case(8106, 2, 256, 8, 2, 128, [0, 256])
    ow, lw, on, lnn = _both(q, k, v, ln, 0.1, None)
    assert np.array_equal(_bits(ow), _bits(on))
    assert np.isneginf(lnn[0].cpu().numpy()).all()


def test_noalloc_under_graph_capture():
    """The callers this entry point is for include code under HIP graph
    capture: the call is captured once (after eager warm-up calls), the graph
    is replayed with fresh cache contents copied into the captured buffers,
    and every replay equals an eager call of the same entry point bitwise."""
    B, S_max, H_q, H_kv, d = 3, 2000, 16, 4, 128
    lens = torch.tensor([2000, 1234, 7], dtype=torch.int32, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(8107)

    def fresh():
        return [(0.5 * torch.randn(shape, device="cuda", generator=gen)).to(torch.bfloat16)
                for shape in ((B, H_q, d), (B, S_max, H_kv, d), (B, S_max, H_kv, d))]

    q, k, v = fresh()
    out = torch.empty_like(q)
    lse = torch.empty((B, H_q), dtype=torch.float32, device="cuda")

    def call(o, l):
        st = sqa.attn_decode_noalloc_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), lens.data_ptr(), o.data_ptr(),
                                         l.data_ptr(), B, S_max, H_q, H_kv, d, sqa.SQA_BF16, 1 / math.sqrt(d),
                                         torch.cuda.current_stream().cuda_stream)
        assert st == sqa.SQA_OK, sqa.status_string(st)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            call(out, lse)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out, lse)
    torch.cuda.synchronize()
    ref_out, ref_lse = torch.empty_like(out), torch.empty_like(lse)
    for rep in range(3):
        for dst, src in zip((q, k, v), fresh()):
            dst.copy_(src)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        call(ref_out, ref_lse)           # eager, same inputs
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), f"replay {rep}: out"
        assert torch.equal(lse, ref_lse), f"replay {rep}: lse"
        _say(f"no-alloc graph replay {rep}: equal")
