"""The Python binding rejects caller-supplied buffers the C ABI cannot check.

The C entry points receive bare device addresses, so a host tensor, a buffer
of the wrong shape or dtype, or a short workspace given for an output would
be written through a host address or past its end.  The binding checks every
supplied output, log-normaliser and workspace tensor (device, shape, dtype,
contiguity, size) and raises ValueError before any kernel is enqueued; each
case below also checks that the output it was given was not written.
"""
import pytest

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
import reduced_query_head_amd as sqa  # noqa: E402

B, S, H_q, H_kv, d = 1, 64, 4, 2, 32


def _inputs():
    g = torch.Generator(device="cuda").manual_seed(5)
    q = torch.randn(B, S, H_q, d, device="cuda", generator=g).to(torch.bfloat16)
    k = torch.randn(B, S, H_kv, d, device="cuda", generator=g).to(torch.bfloat16)
    v = torch.randn(B, S, H_kv, d, device="cuda", generator=g).to(torch.bfloat16)
    return q, k, v


def _sentinel(shape, dtype, device="cuda"):
    return torch.full(shape, 7.0, dtype=dtype, device=device)


def test_fwd_rejects_bad_out_and_lse():
    q, k, v = _inputs()
    bad_outs = [_sentinel((B, S, H_q, d), torch.bfloat16, "cpu"),        # host memory
                _sentinel((B, S - 1, H_q, d), torch.bfloat16),            # short
                _sentinel((B, S, H_q, d), torch.float32),                 # wrong dtype
                _sentinel((B, S, d, H_q), torch.bfloat16).transpose(2, 3)]  # not contiguous
    for out in bad_outs:
        with pytest.raises(ValueError):
            sqa.attn_fwd(q, k, v, out=out)
    good = _sentinel((B, S, H_q, d), torch.bfloat16)
    bad_lses = [_sentinel((B, S, H_q), torch.float32, "cpu"), _sentinel((B, S, H_q - 1), torch.float32),
                _sentinel((B, S, H_q), torch.bfloat16)]
    for lse in bad_lses:
        with pytest.raises(ValueError):
            sqa.attn_fwd(q, k, v, out=good, lse=lse)
    torch.cuda.synchronize()
    assert (good == 7.0).all(), "a rejected call must not write out"
    with pytest.raises(ValueError):
        sqa.attn_fwd(q, k.cpu(), v)                                        # input on the host


def test_bwd_rejects_bad_outputs_and_workspace():
    q, k, v = _inputs()
    out, lse = sqa.attn_fwd(q, k, v, return_lse=True)
    dout = torch.randn_like(q)
    ws_need = sqa.attn_bwd_workspace_size(B, S, H_q)
    cases = [
        dict(lse=lse.cpu()),                                               # host lse
        dict(dq=_sentinel((B, S - 1, H_q, d), torch.bfloat16)),            # short dq
        dict(dk=_sentinel((B, S, H_kv, d), torch.float32)),                # wrong-dtype dk
        dict(dv=_sentinel((B, S, H_kv, d), torch.bfloat16, "cpu")),        # host dv
        dict(workspace=torch.empty(ws_need, dtype=torch.uint8)),           # host workspace
        dict(workspace=torch.empty(ws_need - 1, dtype=torch.uint8, device="cuda")),  # short workspace
    ]
    dq_keep = _sentinel((B, S, H_q, d), torch.bfloat16)
    for case in cases:
        kw = dict(lse=lse, dq=dq_keep)
        kw.update(case)
        lse_arg = kw.pop("lse")
        with pytest.raises(ValueError):
            sqa.attn_bwd(q, k, v, out, dout, lse_arg, **kw)
    torch.cuda.synchronize()
    assert (dq_keep == 7.0).all(), "a rejected call must not write dq"
    # a workspace of exactly the needed size in a wider dtype is accepted
    ws = torch.empty((ws_need + 3) // 4, dtype=torch.float32, device="cuda")
    dq, dk, dv = sqa.attn_bwd(q, k, v, out, dout, lse, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(dq.float()).all()


def test_decode_rejects_bad_buffers():
    q, k, v = _inputs()
    qd = q[:, 0].contiguous()                                              # [B, H_q, d]
    lens = torch.full((B,), S, dtype=torch.int32, device="cuda")
    ws_need = sqa.attn_decode_workspace_size(B, S, H_q, H_kv, d)
    out_keep = _sentinel((B, H_q, d), torch.bfloat16)
    cases = [
        dict(lse=_sentinel((B, H_q), torch.float32, "cpu")),
        dict(lse=_sentinel((B, H_q + 1), torch.float32)),
        dict(seqlens=lens.cpu()),
        dict(seqlens=lens.to(torch.int64)),
        dict(workspace=torch.empty(ws_need, dtype=torch.uint8)),
        dict(workspace=torch.empty(max(ws_need - 16, 0), dtype=torch.uint8, device="cuda")),
    ]
    for case in cases:
        kw = dict(seqlens=lens, out=out_keep)
        kw.update(case)
        with pytest.raises(ValueError):
            sqa.attn_decode(qd, k, v, **kw)
    with pytest.raises(ValueError):
        sqa.attn_decode(qd, k, v, seqlens=lens, out=_sentinel((B, H_q, d), torch.bfloat16, "cpu"))
    torch.cuda.synchronize()
    assert (out_keep == 7.0).all(), "a rejected call must not write out"


def test_layer_rejects_bad_buffers():
    dm = 64
    g = torch.Generator(device="cuda").manual_seed(6)
    x = torch.randn(B, S, dm, device="cuda", generator=g).to(torch.bfloat16)
    w_qkv = (0.1 * torch.randn((H_q + 2 * H_kv) * d, dm, device="cuda", generator=g)).to(torch.bfloat16)
    w_o = (0.1 * torch.randn(dm, H_q * d, device="cuda", generator=g)).to(torch.bfloat16)
    ws_need = sqa.layer_workspace_size(B, S, H_q, H_kv, d)
    out_keep = _sentinel((B, S, dm), torch.bfloat16)
    for ws in (torch.empty(ws_need, dtype=torch.uint8), torch.empty(ws_need - 1, dtype=torch.uint8, device="cuda")):
        with pytest.raises(ValueError):
            sqa.layer_fwd(x, w_qkv, w_o, H_q, H_kv, out=out_keep, workspace=ws)
    with pytest.raises(ValueError):
        sqa.layer_fwd(x, w_qkv, w_o, H_q, H_kv, out=_sentinel((B, S, dm), torch.float32))
    with pytest.raises(ValueError):
        sqa.layer_fwd(x, w_qkv.cpu(), w_o, H_q, H_kv)
    torch.cuda.synchronize()
    assert (out_keep == 7.0).all(), "a rejected call must not write out"
