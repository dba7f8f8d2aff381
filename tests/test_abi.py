"""The C-ABI library loads, exports what include/sqa.h declares, and rejects
bad arguments before touching the GPU (these calls return before any HIP
call, so they run without a GPU)."""
import ctypes
import os
import re

import pytest

import reduced_query_head_amd as sqa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# The host sanitizer test reruns this file against a host-only build of the
# same C-ABI source whose kernel launchers are stubs (tests/sanitize); every
# call below then goes to that build.
STUB_LIB = os.environ.get("SQA_TEST_STUB_LIB")
if STUB_LIB:
    sqa.load_library(STUB_LIB)


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "sqa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sqa_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = sqa.load_library()
    names = _declared_functions()
    assert "sqa_attn_fwd" in names and "sqa_status_string" in names
    for name in names:
        assert hasattr(lib, name), f"{name} declared in sqa.h but not exported"


def test_status_strings():
    assert sqa.status_string(0) == "success"
    assert sqa.status_string(1) == "invalid argument"
    assert sqa.status_string(2) == "unsupported configuration"
    assert sqa.status_string(3) == "HIP runtime error"


FAKE = 0x7F0000000000  # 16-byte aligned, never dereferenced (rejected first)


def _call(q=FAKE, k=FAKE + (1 << 30), v=FAKE + (2 << 30), out=FAKE + (3 << 30), B=1, S=128, H_q=8,
          H_kv=2, d=128, dtype=0, scale=0.088, causal=0):
    return sqa.attn_fwd_raw(q, k, v, out, B, S, H_q, H_kv, d, dtype, scale, causal, 0)


@pytest.mark.parametrize("kw", [
    dict(H_q=6, H_kv=4),          # groups must divide heads
    dict(H_q=2, H_kv=4),          # fewer query heads than K/V heads
    dict(H_q=0), dict(H_kv=0), dict(B=-1), dict(S=-5), dict(d=0),
    dict(dtype=7), dict(causal=2),
    dict(scale=float("inf")), dict(scale=float("nan")), dict(scale=3e38),
    dict(q=0), dict(k=0), dict(v=0), dict(out=0),
    dict(q=FAKE + 8),             # misaligned
    dict(out=FAKE + 64),          # out overlaps q
    dict(out=FAKE + (1 << 30) + 1024),   # out overlaps k
])
def test_invalid_arguments(kw):
    assert _call(**kw) == sqa.SQA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("kw", [dict(d=96), dict(d=256), dict(d=16)])
def test_unsupported(kw):
    assert _call(**kw) == sqa.SQA_ERR_UNSUPPORTED


def test_row_too_wide_is_unsupported():
    # tiles are addressed with 32-bit offsets from a 64-bit base: rows of at
    # most 2^22 elements
    assert _call(S=1, H_q=65536, H_kv=65536) == sqa.SQA_ERR_UNSUPPORTED
    assert _call(S=1, H_q=65536, H_kv=1) == sqa.SQA_ERR_UNSUPPORTED
    assert _call_bwd(S=1, H_q=65536, H_kv=65536) == sqa.SQA_ERR_UNSUPPORTED
    assert _call_dec(S_max=1, H_q=65536, H_kv=65536) == sqa.SQA_ERR_UNSUPPORTED
    assert _call_layer(S=1, d_model=8, H_q=16384, H_kv=16384) == sqa.SQA_ERR_UNSUPPORTED


def test_sequence_too_long_is_unsupported():
    far = 1 << 44   # buffers spaced wider than the 2^41-byte tensors
    assert _call(q=far, k=2 * far, v=3 * far, out=4 * far, S=(1 << 30) + 1) == sqa.SQA_ERR_UNSUPPORTED


def test_empty_is_noop():
    assert _call(B=0, q=0, k=0, v=0, out=0) == sqa.SQA_OK
    assert _call(S=0, q=0, k=0, v=0, out=0) == sqa.SQA_OK


def _call_lse(lse, **kw):
    args = dict(q=FAKE, k=FAKE + (1 << 30), v=FAKE + (2 << 30), out=FAKE + (3 << 30), B=1, S=128, H_q=8,
                H_kv=2, d=128, dtype=0, scale=0.088, causal=0)
    args.update(kw)
    a = args
    return sqa.attn_fwd_lse_raw(a["q"], a["k"], a["v"], a["out"], lse, a["B"], a["S"], a["H_q"], a["H_kv"],
                                a["d"], a["dtype"], a["scale"], a["causal"], 0)


@pytest.mark.parametrize("lse", [FAKE + (4 << 30) + 2,        # misaligned
                                 FAKE + (3 << 30) + 4096,     # inside out
                                 FAKE + 64])                  # inside q
def test_lse_invalid(lse):
    assert _call_lse(lse) == sqa.SQA_ERR_INVALID_ARGUMENT


def test_lse_rejects_the_same_errors_as_forward():
    assert _call_lse(FAKE + (4 << 30), H_q=6, H_kv=4) == sqa.SQA_ERR_INVALID_ARGUMENT
    assert _call_lse(FAKE + (4 << 30), d=96) == sqa.SQA_ERR_UNSUPPORTED
    assert _call_lse(0, B=0, q=0, k=0, v=0, out=0) == sqa.SQA_OK


def _call_bwd(**kw):
    G = 1 << 32
    a = dict(q=FAKE, k=FAKE + G, v=FAKE + 2 * G, out=FAKE + 3 * G, dout=FAKE + 4 * G, lse=FAKE + 5 * G,
             dq=FAKE + 6 * G, dk=FAKE + 7 * G, dv=FAKE + 8 * G, ws=FAKE + 9 * G, ws_bytes=1 << 30, B=1, S=128,
             H_q=8, H_kv=2, d=128, dtype=0, scale=0.088, causal=1)
    a.update(kw)
    return sqa.attn_bwd_raw(a["q"], a["k"], a["v"], a["out"], a["dout"], a["lse"], a["dq"], a["dk"], a["dv"], a["ws"],
                            a["ws_bytes"], a["B"], a["S"], a["H_q"], a["H_kv"], a["d"], a["dtype"], a["scale"],
                            a["causal"], 0)


def test_bwd_workspace_size():
    assert sqa.attn_bwd_workspace_size(2, 100, 8) == 2 * 2 * 8 * 128 * 4
    assert sqa.attn_bwd_workspace_size(1, 128, 1) == 2 * 128 * 4
    assert sqa.attn_bwd_workspace_size(-1, 10, 1) == -1
    # sizes whose workspace is not representable in int64
    assert sqa.attn_bwd_workspace_size(1 << 31, 1 << 30, 1 << 20) == -1
    assert sqa.attn_bwd_workspace_size(1, (1 << 63) - 1, 1) == -1


@pytest.mark.parametrize("kw", [
    dict(H_q=6, H_kv=4), dict(dout=0), dict(lse=0), dict(ws=0), dict(dq=FAKE + 8), dict(lse=FAKE + (5 << 32) + 2),
    dict(ws_bytes=2 * 8 * 128 * 4 - 1), dict(dq=FAKE + 64), dict(dk=FAKE + (6 << 32) + 128),
    dict(ws=FAKE + (8 << 32) + 256), dict(causal=3), dict(scale=float("nan")),
])
def test_bwd_invalid(kw):
    assert _call_bwd(**kw) == sqa.SQA_ERR_INVALID_ARGUMENT


def test_bwd_unsupported_and_empty():
    assert _call_bwd(d=80) == sqa.SQA_ERR_UNSUPPORTED
    assert _call_bwd(B=0, q=0, k=0, v=0, out=0, dout=0, lse=0, dq=0, dk=0, dv=0, ws=0, ws_bytes=0) == sqa.SQA_OK


G = 1 << 30


def _call_dec(**kw):
    a = dict(q=FAKE, k=FAKE + G, v=FAKE + 2 * G, seqlens=FAKE + 3 * G, out=FAKE + 4 * G, lse=FAKE + 5 * G,
             ws=FAKE + 6 * G, ws_bytes=None, B=4, S_max=4096, H_q=32, H_kv=8, d=128, dtype=0, scale=0.088)
    a.update(kw)
    if a["ws_bytes"] is None:
        a["ws_bytes"] = max(0, sqa.attn_decode_workspace_size(a["B"], a["S_max"], a["H_q"], a["H_kv"], a["d"]))
    return sqa.attn_decode_raw(a["q"], a["k"], a["v"], a["seqlens"], a["out"], a["lse"], a["ws"], a["ws_bytes"],
                               a["B"], a["S_max"], a["H_q"], a["H_kv"], a["d"], a["dtype"], a["scale"], 0)


def test_decode_workspace_size():
    n = sqa.attn_decode_workspace_size(4, 4096, 32, 8, 128)
    assert n > 0 and n % 16 == 0
    # partials of every query head of every split: at least one (d + 2) fp32 record per head
    assert n >= 4 * 32 * (128 + 2) * 4
    assert sqa.attn_decode_workspace_size(4, 0, 32, 8, 128) > 0
    for bad in [(-1, 10, 4, 2, 64), (1, -1, 4, 2, 64), (1, 10, 0, 1, 64), (1, 10, 6, 4, 64), (1, 10, 4, 2, 0),
                (1, (1 << 30) + 1, 4, 2, 64),
                (1 << 20, 1 << 30, 1 << 20, 1, 32)]:      # a split plan beyond int64
        assert sqa.attn_decode_workspace_size(*bad) == -1


@pytest.mark.parametrize("kw", [
    dict(H_q=6, H_kv=4), dict(H_q=2, H_kv=4), dict(H_q=0), dict(B=-1), dict(S_max=-1), dict(d=0),
    dict(dtype=5), dict(scale=float("nan")), dict(scale=float("-inf")), dict(scale=-3e38),
    dict(q=0), dict(k=0), dict(v=0), dict(out=0), dict(ws=0),
    dict(q=FAKE + 8), dict(out=FAKE + 4 * G + 4), dict(ws=FAKE + 6 * G + 2), dict(lse=FAKE + 5 * G + 2),
    dict(seqlens=FAKE + 3 * G + 1),
    dict(ws_bytes=16),                         # workspace too small
    dict(out=FAKE + 64),                       # out overlaps q
    dict(ws=FAKE + G + 4096),                  # workspace overlaps the k cache
    dict(lse=FAKE + 4 * G + 256),              # lse overlaps out
    dict(out=FAKE + 3 * G),                    # out overlaps seqlens
])
def test_decode_invalid(kw):
    assert _call_dec(**kw) == sqa.SQA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("kw", [dict(d=96), dict(d=16), dict(d=256), dict(dtype=1, d=96),
                                # caches and q fit int64, the split plan over all 2^20 query heads does not
                                dict(B=1 << 20, S_max=1 << 30, H_q=1 << 20, H_kv=1, d=32, ws_bytes=1 << 40,
                                     q=FAKE, k=FAKE + (1 << 58), v=FAKE + (1 << 59), seqlens=0, out=FAKE + (3 << 58),
                                     lse=0, ws=FAKE + (7 << 57))])
def test_decode_unsupported(kw):
    assert _call_dec(**kw) == sqa.SQA_ERR_UNSUPPORTED


def test_decode_empty_and_optional_pointers():
    assert _call_dec(B=0, q=0, k=0, v=0, out=0, ws=0) == sqa.SQA_OK
    # seqlens and lse are optional; they still may not be misaligned (checked above)
    assert _call_dec(B=0, seqlens=0, lse=0) == sqa.SQA_OK


def _call_layer(**kw):
    a = dict(x=FAKE, wqkv=FAKE + G, wo=FAKE + 2 * G, out=FAKE + 3 * G, ws=FAKE + 4 * G, ws_bytes=None, B=1, S=1024,
             d_model=2048, H_q=8, H_kv=8, d=128, scale=0.088, causal=0)
    a.update(kw)
    if a["ws_bytes"] is None:
        a["ws_bytes"] = max(0, sqa.layer_workspace_size(a["B"], a["S"], a["H_q"], a["H_kv"], a["d"]))
    return sqa.layer_fwd_raw(a["x"], a["wqkv"], a["wo"], a["out"], a["ws"], a["ws_bytes"], a["B"], a["S"],
                             a["d_model"], a["H_q"], a["H_kv"], a["d"], a["scale"], a["causal"], 0)


def test_layer_workspace_size():
    n = sqa.layer_workspace_size(1, 1024, 8, 8, 128)
    # the projection output and the attention output at least
    assert n >= 1024 * (8 + 16) * 128 * 2 + 1024 * 8 * 128 * 2
    assert sqa.layer_workspace_size(1, 10, 6, 4, 64) == -1 and sqa.layer_workspace_size(-1, 10, 4, 4, 64) == -1


@pytest.mark.parametrize("kw", [
    dict(H_q=6, H_kv=4), dict(d_model=0), dict(B=-1), dict(causal=3), dict(scale=float("nan")),
    dict(x=0), dict(wqkv=0), dict(wo=0), dict(out=0), dict(ws=0), dict(x=FAKE + 4), dict(ws=FAKE + 4 * G + 8),
    dict(ws_bytes=1024), dict(out=FAKE + 4096), dict(ws=FAKE + G + 256), dict(out=FAKE + 4 * G + 512),
])
def test_layer_invalid(kw):
    assert _call_layer(**kw) == sqa.SQA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("kw", [dict(d=96), dict(d=16), dict(d_model=2044)])
def test_layer_unsupported(kw):
    assert _call_layer(**kw) == sqa.SQA_ERR_UNSUPPORTED


def test_layer_empty():
    assert _call_layer(S=0, x=0, wqkv=0, wo=0, out=0, ws=0) == sqa.SQA_OK


def _call_dec_noalloc(**kw):
    a = dict(q=FAKE, k=FAKE + G, v=FAKE + 2 * G, seqlens=FAKE + 3 * G, out=FAKE + 4 * G, lse=FAKE + 5 * G,
             B=4, S_max=4096, H_q=32, H_kv=8, d=128, dtype=0, scale=0.088)
    a.update(kw)
    return sqa.attn_decode_noalloc_raw(a["q"], a["k"], a["v"], a["seqlens"], a["out"], a["lse"], a["B"],
                                       a["S_max"], a["H_q"], a["H_kv"], a["d"], a["dtype"], a["scale"], 0)


@pytest.mark.parametrize("kw", [
    dict(H_q=6, H_kv=4), dict(H_q=0), dict(B=-1), dict(S_max=-1), dict(dtype=5), dict(scale=float("nan")),
    dict(q=0), dict(out=0), dict(k=0), dict(q=FAKE + 8), dict(lse=FAKE + 5 * G + 2),
    dict(out=FAKE + 64),          # out overlaps q
])
def test_decode_noalloc_invalid_arguments(kw):
    assert _call_dec_noalloc(**kw) == sqa.SQA_ERR_INVALID_ARGUMENT


def test_decode_noalloc_scratch_limit():
    # one split per head needs B * H_q * (d + 2) * 4 bytes of the 16 MiB
    # scratch: 32264 bf16 sequence-heads at d = 128 do not fit (rejected
    # before any HIP call)
    far = 1 << 40
    rows_max = (16 << 20) // ((128 + 2) * 4)
    assert rows_max == 32263
    big = dict(q=far, k=2 * far, v=3 * far, seqlens=0, out=4 * far, lse=0, S_max=64, H_q=1, H_kv=1)
    assert _call_dec_noalloc(B=rows_max + 1, **big) == sqa.SQA_ERR_UNSUPPORTED
    assert _call_dec_noalloc(B=0, q=0, k=0, v=0, out=0) == sqa.SQA_OK
    assert _call_dec_noalloc(d=96) == sqa.SQA_ERR_UNSUPPORTED


# ---------------------------------------------------------------------------
# Only against the stub build: valid calls reach the launcher with the
# arguments the kernels expect (no GPU involved).


def _stub_last():
    lib = sqa.load_library()
    c, neg, qs, kvs, ws = (ctypes.c_float(), ctypes.c_int(), ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int())
    kind = lib.sqa_stub_last(ctypes.byref(c), ctypes.byref(neg), ctypes.byref(qs), ctypes.byref(kvs),
                             ctypes.byref(ws))
    return kind, c.value, neg.value, qs.value, kvs.value, ws.value


@pytest.mark.skipif(not STUB_LIB, reason="needs the host-only stub build of the C ABI")
def test_stub_valid_calls_reach_launchers():
    lib = sqa.load_library()
    lib.sqa_stub_reset()
    log2e = 1.4426950408889634
    assert _call(H_q=8, H_kv=2, d=128, scale=-0.25) == sqa.SQA_OK
    kind, c, neg, qs, kvs, _ = _stub_last()
    assert kind == 1 and neg == 1 and qs == 8 * 128 and kvs == 2 * 128
    assert abs(c - 0.25 * log2e) <= 1e-6
    assert _call(scale=0.0) == sqa.SQA_OK and 0 < _stub_last()[1] < 1e-20   # scale 0: a tiny positive factor
    assert _call_bwd() == sqa.SQA_OK and _stub_last()[0] == 2 and _stub_last()[5] == 1
    assert _call_dec() == sqa.SQA_OK and _stub_last()[0] == 3 and _stub_last()[5] == 1
    assert _call_dec_noalloc() == sqa.SQA_OK and _stub_last()[0] == 4 and _stub_last()[5] == 0
    assert _call_layer() == sqa.SQA_OK and _stub_last()[0] == 5 and _stub_last()[5] == 1
    lib.sqa_stub_reset()
    assert _call(H_q=6, H_kv=4) == sqa.SQA_ERR_INVALID_ARGUMENT and _stub_last()[0] == 0   # rejected: no launch
