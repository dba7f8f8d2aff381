"""Python binding of libsqa: decoupled-head attention on MI355X (forward,
backward, decode, full layer), and `attention`, the forward and backward
joined for torch.autograd.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``lib/libsqa.so`` (sources in ``csrc/``, C-ABI in
``include/sqa.h``).  There is no CPU fallback; if the library is missing the
import of the native entry points fails loudly.
"""
import ctypes
import math
import os

from ._build import build, lib_path

SQA_OK, SQA_ERR_INVALID_ARGUMENT, SQA_ERR_UNSUPPORTED, SQA_ERR_HIP = 0, 1, 2, 3
SQA_BF16, SQA_FP32 = 0, 1

_lib = None


class SqaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{message} (status {status})")
        self.status = status


def _check_buffer(name, t, shape, dtype, device):
    """A caller-supplied output or lse tensor: on the GPU next to the inputs,
    contiguous, with exactly the expected shape and dtype (the C ABI sees only
    the address, so a wrong buffer would be written out of bounds)."""
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be a GPU tensor on {device}")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)}; "
                         f"got {t.dtype} {tuple(t.shape)}")


def _workspace(t, need, device):
    """A caller-supplied workspace (or a new one): a contiguous GPU tensor on
    `device` of at least `need` bytes.  Returns it and its size in bytes."""
    import torch

    if t is None:
        t = torch.empty(max(need, 16), dtype=torch.uint8, device=device)
    if not t.is_cuda or t.device != device or not t.is_contiguous():
        raise ValueError(f"workspace must be a contiguous GPU tensor on {device}")
    nbytes = t.numel() * t.element_size()
    if nbytes < need:
        raise ValueError(f"workspace holds {nbytes} bytes; {need} needed")
    return t, nbytes


def _check_inputs(tensors, device):
    for name, t in tensors:
        if not t.is_cuda or t.device != device:
            raise ValueError(f"{name} must be a GPU tensor on {device}")


def load_library(path=None):
    """Load libsqa.so (build it first if it is absent) and declare its symbols."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    path = path or lib_path()
    if not os.path.exists(path):
        build()
    lib = ctypes.CDLL(path)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.sqa_attn_fwd.restype = ctypes.c_int
    lib.sqa_attn_fwd.argtypes = [vp, vp, vp, vp, i64, i64, i32, i32, i32, ctypes.c_int, ctypes.c_float,
                                 ctypes.c_int, vp]
    lib.sqa_attn_fwd_lse.restype = ctypes.c_int
    lib.sqa_attn_fwd_lse.argtypes = [vp, vp, vp, vp, vp, i64, i64, i32, i32, i32, ctypes.c_int, ctypes.c_float,
                                     ctypes.c_int, vp]
    lib.sqa_attn_bwd.restype = ctypes.c_int
    lib.sqa_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, ctypes.c_int,
                                 ctypes.c_float, ctypes.c_int, vp]
    lib.sqa_attn_bwd_workspace_size.restype = i64
    lib.sqa_attn_bwd_workspace_size.argtypes = [i64, i64, i32]
    lib.sqa_attn_decode.restype = ctypes.c_int
    lib.sqa_attn_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, ctypes.c_int,
                                    ctypes.c_float, vp]
    lib.sqa_attn_decode_noalloc.restype = ctypes.c_int
    lib.sqa_attn_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i32, i32, i32, ctypes.c_int,
                                            ctypes.c_float, vp]
    lib.sqa_attn_decode_workspace_size.restype = i64
    lib.sqa_attn_decode_workspace_size.argtypes = [i64, i64, i32, i32, i32]
    lib.sqa_layer_fwd.restype = ctypes.c_int
    lib.sqa_layer_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, i32, ctypes.c_float, ctypes.c_int,
                                  vp]
    lib.sqa_layer_workspace_size.restype = i64
    lib.sqa_layer_workspace_size.argtypes = [i64, i64, i32, i32, i32]
    lib.sqa_status_string.restype = ctypes.c_char_p
    lib.sqa_status_string.argtypes = [ctypes.c_int]
    _lib = lib
    return lib


def status_string(status):
    return load_library().sqa_status_string(status).decode()


def attn_fwd_raw(q, k, v, out, B, S, H_q, H_kv, d, dtype, scale, causal, stream):
    """Direct call of sqa_attn_fwd with integer device addresses; returns the status."""
    return load_library().sqa_attn_fwd(q, k, v, out, B, S, H_q, H_kv, d, dtype, scale, int(causal),
                                       stream)


def attn_fwd_lse_raw(q, k, v, out, lse, B, S, H_q, H_kv, d, dtype, scale, causal, stream):
    """Direct call of sqa_attn_fwd_lse with integer device addresses; returns the status."""
    return load_library().sqa_attn_fwd_lse(q, k, v, out, lse, B, S, H_q, H_kv, d, dtype, scale, int(causal),
                                           stream)


def attn_fwd(q, k, v, out=None, scale=None, causal=False, stream=None, return_lse=False, lse=None):
    """out[b,i,h] = softmax_j(scale * q[b,i,h].k[b,j,h//R]) . v[b,j,h//R].

    q: [B, S, H_q, d], k and v: [B, S, H_kv, d], torch tensors on the GPU,
    contiguous, all bfloat16 or all float32.  scale defaults to 1/sqrt(d).
    The kernel is enqueued on `stream` (default: torch's current stream).
    With return_lse (or an `lse` tensor given) also returns the fp32
    [B, S, H_q] row log-normaliser ln(sum_j exp(scale * q.k_j)).
    """
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or not t.is_contiguous() or t.dim() != 4:
            raise ValueError(f"{name} must be a contiguous 4-d GPU tensor")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share one dtype")
    if q.dtype == torch.bfloat16:
        dtype = SQA_BF16
    elif q.dtype == torch.float32:
        dtype = SQA_FP32
    else:
        raise ValueError(f"unsupported dtype {q.dtype}")
    B, S, H_q, d = q.shape
    if tuple(k.shape[:2]) != (B, S) or k.shape[3] != d or k.shape != v.shape:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    H_kv = k.shape[2]
    _check_inputs((("k", k), ("v", v)), q.device)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_buffer("out", out, q.shape, q.dtype, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    if return_lse or lse is not None:
        if lse is None:
            lse = torch.empty((B, S, H_q), dtype=torch.float32, device=q.device)
        else:
            _check_buffer("lse", lse, (B, S, H_q), torch.float32, q.device)
        st = attn_fwd_lse_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, S,
                              H_q, H_kv, d, dtype, float(scale), causal, handle)
        if st != SQA_OK:
            raise SqaError(st, status_string(st))
        return out, lse
    st = attn_fwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, S, H_q, H_kv, d,
                      dtype, float(scale), causal, handle)
    if st != SQA_OK:
        raise SqaError(st, status_string(st))
    return out


def attn_bwd_workspace_size(B, S, H_q):
    return int(load_library().sqa_attn_bwd_workspace_size(B, S, H_q))


def attn_bwd_raw(q, k, v, out, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, S, H_q, H_kv, d, dtype, scale,
                 causal, stream):
    """Direct call of sqa_attn_bwd with integer device addresses; returns the status."""
    return load_library().sqa_attn_bwd(q, k, v, out, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, S, H_q,
                                       H_kv, d, dtype, scale, int(causal), stream)


def attn_bwd(q, k, v, out, dout, lse, scale=None, causal=False, stream=None, dq=None, dk=None, dv=None,
             workspace=None):
    """Gradients (dq, dk, dv) of attn_fwd's output for upstream gradient dout.

    q, k, v, out and lse as given to / returned by attn_fwd(..., return_lse=True)
    with the same scale and causal flag; dout shaped like out.  Returns new
    tensors unless dq, dk, dv are given.  A uint8 workspace of
    attn_bwd_workspace_size(B, S, H_q) bytes is allocated if none is given.
    """
    import torch

    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
        if not t.is_cuda or not t.is_contiguous() or t.dim() != 4:
            raise ValueError(f"{name} must be a contiguous 4-d GPU tensor")
    if not (q.dtype == k.dtype == v.dtype == out.dtype == dout.dtype):
        raise ValueError("q, k, v, out, dout must share one dtype")
    dtype = SQA_BF16 if q.dtype == torch.bfloat16 else SQA_FP32 if q.dtype == torch.float32 else None
    if dtype is None:
        raise ValueError(f"unsupported dtype {q.dtype}")
    B, S, H_q, d = q.shape
    H_kv = k.shape[2]
    if out.shape != q.shape or dout.shape != q.shape or k.shape != v.shape or tuple(k.shape[:2]) != (B, S):
        raise ValueError("shape mismatch")
    _check_inputs((("k", k), ("v", v), ("out", out), ("dout", dout)), q.device)
    _check_buffer("lse", lse, (B, S, H_q), torch.float32, q.device)
    for name, t, like in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t is not None:
            _check_buffer(name, t, like.shape, like.dtype, q.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    ws_bytes = attn_bwd_workspace_size(B, S, H_q)
    if ws_bytes < 0:
        raise ValueError("invalid sizes")
    workspace, ws_have = _workspace(workspace, ws_bytes, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    st = attn_bwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                      dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(), ws_have, B, S, H_q,
                      H_kv, d, dtype, float(scale), causal, handle)
    if st != SQA_OK:
        raise SqaError(st, status_string(st))
    return dq, dk, dv


_attention_fn = None


def attention(q, k, v, scale=None, causal=False):
    """attn_fwd with autograd: the forward runs sqa_attn_fwd_lse and keeps
    its output and row log-normaliser; backward() runs sqa_attn_bwd on
    them.  q, k, v as for attn_fwd (contiguous GPU tensors, one dtype);
    gradients flow to whichever of them require them.  The upstream
    gradient is made contiguous (a copy only if it is not)."""
    global _attention_fn
    import torch

    if _attention_fn is None:
        class _Attention(torch.autograd.Function):
            @staticmethod
            def forward(ctx, q_, k_, v_, scale_, causal_):
                out, lse = attn_fwd(q_, k_, v_, scale=scale_, causal=causal_, return_lse=True)
                ctx.save_for_backward(q_, k_, v_, out, lse)
                ctx.scale, ctx.causal = scale_, causal_
                return out

            @staticmethod
            def backward(ctx, dout):
                q_, k_, v_, out, lse = ctx.saved_tensors
                dq, dk, dv = attn_bwd(q_, k_, v_, out, dout.contiguous(), lse, scale=ctx.scale, causal=ctx.causal)
                return dq, dk, dv, None, None

        _attention_fn = _Attention
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    return _attention_fn.apply(q, k, v, float(scale), bool(causal))


def attn_decode_workspace_size(B, S_max, H_q, H_kv, d):
    return int(load_library().sqa_attn_decode_workspace_size(B, S_max, H_q, H_kv, d))


def attn_decode_raw(q, k_cache, v_cache, seqlens, out, lse, workspace, workspace_bytes, B, S_max, H_q, H_kv, d,
                    dtype, scale, stream):
    """Direct call of sqa_attn_decode with integer device addresses; returns the status."""
    return load_library().sqa_attn_decode(q, k_cache, v_cache, seqlens, out, lse, workspace, workspace_bytes, B,
                                          S_max, H_q, H_kv, d, dtype, scale, stream)


def attn_decode(q, k_cache, v_cache, seqlens=None, out=None, scale=None, stream=None, return_lse=False, lse=None,
                workspace=None):
    """One query token per sequence against its key/value cache.

    q: [B, H_q, d]; k_cache, v_cache: [B, S_max, H_kv, d]; all bfloat16 or all float32;
    seqlens: int32 [B] GPU tensor of cache lengths (None = S_max).  Returns
    out [B, H_q, d] (and the fp32 [B, H_q] log-normaliser with return_lse).
    A uint8 workspace of attn_decode_workspace_size(...) bytes is allocated
    if none is given.
    """
    import torch

    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        if not t.is_cuda or not t.is_contiguous() or t.dtype not in (torch.bfloat16, torch.float32):
            raise ValueError(f"{name} must be a contiguous bfloat16 or float32 GPU tensor")
    if not (q.dtype == k_cache.dtype == v_cache.dtype):
        raise ValueError("q, k_cache, v_cache must share one dtype")
    dtype = SQA_BF16 if q.dtype == torch.bfloat16 else SQA_FP32
    if q.dim() != 3 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError(f"expected q [B,H_q,d], caches [B,S_max,H_kv,d]; got q{tuple(q.shape)} "
                         f"k{tuple(k_cache.shape)} v{tuple(v_cache.shape)}")
    B, H_q, d = q.shape
    S_max, H_kv = k_cache.shape[1], k_cache.shape[2]
    if k_cache.shape[0] != B or k_cache.shape[3] != d:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k_cache.shape)}")
    _check_inputs((("k_cache", k_cache), ("v_cache", v_cache)), q.device)
    if seqlens is not None:
        _check_buffer("seqlens", seqlens, (B,), torch.int32, q.device)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_buffer("out", out, q.shape, q.dtype, q.device)
    if return_lse and lse is None:
        lse = torch.empty((B, H_q), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check_buffer("lse", lse, (B, H_q), torch.float32, q.device)
    ws_bytes = attn_decode_workspace_size(B, S_max, H_q, H_kv, d)
    if ws_bytes < 0:
        raise ValueError("invalid sizes")
    workspace, ws_have = _workspace(workspace, ws_bytes, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    st = attn_decode_raw(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                         seqlens.data_ptr() if seqlens is not None else None, out.data_ptr(),
                         lse.data_ptr() if lse is not None else None, workspace.data_ptr(), ws_have,
                         B, S_max, H_q, H_kv, d, dtype,
                         float(scale), handle)
    if st != SQA_OK:
        raise SqaError(st, status_string(st))
    return (out, lse) if (return_lse or lse is not None) else out


def attn_decode_noalloc_raw(q, k_cache, v_cache, seqlens, out, lse, B, S_max, H_q, H_kv, d, dtype, scale, stream):
    """Direct call of sqa_attn_decode_noalloc (no workspace: the library's
    fixed per-GPU scratch holds the partial results); returns the status."""
    return load_library().sqa_attn_decode_noalloc(q, k_cache, v_cache, seqlens, out, lse, B, S_max, H_q, H_kv, d,
                                                  dtype, scale, stream)


def layer_workspace_size(B, S, H_q, H_kv, d):
    return int(load_library().sqa_layer_workspace_size(B, S, H_q, H_kv, d))


def layer_fwd_raw(x, w_qkv, w_o, out, workspace, workspace_bytes, B, S, d_model, H_q, H_kv, d, scale, causal, stream):
    """Direct call of sqa_layer_fwd with integer device addresses; returns the status."""
    return load_library().sqa_layer_fwd(x, w_qkv, w_o, out, workspace, workspace_bytes, B, S, d_model, H_q, H_kv, d,
                                        scale, int(causal), stream)


def layer_fwd(x, w_qkv, w_o, H_q, H_kv, out=None, scale=None, causal=False, stream=None, workspace=None):
    """Attention layer forward: [q|k|v] = x W_qkv^T, attention with H_q query
    and H_kv K/V heads (head size (W_qkv rows) / (H_q + 2 H_kv)), out = attn W_o^T.

    x: [B, S, d_model]; w_qkv: [(H_q + 2 H_kv) d, d_model]; w_o: [d_model, H_q d];
    contiguous bfloat16 GPU tensors.  A uint8 workspace of
    layer_workspace_size(B, S, H_q, H_kv, d) bytes is allocated if none is given.
    """
    import torch

    for name, t in (("x", x), ("w_qkv", w_qkv), ("w_o", w_o)):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be a contiguous bfloat16 GPU tensor")
    if x.dim() != 3 or w_qkv.dim() != 2 or w_o.dim() != 2:
        raise ValueError("expected x [B,S,d_model], w_qkv [(H_q+2H_kv)d, d_model], w_o [d_model, H_q d]")
    B, S, d_model = x.shape
    rows_qkv = w_qkv.shape[0]
    if rows_qkv % (H_q + 2 * H_kv) != 0:
        raise ValueError("w_qkv rows must be (H_q + 2 H_kv) * d")
    d = rows_qkv // (H_q + 2 * H_kv)
    if w_qkv.shape[1] != d_model or tuple(w_o.shape) != (d_model, H_q * d):
        raise ValueError(f"weight shapes {tuple(w_qkv.shape)} {tuple(w_o.shape)} do not match x {tuple(x.shape)}")
    _check_inputs((("w_qkv", w_qkv), ("w_o", w_o)), x.device)
    if out is None:
        out = torch.empty_like(x)
    else:
        _check_buffer("out", out, x.shape, x.dtype, x.device)
    ws_bytes = layer_workspace_size(B, S, H_q, H_kv, d)
    if ws_bytes < 0:
        raise ValueError("invalid sizes")
    workspace, ws_have = _workspace(workspace, ws_bytes, x.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    st = layer_fwd_raw(x.data_ptr(), w_qkv.data_ptr(), w_o.data_ptr(), out.data_ptr(), workspace.data_ptr(),
                       ws_have, B, S, d_model, H_q, H_kv, d, float(scale),
                       causal, handle)
    if st != SQA_OK:
        raise SqaError(st, status_string(st))
    return out
