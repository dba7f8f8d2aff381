"""Oracle for decoupled-head attention: plain fp64 CPU definition.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The product path
(the HIP library and its binding) never calls it and shares no code with it.

The arithmetic lives in ``sqa_oracle.c``; its header states what it computes
and which passage of the source pages each step follows.  This module only
marshals arguments.

Parity status: every function here is pinned by the not-gpu tests in
tests/test_oracle_pins.py (closed forms, invariants, a library routine and a
hand-derived fixture); none is "parity unpinned".
"""
import ctypes
import os

import numpy as np

from .build import build, lib_path

_lib = None

_DTYPE_CODE = {np.dtype(np.uint16): 0, np.dtype(np.float32): 1, np.dtype(np.float64): 2}


def _load():
    global _lib
    if _lib is None:
        # a test may point at another build of the same source (sanitizers)
        path = os.environ.get("SQA_ORACLE_LIB") or lib_path()
        if not os.path.exists(path):
            build()
        lib = ctypes.CDLL(path)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        lib.sqa_oracle_fwd.restype = ctypes.c_int
        lib.sqa_oracle_fwd.argtypes = [vp, vp, vp, ctypes.c_int, vp, i64, i64, i32, i32, i32,
                                       ctypes.c_double, ctypes.c_int, vp, i64, ctypes.c_int, vp]
        lib.sqa_oracle_lse.restype = ctypes.c_int
        lib.sqa_oracle_lse.argtypes = [vp, vp, ctypes.c_int, vp, i64, i64, i32, i32, i32, ctypes.c_double,
                                       ctypes.c_int, vp, i64, ctypes.c_int]
        lib.sqa_oracle_bwd.restype = ctypes.c_int
        lib.sqa_oracle_bwd.argtypes = [vp, vp, vp, vp, ctypes.c_int, vp, vp, vp, i64, i64, i32, i32, i32,
                                       ctypes.c_double, ctypes.c_int, ctypes.c_int]
        lib.sqa_oracle_bwd_dq_rows.restype = ctypes.c_int
        lib.sqa_oracle_bwd_dq_rows.argtypes = [vp, vp, vp, vp, ctypes.c_int, vp, i64, i64, i32, i32, i32,
                                               ctypes.c_double, ctypes.c_int, vp, i64, ctypes.c_int]
        lib.sqa_oracle_decode.restype = ctypes.c_int
        lib.sqa_oracle_decode.argtypes = [vp, vp, vp, ctypes.c_int, vp, vp, vp, i64, i64, i32, i32, i32,
                                          ctypes.c_double, ctypes.c_int]
        _lib = lib
    return _lib


def attention(q, k, v, scale, causal=False, rows=None, n_threads=0, return_pairs=False):
    """fp64 attention output.

    q: [B, S, H_q, d]; k, v: [B, S, H_kv, d]; all the same dtype: uint16
    (raw bf16 bits), float32 or float64.  `scale` is used as a double.
    rows: optional query positions; then the result is [B, len(rows), H_q, d]
    holding those positions only.  Returns float64 (and the number of
    (b, h, i, j) score terms evaluated if return_pairs).
    """
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in _DTYPE_CODE:
        raise TypeError("q, k, v must share one dtype among uint16(bf16 bits), float32, float64")
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be 4-d BSHD arrays")
    B, S, H_q, d = q.shape
    if k.shape[:2] != (B, S) or k.shape[3] != d or v.shape != k.shape:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
    H_kv = k.shape[2]
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        n_out = rows.size
        rows_ptr = ctypes.c_void_p(rows.ctypes.data)
    else:
        n_out = S
        rows_ptr = None
    out = np.zeros((B, n_out, H_q, d), dtype=np.float64)
    pairs = ctypes.c_int64(0)
    rc = _load().sqa_oracle_fwd(
        ctypes.c_void_p(q.ctypes.data), ctypes.c_void_p(k.ctypes.data), ctypes.c_void_p(v.ctypes.data),
        _DTYPE_CODE[q.dtype], ctypes.c_void_p(out.ctypes.data), B, S, H_q, H_kv, d, float(scale),
        1 if causal else 0, rows_ptr, n_out if rows is not None else 0, int(n_threads),
        ctypes.byref(pairs))
    if rc == -1:
        raise ValueError("oracle: invalid arguments")
    if rc != 0:
        raise MemoryError("oracle: allocation failed")
    return (out, pairs.value) if return_pairs else out


def lse(q, k, scale, causal=False, rows=None, n_threads=0):
    """fp64 log of the softmax normaliser per (b, row, head): [B, n_rows, H_q]."""
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    if q.dtype != k.dtype or q.dtype not in _DTYPE_CODE:
        raise TypeError("q, k must share one dtype among uint16(bf16 bits), float32, float64")
    B, S, H_q, d = q.shape
    if k.shape[:2] != (B, S) or k.shape[3] != d:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape}")
    H_kv = k.shape[2]
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        n_out, rows_ptr = rows.size, ctypes.c_void_p(rows.ctypes.data)
    else:
        n_out, rows_ptr = S, None
    out = np.zeros((B, n_out, H_q), dtype=np.float64)
    rc = _load().sqa_oracle_lse(ctypes.c_void_p(q.ctypes.data), ctypes.c_void_p(k.ctypes.data),
                                _DTYPE_CODE[q.dtype], ctypes.c_void_p(out.ctypes.data), B, S, H_q, H_kv, d,
                                float(scale), 1 if causal else 0, rows_ptr, n_out if rows is not None else 0,
                                int(n_threads))
    if rc == -1:
        raise ValueError("oracle: invalid arguments")
    if rc != 0:
        raise MemoryError("oracle: allocation failed")
    return out


def attention_grad(q, k, v, dout, scale, causal=False, n_threads=0):
    """fp64 (dq, dk, dv) of the attention for upstream gradient dout (shape of q)."""
    arrs = [np.ascontiguousarray(a) for a in (q, k, v, dout)]
    q, k, v, dout = arrs
    if len({a.dtype for a in arrs}) != 1 or q.dtype not in _DTYPE_CODE:
        raise TypeError("q, k, v, dout must share one dtype among uint16(bf16 bits), float32, float64")
    B, S, H_q, d = q.shape
    if k.shape[:2] != (B, S) or k.shape[3] != d or v.shape != k.shape or dout.shape != q.shape:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape} dout{dout.shape}")
    H_kv = k.shape[2]
    dq = np.zeros(q.shape, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(k.shape, dtype=np.float64)
    ptr = lambda a: ctypes.c_void_p(a.ctypes.data)
    rc = _load().sqa_oracle_bwd(ptr(q), ptr(k), ptr(v), ptr(dout), _DTYPE_CODE[q.dtype], ptr(dq), ptr(dk), ptr(dv),
                                B, S, H_q, H_kv, d, float(scale), 1 if causal else 0, int(n_threads))
    if rc == -1:
        raise ValueError("oracle: invalid arguments")
    if rc != 0:
        raise MemoryError("oracle: allocation failed")
    return dq, dk, dv


def attention_grad_dq_rows(q, k, v, dout, scale, rows, causal=False, n_threads=0):
    """fp64 dq at the query positions `rows` only: [B, len(rows), H_q, d]."""
    arrs = [np.ascontiguousarray(a) for a in (q, k, v, dout)]
    q, k, v, dout = arrs
    if len({a.dtype for a in arrs}) != 1 or q.dtype not in _DTYPE_CODE:
        raise TypeError("q, k, v, dout must share one dtype")
    B, S, H_q, d = q.shape
    H_kv = k.shape[2]
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.zeros((B, rows.size, H_q, d), dtype=np.float64)
    ptr = lambda a: ctypes.c_void_p(a.ctypes.data)
    rc = _load().sqa_oracle_bwd_dq_rows(ptr(q), ptr(k), ptr(v), ptr(dout), _DTYPE_CODE[q.dtype], ptr(out), B, S, H_q,
                                        H_kv, d, float(scale), 1 if causal else 0, ptr(rows), rows.size, int(n_threads))
    if rc == -1:
        raise ValueError("oracle: invalid arguments")
    if rc != 0:
        raise MemoryError("oracle: allocation failed")
    return out


def decode(q, k, v, scale, seqlens=None, n_threads=0):
    """fp64 attention of one query token per sequence against its K/V cache.

    q: [B, H_q, d]; k, v: [B, S_max, H_kv, d]; one dtype among uint16 (bf16
    bits), float32, float64.  seqlens: per-sequence valid cache length
    (None = S_max); lengths above S_max count as S_max, lengths <= 0 give
    out = 0 and lse = -inf.  Returns (out [B, H_q, d], lse [B, H_q]), float64.
    """
    arrs = [np.ascontiguousarray(a) for a in (q, k, v)]
    q, k, v = arrs
    if len({a.dtype for a in arrs}) != 1 or q.dtype not in _DTYPE_CODE:
        raise TypeError("q, k, v must share one dtype among uint16(bf16 bits), float32, float64")
    if q.ndim != 3 or k.ndim != 4 or v.shape != k.shape:
        raise ValueError(f"expected q [B,H_q,d] and k, v [B,S_max,H_kv,d]; got q{q.shape} k{k.shape} v{v.shape}")
    B, H_q, d = q.shape
    S_max, H_kv = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != d:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape}")
    lens = None
    if seqlens is not None:
        lens = np.ascontiguousarray(seqlens, dtype=np.int64)
        if lens.shape != (B,):
            raise ValueError("seqlens must have one entry per sequence")
    out = np.zeros((B, H_q, d), dtype=np.float64)
    lse_out = np.zeros((B, H_q), dtype=np.float64)
    ptr = lambda a: ctypes.c_void_p(a.ctypes.data)
    rc = _load().sqa_oracle_decode(ptr(q), ptr(k), ptr(v), _DTYPE_CODE[q.dtype], ptr(lens) if lens is not None else None,
                                   ptr(out), ptr(lse_out), B, S_max, H_q, H_kv, d, float(scale), int(n_threads))
    if rc == -1:
        raise ValueError("oracle: invalid arguments")
    if rc != 0:
        raise MemoryError("oracle: allocation failed")
    return out, lse_out


def _as_f64(a):
    """bf16 bits (uint16), float32 or float64 array -> float64 (exact)."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def layer(x, w_qkv, w_o, H_q, H_kv, d, scale, causal=False, rows=None, n_threads=0):
    """fp64 forward of the full attention layer (GQA explainer, PyTorch module:
    q/k/v projections, K/V shared by groups of query heads, scaled dot-product
    attention, output projection; with the query-head count H_q free as in the
    SQA abstract):

        [q | k | v] = x W_qkv^T,   attn = attention(q, k, v),   out = attn W_o^T

    x [B, S, d_model]; w_qkv [(H_q + 2 H_kv) d, d_model] (q, k, v weights stacked,
    nn.Linear layout); w_o [d_model, H_q d].  The projections are library
    matrix products in fp64 (no rounding in between); the attention is
    attention() above.  rows: optional output positions (all keys are still
    projected).  Returns float64 [B, n_rows, d_model].
    """
    xf, wq, wo = _as_f64(x), _as_f64(w_qkv), _as_f64(w_o)
    B, S, dm = xf.shape
    nq, nkv = H_q * d, H_kv * d
    if wq.shape != (nq + 2 * nkv, dm) or wo.shape != (dm, nq):
        raise ValueError(f"weight shapes {wq.shape} {wo.shape} do not match H_q={H_q} H_kv={H_kv} d={d} d_model={dm}")
    kv = xf @ wq[nq:].T                                         # [B, S, 2 H_kv d]
    k = np.ascontiguousarray(kv[..., :nkv].reshape(B, S, H_kv, d))
    v = np.ascontiguousarray(kv[..., nkv:].reshape(B, S, H_kv, d))
    xq = xf if rows is None else xf[:, np.asarray(rows)]
    q_rows = xq @ wq[:nq].T                                    # [B, n, H_q d]
    if rows is None:
        q = np.ascontiguousarray(q_rows.reshape(B, S, H_q, d))
        attn = attention(q, k, v, scale, causal=causal, n_threads=n_threads)
    else:
        # place the selected query rows at their positions; the others are unused
        q = np.zeros((B, S, H_q, d))
        q[:, np.asarray(rows)] = q_rows.reshape(B, -1, H_q, d)
        attn = attention(q, k, v, scale, causal=causal, rows=rows, n_threads=n_threads)
    return attn.reshape(B, attn.shape[1], nq) @ wo.T
