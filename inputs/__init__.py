"""Seeded synthetic inputs for decoupled-head attention.

The generator (``gen.c``) draws counter-based SplitMix64 uniforms and turns
them into normals by Box-Muller; values are encoded as fp32 or bf16 (round to
nearest even).  It holds no attention arithmetic, so both sides of every
comparison (the HIP library and the oracle) read the same input bits from it.
"""
import ctypes
import os

import numpy as np

from .build import build, lib_path

_lib = None


def _load():
    global _lib
    if _lib is None:
        # a test may point at another build of the same source (sanitizers)
        path = os.environ.get("SQA_INPUTS_LIB") or lib_path()
        if not os.path.exists(path):
            build()
        lib = ctypes.CDLL(path)
        i64, u64, f64 = ctypes.c_int64, ctypes.c_uint64, ctypes.c_double
        vp = ctypes.c_void_p
        lib.sqa_gen_splitmix64.restype = u64
        lib.sqa_gen_splitmix64.argtypes = [u64]
        lib.sqa_gen_hash.restype = u64
        lib.sqa_gen_hash.argtypes = [u64, u64, u64]
        lib.sqa_gen_uniform.restype = f64
        lib.sqa_gen_uniform.argtypes = [u64, u64, u64]
        lib.sqa_gen_normal_f32.restype = None
        lib.sqa_gen_normal_f32.argtypes = [u64, u64, f64, i64, vp]
        lib.sqa_gen_normal_bf16.restype = None
        lib.sqa_gen_normal_bf16.argtypes = [u64, u64, f64, i64, vp]
        lib.sqa_gen_f32_to_bf16.restype = None
        lib.sqa_gen_f32_to_bf16.argtypes = [vp, i64, vp]
        lib.sqa_gen_select_positions.restype = ctypes.c_int
        lib.sqa_gen_select_positions.argtypes = [u64, u64, i64, i64, vp]
        lib.sqa_gen_scale_positions_bf16.restype = None
        lib.sqa_gen_scale_positions_bf16.argtypes = [vp, i64, i64, i64, vp, i64, ctypes.c_float]
        _lib = lib
    return _lib


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data)


def splitmix64(state):
    """First SplitMix64 output for the given state (state + gamma, then mix)."""
    return int(_load().sqa_gen_splitmix64(state))


def hash64(seed, stream, counter):
    return int(_load().sqa_gen_hash(seed, stream, counter))


def uniform(seed, stream, counter):
    return float(_load().sqa_gen_uniform(seed, stream, counter))


def normal(seed, stream, shape, dtype="bf16", mul=1.0):
    """Array of shape `shape` with element i = encode(mul * z(i)).

    dtype "bf16" returns raw bf16 bits as uint16; "f32" returns float32.
    """
    n = int(np.prod(shape, dtype=np.int64))
    if dtype == "bf16":
        out = np.empty(shape, dtype=np.uint16)
        _load().sqa_gen_normal_bf16(seed, stream, float(mul), n, _ptr(out))
    elif dtype == "f32":
        out = np.empty(shape, dtype=np.float32)
        _load().sqa_gen_normal_f32(seed, stream, float(mul), n, _ptr(out))
    else:
        raise ValueError(f"unknown dtype {dtype!r}")
    return out


def f32_to_bf16_bits(x):
    """Round-to-nearest-even fp32 -> bf16, returned as uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().sqa_gen_f32_to_bf16(_ptr(x), x.size, _ptr(out))
    return out


def bf16_bits_to_f32(bits):
    """Exact bf16 -> fp32 widening (the bf16 bits are an fp32's upper half)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def select_positions(seed, stream, S, n):
    """n distinct positions of [0, S), seeded partial Fisher-Yates, ascending."""
    out = np.empty(n, dtype=np.int64)
    if _load().sqa_gen_select_positions(seed, stream, S, n, _ptr(out)) != 0:
        raise ValueError("select_positions: n > S or out of memory")
    return out


def scale_positions_bf16(x, positions, factor):
    """In place: x[b, s, ...] *= factor for s in positions (bf16 bits, RNE)."""
    assert x.dtype == np.uint16 and x.flags.c_contiguous
    B, S = x.shape[0], x.shape[1]
    row = int(np.prod(x.shape[2:], dtype=np.int64))
    pos = np.ascontiguousarray(positions, dtype=np.int64)
    _load().sqa_gen_scale_positions_bf16(_ptr(x), B, S, row, _ptr(pos), pos.size, float(factor))
    return x
