"""Workload recipes: the five attention shapes the method is measured on.

Shapes follow the Sparse Query Attention abstract's setting (long sequences
of 32k-200k tokens, compute-bound full-sequence passes) plus a tiny fp32 case
and a 4k head-configuration sweep.  Inputs are synthetic: i.i.d. normals from
the seeded generator, scaled by 0.5 and rounded to bf16 for the bf16 cases.
The 200k case also multiplies 1% of the key positions by 8 so that some
softmax rows are sharply peaked.

Seeds: 0x5A510000 + 16 * config_number + variant_index.
Streams: q = 0, k = 1, v = 2, key-position selection = 3, cache lengths = 4,
layer input x = 6, W_qkv = 7, W_o = 8.

Decode workloads (one new token per sequence against its key/value cache)
take their head shapes from the GQA explainer's KV-cache table (32 query
heads with 8 K/V groups as in Llama 3 8B, MHA with 32, MQA with 1; d_h = 128)
and its note that GQA-8 brings 128K-token contexts within reach; the SQA
variant halves the query heads at the same 8 K/V groups.  Cache lengths are a
seeded mix shared by all variants of a workload (seed of its first variant):
sequence 0 fills the cache, the others are uniform in [S_max/4, S_max].
"""
import math
from dataclasses import dataclass, field

import numpy as np

from . import normal, scale_positions_bf16, select_positions, uniform

SEED_BASE = 0x5A510000
STREAM_Q, STREAM_K, STREAM_V, STREAM_SEL, STREAM_LEN = 0, 1, 2, 3, 4
STREAM_X, STREAM_WQKV, STREAM_WO = 6, 7, 8


@dataclass(frozen=True)
class Variant:
    name: str
    H_q: int
    H_kv: int


@dataclass(frozen=True)
class Workload:
    number: int
    name: str
    B: int
    S: int
    d: int
    causal: bool
    dtype: str          # "bf16" or "f32"
    mul: float          # values are mul * N(0, 1)
    variants: tuple
    peaked_fraction: float = 0.0   # fraction of key positions scaled
    peaked_factor: float = 1.0
    notes: str = ""

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.d)

    def variant(self, name):
        for v in self.variants:
            if v.name == name:
                return v
        raise KeyError(name)

    def seed(self, variant_name):
        idx = [v.name for v in self.variants].index(variant_name)
        return SEED_BASE + 16 * self.number + idx


WORKLOADS = {
    "tiny_f32": Workload(1, "tiny_f32", B=1, S=256, d=32, causal=False, dtype="f32", mul=1.0,
                         variants=(Variant("gqa", 4, 2),)),
    "sweep_s4096": Workload(2, "sweep_s4096", B=2, S=4096, d=64, causal=False, dtype="bf16", mul=0.5,
                            variants=(Variant("mha", 16, 16), Variant("gqa", 16, 4),
                                      Variant("sqa", 8, 4), Variant("xsqa", 4, 4))),
    "encoder_s32k": Workload(3, "encoder_s32k", B=1, S=32768, d=128, causal=False, dtype="bf16", mul=0.5,
                             variants=(Variant("sqa", 8, 8), Variant("mha", 16, 16))),
    "causal_s131k": Workload(4, "causal_s131k", B=1, S=131072, d=128, causal=True, dtype="bf16", mul=0.5,
                             variants=(Variant("sqa", 4, 4), Variant("mha", 16, 16))),
    "ragged_s200k": Workload(5, "ragged_s200k", B=1, S=200000, d=128, causal=True, dtype="bf16", mul=0.5,
                             variants=(Variant("sqa", 8, 2), Variant("gqa", 16, 2)),
                             peaked_fraction=0.01, peaked_factor=8.0),
}


def make_inputs(workload, variant_name, S=None, B=None):
    """Host arrays (q, k, v) for one workload variant.

    bf16 workloads return uint16 bf16 bits, fp32 ones float32; all BSHD.
    S and B may be overridden to get a shorter sequence with the same recipe.
    """
    w = workload
    v = w.variant(variant_name)
    S = w.S if S is None else S
    B = w.B if B is None else B
    seed = w.seed(variant_name)
    q = normal(seed, STREAM_Q, (B, S, v.H_q, w.d), w.dtype, w.mul)
    k = normal(seed, STREAM_K, (B, S, v.H_kv, w.d), w.dtype, w.mul)
    vv = normal(seed, STREAM_V, (B, S, v.H_kv, w.d), w.dtype, w.mul)
    peaked = np.empty(0, dtype=np.int64)
    if w.peaked_fraction > 0:
        n = int(math.floor(w.peaked_fraction * S))
        peaked = select_positions(seed, STREAM_SEL, S, n)
        scale_positions_bf16(k, peaked, w.peaked_factor)
    return q, k, vv, peaked



@dataclass(frozen=True)
class DecodeWorkload:
    number: int
    name: str
    B: int
    S_max: int
    d: int
    mul: float
    variants: tuple
    min_len_frac: float = 0.25
    dtype: str = "bf16"

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.d)

    def variant(self, name):
        for v in self.variants:
            if v.name == name:
                return v
        raise KeyError(name)

    def seed(self, variant_name):
        idx = [v.name for v in self.variants].index(variant_name)
        return SEED_BASE + 16 * self.number + idx


DECODE_WORKLOADS = {
    "decode_s128k": DecodeWorkload(6, "decode_s128k", B=4, S_max=131072, d=128, mul=0.5,
                                   variants=(Variant("gqa", 32, 8), Variant("mha", 32, 32),
                                             Variant("mqa", 32, 1), Variant("sqa", 16, 8))),
}


def decode_lengths(seed, B, S_max, min_len_frac):
    """Cache length per sequence: sequence 0 is full, the others uniform
    integers in [ceil(min_len_frac * S_max), S_max] from stream 4."""
    lo = max(1, int(math.ceil(min_len_frac * S_max)))
    lens = np.empty(B, dtype=np.int64)
    for b in range(B):
        if b == 0:
            lens[b] = S_max
        else:
            u = uniform(seed, STREAM_LEN, b)          # in (0, 1]
            lens[b] = min(S_max, lo + int(math.floor(u * (S_max - lo + 1))))
    return lens


def make_decode_inputs(workload, variant_name, S_max=None, B=None):
    """Host arrays for one decode variant: q [B, H_q, d], k and v caches
    [B, S_max, H_kv, d] (bf16 bits), and the int64 cache lengths [B].
    Cache positions at or past a sequence's length hold values too (as a
    reused cache buffer would); they must not affect the result."""
    w = workload
    v = w.variant(variant_name)
    S_max = w.S_max if S_max is None else S_max
    B = w.B if B is None else B
    seed = w.seed(variant_name)
    q = normal(seed, STREAM_Q, (B, v.H_q, w.d), w.dtype, w.mul)
    k = normal(seed, STREAM_K, (B, S_max, v.H_kv, w.d), w.dtype, w.mul)
    vv = normal(seed, STREAM_V, (B, S_max, v.H_kv, w.d), w.dtype, w.mul)
    lens = decode_lengths(w.seed(w.variants[0].name), B, S_max, w.min_len_frac)
    return q, k, vv, lens


@dataclass(frozen=True)
class LayerWorkload:
    """A full attention layer (projections + attention) at one shape.  The
    model width is the baseline's H * d; SQA variants shrink the query heads
    (and so the q and output projections) at that width."""
    number: int
    name: str
    B: int
    S: int
    d_model: int
    d: int
    causal: bool
    variants: tuple
    dtype: str = "bf16"

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.d)

    def variant(self, name):
        for v in self.variants:
            if v.name == name:
                return v
        raise KeyError(name)

    def seed(self, variant_name):
        idx = [v.name for v in self.variants].index(variant_name)
        return SEED_BASE + 16 * self.number + idx


LAYER_WORKLOADS = {
    "layer_s32k": LayerWorkload(7, "layer_s32k", B=1, S=32768, d_model=2048, d=128, causal=False,
                                variants=(Variant("sqa", 8, 8), Variant("mha", 16, 16), Variant("xsqa", 4, 4),
                                          Variant("gqa", 16, 4))),
}


def make_layer_inputs(workload, variant_name, S=None, B=None, d_model=None):
    """x [B, S, d_model] ~ N(0, 1); W_qkv [(H_q + 2 H_kv) d, d_model] and
    W_o [d_model, H_q d] ~ N(0, 1/fan_in) (the spread of nn.Linear's default
    initialisation); all bf16 bits."""
    w = workload
    v = w.variant(variant_name)
    S = w.S if S is None else S
    B = w.B if B is None else B
    dm = w.d_model if d_model is None else d_model
    seed = w.seed(variant_name)
    x = normal(seed, STREAM_X, (B, S, dm), w.dtype, 1.0)
    w_qkv = normal(seed, STREAM_WQKV, ((v.H_q + 2 * v.H_kv) * w.d, dm), w.dtype, 1.0 / math.sqrt(dm))
    w_o = normal(seed, STREAM_WO, (dm, v.H_q * w.d), w.dtype, 1.0 / math.sqrt(v.H_q * w.d))
    return x, w_qkv, w_o
