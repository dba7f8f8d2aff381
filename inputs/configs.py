"""Workload recipes: the five attention shapes the method is measured on.

Shapes follow the Sparse Query Attention abstract's setting (long sequences
of 32k-200k tokens, compute-bound full-sequence passes) plus a tiny fp32 case
and a 4k head-configuration sweep.  Inputs are synthetic: i.i.d. normals from
the seeded generator, scaled by 0.5 and rounded to bf16 for the bf16 cases.
The 200k case also multiplies 1% of the key positions by 8 so that some
softmax rows are sharply peaked.

Seeds: 0x5A510000 + 16 * config_number + variant_index.
Streams: q = 0, k = 1, v = 2, key-position selection = 3.
"""
import math
from dataclasses import dataclass, field

import numpy as np

from . import normal, scale_positions_bf16, select_positions

SEED_BASE = 0x5A510000
STREAM_Q, STREAM_K, STREAM_V, STREAM_SEL = 0, 1, 2, 3


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

