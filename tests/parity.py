"""Comparison of a GPU result against the fp64 oracle.

Bounds (bf16 inputs, fp32 accumulation): max |err| <= 2e-2 and mean |err| <=
2e-3 over all elements, plus two relative checks that a zero or partly
missing output cannot pass at long sequence lengths (where |o| is ~1e-3):
relative L2 error <= 1e-2 overall and <= 3e-2 for the worst (b, i, h) row.
fp32: max |err| <= 1e-4 and relative L2 <= 1e-5.

Derivation of the bf16 relative bounds: the output is rounded to bf16 (<= 2^-9
relative, ~1.1e-3 RMS), the probabilities are rounded to bf16 before the P.V
product (same order, averaging over the keys), and fp32 accumulation adds
~1e-5: about 2e-3 relative L2 expected, so 1e-2 leaves 5x headroom.
"""
import numpy as np

BOUNDS = {
    "bf16": dict(max_abs=2e-2, mean_abs=2e-3, rel_l2=1e-2, row_rel_l2=3e-2),
    "f32": dict(max_abs=1e-4, mean_abs=1e-4, rel_l2=1e-5, row_rel_l2=1e-4),
}


def error_stats(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    diff = got - ref
    ad = np.abs(diff)
    d = ref.shape[-1]
    row_err = np.sqrt((diff.reshape(-1, d) ** 2).sum(axis=1))
    row_ref = np.sqrt((ref.reshape(-1, d) ** 2).sum(axis=1))
    row_rel = row_err / np.maximum(row_ref, 1e-30)
    return dict(
        max_abs=float(ad.max()) if ad.size else 0.0,
        mean_abs=float(ad.mean()) if ad.size else 0.0,
        rel_l2=float(np.sqrt((diff ** 2).sum()) / max(np.sqrt((ref ** 2).sum()), 1e-30)),
        row_rel_l2=float(row_rel.max()) if row_rel.size else 0.0,
        nonfinite=int((~np.isfinite(got)).sum()),
    )


def check(got, ref, dtype, what=""):
    st = error_stats(got, ref)
    bounds = BOUNDS[dtype]
    bad = [k for k, lim in bounds.items() if not st[k] <= lim]
    if st["nonfinite"]:
        bad.append("nonfinite")
    assert not bad, f"{what}: parity failed on {bad}: {st} (bounds {bounds})"
    return st
