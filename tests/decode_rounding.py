"""A float32 model of how the decode kernel rounds one query row that sees a few keys,
used to pick adversarial test inputs (test infrastructure; it is neither the oracle
nor the HIP path and imports neither).

The rows at risk are the ones whose softmax weights are dominated by one or two keys
(a short request, the first draft rows): there the bf16 rounding of each weight
(relative 2^-9) does not average out. The model follows the arithmetic the kernel
applies to such a row when all its keys lie in one 32-token chunk of one wave (every
request shorter than 33 tokens):
- scores in log2 units s_j = (q . k_j) * (scale * log2 e) in float32;
- p_j = 2^(s_j - max s) in float32;
- P.V sees bf16(p_j), plus bf16(p_j - bf16(p_j)) when the chunk takes the low part
  (bf16 KV), or fp16(p_j) (FP8 KV, whose V is converted to fp16);
- the output is (sum of used weight x v_j) / (sum of used weights), in float32, then
  rounded to bf16 (nearest even).
Summation order inside the matrix core is not modelled (fp32 accumulation of a few
terms moves the result by ~1e-7, far below the bf16 effects searched for).

`search_rows` scans rows of two to four keys (q = e_0, k_0 = 0, k_j = a_j e_0 with
a_j bf16, bf16 values) for the largest error against the exact softmax with and
without the low part, and returns the inputs of the worst cases.
"""

import numpy as np

LOG2E = 1.4426950408889634


def bf16_round(x):
    """float32 -> nearest bf16 value (ties to even), as float32."""
    x = np.asarray(x, np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = (u >> np.uint64(16)) & np.uint64(1)
    u = ((u + np.uint64(0x7FFF) + r) >> np.uint64(16)) << np.uint64(16)
    return u.astype(np.uint32).view(np.float32)


def model_row(s2, v, low, p_format="bf16"):
    """Output (bf16-rounded, float64) of one row with log2-unit scores s2 [..., k]
    (float32) and values v [..., k] (float32), with P rounded to bf16 (with or without
    the low part) or to fp16 (the FP8-KV path, p_format="f16")."""
    s2 = np.asarray(s2, np.float32)
    m = s2.max(axis=-1, keepdims=True)
    p = np.exp2((s2 - m).astype(np.float64)).astype(np.float32)
    if p_format == "f16":
        w = p.astype(np.float16).astype(np.float32)
    else:
        ph = bf16_round(p)
        w = ph + bf16_round((p - ph).astype(np.float32)) if low else ph
    num = np.sum((w.astype(np.float64) * v), axis=-1).astype(np.float32)
    den = np.sum(w.astype(np.float64), axis=-1).astype(np.float32)
    return bf16_round((num / den).astype(np.float32)).astype(np.float64)


def exact_row(s2, v):
    """The softmax-weighted mean in float64 of the same scores (log2 units) and values."""
    s2 = np.asarray(s2, np.float64)
    p = np.exp2(s2 - s2.max(axis=-1, keepdims=True))
    return np.sum(p * v, axis=-1) / np.sum(p, axis=-1)


def tolerance(ref, tol=1e-2):
    """The test tolerance: max(tol, 0.6 bf16 ulp of the reference)."""
    _, e = np.frexp(np.maximum(np.abs(ref), 2.0 ** -126))
    return np.maximum(tol, 0.6 * np.ldexp(1.0, e - 8))


def search_rows(scale, keys=2, n_rows=64, seed=0, a_range=(-4.0, 4.0), v_range=(-6.0, 6.0),
                samples=400_000):
    """Rows of `keys` keys: q = e_0 (bf16 1.0), key 0 = 0, key j = a_j e_0 (j >= 1),
    values v_j; a_j and v_j uniform in their ranges, rounded to bf16 (`samples`
    random rows).

    Keeps the n_rows rows with the largest excess of |model - exact| over the
    tolerance for the arithmetic without the low part. Returns dict(a float32
    [n_rows, keys] (a[:, 0] = 0), v float32 [n_rows, keys], ref (exact outputs), err_plain, err_low,
    excess_plain, excess_low float64 [n_rows]; max_excess_low_all, max_err_low_all,
    max_excess_plain_all, max_excess_f16_all, max_err_f16_all over every sample)."""
    rng = np.random.default_rng(seed)
    a = bf16_round(rng.uniform(*a_range, size=(samples, keys)).astype(np.float32))
    a[:, 0] = 0.0
    v = bf16_round(rng.uniform(*v_range, size=(samples, keys)).astype(np.float32))
    c = np.float32(np.float32(scale) * np.float32(LOG2E))
    s2 = (a * c).astype(np.float32)
    vd = v.astype(np.float64)
    ref = exact_row(s2, vd)
    tol = tolerance(ref)
    err_plain = np.abs(model_row(s2, vd, low=False) - ref)
    err_low = np.abs(model_row(s2, vd, low=True) - ref)
    err_f16 = np.abs(model_row(s2, vd, low=False, p_format="f16") - ref)
    order = np.argsort(-(err_plain - tol))[:n_rows]
    return dict(a=a[order], v=v[order], ref=ref[order], err_plain=err_plain[order], err_low=err_low[order],
                excess_plain=(err_plain - tol)[order], excess_low=(err_low - tol)[order],
                max_excess_low_all=float(np.max(err_low - tol)), max_err_low_all=float(np.max(err_low)),
                max_excess_plain_all=float(np.max(err_plain - tol)),
                max_excess_f16_all=float(np.max(err_f16 - tol)), max_err_f16_all=float(np.max(err_f16)))
