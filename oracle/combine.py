"""Log-sum-exp merge of split-KV partial results (oracle; test infrastructure only).

The HPC-Ops review ("How the kernels are organized around specific workload
shapes") says a combine kernel merges the split results without giving the rule.
The only merge that reproduces full softmax attention exactly is the
log-sum-exp weighting: with partial i holding o_i (softmax-normalised over its own
keys) and lse_i = ln sum over its keys of exp(s):

  M   = max_i lse_i
  w_i = exp(lse_i - M)
  o   = sum_i w_i o_i / sum_i w_i
  lse = M + ln sum_i w_i

A partial with lse_i = -inf (no visible key) gets weight 0.
"""

import numpy as np


def lse_merge(o_parts, lse_parts):
    """Merge partials along axis 0.

    o_parts: float [n, ..., D]; lse_parts: float [n, ...]. Returns (o, lse) in
    float64. If every partial of a row is empty the row is o = 0, lse = -inf."""
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    M = lse_parts.max(axis=0)
    finite = np.isfinite(M)
    Ms = np.where(finite, M, 0.0)
    w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - Ms), 0.0)
    den = w.sum(axis=0)
    num = (w[..., None] * o_parts).sum(axis=0)
    o = np.where(finite[..., None], num / np.where(den > 0, den, 1.0)[..., None], 0.0)
    lse = np.where(finite, Ms + np.log(np.where(den > 0, den, 1.0)), -np.inf)
    return o, lse
