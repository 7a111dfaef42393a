"""Oracle sampler: temperature, top-k filter, softmax, inverse-CDF draw
(TEST INFRASTRUCTURE ONLY).

Follows ``generate()`` on the serving page "原生 nanoGPT 模型服务首选",
section 2: take the last-position logits, divide by the temperature, keep
only values not below the k-th largest (k = min(top_k, vocab)), softmax,
draw one id from the resulting distribution.

``torch.multinomial``'s internal algorithm is not given on the pages, so the
draw is the plain inverse-CDF reading, with the caller's uniform u in [0, 1)
replacing the library's random number:

1. s_i = float32(logit_i / T) (correctly rounded float32 division).
2. With top_k > 0: k' = min(top_k, V); v = the k'-th largest s counting
   repeats; the kept set K = {i : s_i >= v} (the page replaces values
   strictly below v by -inf, so ties with v survive).  Otherwise K = all.
3. m = max over K; w_i = exp(float64(s_i) - m); S = sum of w over K in
   ascending id order.
4. The draw is the smallest i in K (ascending ids) whose running sum c_i
   exceeds u * S; if rounding leaves none, the largest id in K.
5. Greedy mode (the limit of the temperature going to 0): the argmax of the
   logits, lowest id among equal maxima.

The running-sum comparison is done in float64; two correct implementations
can differ there only when u * S is within a few ulps of some c_i, so every
draw also reports its margin min_i |c_i - u S| / S.
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def topk_keep_set(s: np.ndarray, top_k: int) -> np.ndarray:
    """Boolean mask of the kept ids for one row of scaled logits ``s``."""
    V = s.shape[0]
    if top_k <= 0:
        return np.ones(V, dtype=bool)
    kp = min(top_k, V)
    v = np.sort(s)[::-1][kp - 1]
    return s >= v


def sample_row(logits: np.ndarray, u: float, temperature: float,
               top_k: int, greedy: bool):
    """Draw one id from one row of float32 logits.

    Returns (id, kept_mask or None, margin).  In greedy mode the mask is None
    and the margin is the gap between the top value and the next distinct
    value (0 when the maximum is tied).
    """
    lg = np.asarray(logits, dtype=np.float32)
    if greedy:
        i = int(np.argmax(lg))
        others = lg[lg < lg[i]]
        gap = float(lg[i] - others.max()) if others.size else float("inf")
        return i, None, gap
    s = lg / np.float32(temperature)          # float32 / float32, RNE
    keep = topk_keep_set(s, top_k)
    ids = np.nonzero(keep)[0]                 # ascending ids
    sk = s[ids].astype(np.float64)
    m = sk.max()
    w = np.exp(sk - m)
    c = np.cumsum(w)                          # sequential, ascending order
    S = c[-1]
    thr = u * S
    hit = np.nonzero(c > thr)[0]
    j = int(hit[0]) if hit.size else len(ids) - 1
    margin = float(np.min(np.abs(c - thr)) / S)
    return int(ids[j]), keep, margin


def sample_rows(logits: np.ndarray, uniforms: Optional[np.ndarray],
                temperature: float, top_k: int, greedy: bool):
    """Row-wise ``sample_row`` over [B, V] logits; returns (ids [B] int32,
    list of kept masks, margins [B])."""
    B = logits.shape[0]
    ids = np.empty(B, dtype=np.int32)
    masks, margins = [], np.empty(B)
    for b in range(B):
        u = 0.0 if uniforms is None else float(uniforms[b])
        ids[b], m, margins[b] = sample_row(logits[b], u, temperature, top_k,
                                           greedy)
        masks.append(m)
    return ids, masks, margins
