"""Softmax attention of one query over an explicit set of cached rows, float64.

Definition followed: scores s_j = scale * <q, k_j> with scale = 1/sqrt(d) by
default, weights a_j = exp(s_j) / sum_m exp(s_m) (which sum to one), output
o = sum_j a_j v_j ([sink] attention-weight formula and its normalisation;
[kvc] §2.2 scaled dot-product attention).  The max is subtracted before
exponentiating, as the [ring] demo does (§4.3); that changes no value.
The log-sum-exp lse = ln sum_j exp(s_j) is returned beside o (natural log).

An empty set gives o = 0 and lse = -inf (a reading: the pages never reach it).

Grouped-query attention: q head h reads kv head h // g with g = Hq / Hkv
([share] §2.2 and §4.1, several query heads share one K/V head; the
consecutive grouping is a reading).

Pins (tests/test_oracle_attention.py): torch's float64 CPU
scaled_dot_product_attention, a pure-Python double loop on tiny shapes,
V = 1 gives output 1, K = 0 gives the mean of V, masked full history equals
the windowed set, scipy's logsumexp.
"""

from __future__ import annotations

import math

import numpy as np


def attend(q, K, V, scale: float | None = None):
    """q [d], K [n, d], V [n, dv] -> (o [dv], lse) in float64."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    if K.shape[0] == 0:
        return np.zeros(V.shape[-1], dtype=np.float64), -math.inf
    s = scale * (K @ q)
    m = s.max()
    e = np.exp(s - m)
    z = e.sum()
    return (e / z) @ V, float(m + math.log(z))


def attend_masked(q, K, V, keep, scale: float | None = None):
    """Attention over all rows with -inf scores where keep is False."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    keep = np.asarray(keep, dtype=bool)
    if not keep.any():
        return np.zeros(V.shape[-1], dtype=np.float64), -math.inf
    s = np.where(keep, scale * (K @ q), -np.inf)
    m = s.max()
    e = np.exp(s - m)
    z = e.sum()
    return (e / z) @ V, float(m + math.log(z))


def attend_loops(q, K, V, scale: float | None = None):
    """Same as `attend`, one scalar at a time (small inputs only)."""
    d = len(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    n = len(K)
    if n == 0:
        return [0.0] * len(V[0]) if len(V) else [], -math.inf
    scores = []
    for j in range(n):
        acc = 0.0
        for i in range(d):
            acc += float(q[i]) * float(K[j][i])
        scores.append(scale * acc)
    m = max(scores)
    w = [math.exp(s - m) for s in scores]
    z = sum(w)
    out = [0.0] * len(V[0])
    for j in range(n):
        for i in range(len(V[0])):
            out[i] += (w[j] / z) * float(V[j][i])
    return out, m + math.log(z)


def attend_heads(q, K, V, scale: float | None = None):
    """GQA over one sequence: q [Hq, d], K/V [n, Hkv, d] -> (o [Hq, d], lse [Hq])."""
    q = np.asarray(q, dtype=np.float64)
    hq, hkv = q.shape[0], K.shape[1]
    if hq % hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    g = hq // hkv
    out = np.empty((hq, V.shape[-1]), dtype=np.float64)
    lse = np.empty(hq, dtype=np.float64)
    for h in range(hq):
        out[h], lse[h] = attend(q[h], K[:, h // g, :], V[:, h // g, :], scale)
    return out, lse
