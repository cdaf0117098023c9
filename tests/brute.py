"""Brute-force NumPy checks that pin the oracle to something other than itself.

None of these helpers sorts or chunks the way the oracle does; each computes
a quantity the method must reproduce from a plain definition:

* ``dense_same_bucket``: with one chunk spanning the whole sequence, LSH
  attention is dense softmax attention restricted to pairs that share a
  bucket (plus the causal and self rules);
* ``multiset_closed_form``: combining the rounds with logsumexp weights is the
  same as one softmax over the multiset of (round, key) hits, so
  out_i = sum_j c_ij e^{s_ij} v_j / sum_j c_ij e^{s_ij} with c_ij the number of
  rounds in which j is a valid key of i; windows are found by enumerating
  positions in (bucket, position) order with ``numpy.argsort(kind="stable")``;
* ``angular_buckets`` and ``multiset_closed_form_qk``: the same closed form
  with separate queries and keys, buckets taken by ``numpy.argmax`` (first
  index) over [x R, -x R], each side's windows enumerated from its own stable
  argsort; a query with no hit in any round gets a zero row.
"""
from __future__ import annotations

import numpy as np

SELF_PENALTY = 1.0e5


def scores(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, np.float64)
    d = x.shape[1]
    s = (x @ x.T) / np.sqrt(d)
    s[np.diag_indices_from(s)] -= SELF_PENALTY
    return s


def dense_same_bucket(x, v, bucket, causal: bool) -> np.ndarray:
    """Dense softmax attention over keys in the query's bucket (one round)."""
    x = np.asarray(x, np.float64)
    v = np.asarray(v, np.float64)
    bucket = np.asarray(bucket)
    L = x.shape[0]
    s = scores(x)
    allowed = bucket[:, None] == bucket[None, :]
    if causal:
        allowed &= np.arange(L)[None, :] <= np.arange(L)[:, None]
    s = np.where(allowed, s, -np.inf)
    s -= s.max(axis=1, keepdims=True)
    w = np.exp(s)
    w /= w.sum(axis=1, keepdims=True)
    return w @ v


def multiplicity(buckets, chunk_len: int, causal: bool) -> np.ndarray:
    """c[i, j] = number of rounds in which key j is valid for query i."""
    buckets = np.asarray(buckets)
    nh, L = buckets.shape
    c = np.zeros((L, L), np.int64)
    for r in range(nh):
        order = np.argsort(buckets[r], kind="stable")
        chunk_of_pos = np.empty(L, np.int64)
        chunk_of_pos[order] = np.arange(L) // chunk_len
        for i in range(L):
            for j in range(L):
                if buckets[r, i] != buckets[r, j]:
                    continue
                if causal and j > i:
                    continue
                if chunk_of_pos[j] in (chunk_of_pos[i], chunk_of_pos[i] - 1):
                    c[i, j] += 1
    return c


def multiset_closed_form(x, v, buckets, chunk_len: int, causal: bool) -> np.ndarray:
    x = np.asarray(x, np.float64)
    v = np.asarray(v, np.float64)
    c = multiplicity(buckets, chunk_len, causal)
    s = scores(x)
    s = np.where(c > 0, s, -np.inf)
    s -= s.max(axis=1, keepdims=True)
    w = c * np.exp(s)
    w /= w.sum(axis=1, keepdims=True)
    return w @ v


def attention_weights(x, buckets, chunk_len: int, causal: bool) -> np.ndarray:
    """The combined attention weights of the closed form (rows sum to 1)."""
    x = np.asarray(x, np.float64)
    c = multiplicity(buckets, chunk_len, causal)
    s = scores(x)
    s = np.where(c > 0, s, -np.inf)
    s -= s.max(axis=1, keepdims=True)
    w = c * np.exp(s)
    return w / w.sum(axis=1, keepdims=True)


def angular_buckets(x, R) -> np.ndarray:
    """[nh, L] first index of the maximum of [x R_r, -x R_r] (numpy.argmax
    returns the first maximal index)."""
    x = np.asarray(x, np.float64)
    out = []
    for Rr in np.asarray(R, np.float64):
        p = x @ Rr
        out.append(np.argmax(np.concatenate([p, -p], axis=1), axis=1))
    return np.array(out, np.int64)


def multiplicity_qk(bq, bk, chunk_len: int, causal: bool) -> np.ndarray:
    """c[i, j] = number of rounds in which key j counts for query i when
    queries and keys are sorted separately (query chunk c sees key chunks c-1
    and c)."""
    bq = np.asarray(bq)
    bk = np.asarray(bk)
    nh, L = bq.shape
    c = np.zeros((L, L), np.int64)
    for r in range(nh):
        qchunk = np.empty(L, np.int64)
        qchunk[np.argsort(bq[r], kind="stable")] = np.arange(L) // chunk_len
        kchunk = np.empty(L, np.int64)
        kchunk[np.argsort(bk[r], kind="stable")] = np.arange(L) // chunk_len
        for i in range(L):
            for j in range(L):
                if bk[r, j] != bq[r, i] or (causal and j > i):
                    continue
                if kchunk[j] in (qchunk[i], qchunk[i] - 1):
                    c[i, j] += 1
    return c


def multiset_closed_form_qk(q, k, v, bq, bk, chunk_len: int, causal: bool) -> np.ndarray:
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    c = multiplicity_qk(bq, bk, chunk_len, causal)
    s = (q @ k.T) / np.sqrt(q.shape[1])
    out = np.zeros((q.shape[0], v.shape[1]))
    for i in range(q.shape[0]):
        hit = c[i] > 0
        if not hit.any():
            continue
        si = s[i, hit] - s[i, hit].max()
        w = c[i, hit] * np.exp(si)
        out[i] = (w / w.sum()) @ v[hit]
    return out
