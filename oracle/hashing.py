"""Hash-bucket sparse causal attention: bucket assignment, reordering by bucket, and attention.

TEST INFRASTRUCTURE ONLY (see the package header).

The SCFA review (nubint.ai, "proposed method" and Figure 3) describes dynamic sparsity from geometric
hashing in the style of Reformer's LSH, computed exactly: queries and keys are reordered by their hash
bucket, which turns causal attention inside buckets into a non-triangular causal mask that the kernel
handles as one range of keys per query.

Readings (the review gives no formulas):
  - Hash: with a random matrix R [d, nb/2] per head (nb even), bucket(x) = argmax over the nb values
    [x R, -x R], the first index on ties. Queries and keys of a head use the same R.
  - Attention: query i attends key j iff both have the same bucket and j <= i. A bucket value outside
    [0, nb) marks a dropped token, which attends and is attended by nothing (the review's query/key
    dropping, in the same encoding).
  - Reordering: queries and keys are each sorted stably by bucket, dropped tokens last. In that order
    the queries of bucket b occupy rows [qs_b, qe_b) in increasing position, so the rows that attend the
    key at sorted column c (original position p, bucket b) are the contiguous range [lo_c, qe_b) with
    lo_c = qs_b + (number of bucket-b queries at positions < p). Its mask in the column-wise encoding is
    UT = [0, lo_c), LT = [qe_b, N), no causal flag; a dropped key masks every row (UT = [0, N)). Empty
    spans are canonical (UT 0, 0; LT N, N).
"""
from __future__ import annotations

import numpy as np

from .attention import attend_rows


def lsh_buckets(x, R) -> np.ndarray:
    """int64 [N]: bucket of each row of x [N, d] under the rotation R [d, nb/2], in float64."""
    p = np.asarray(x, np.float64) @ np.asarray(R, np.float64)
    return np.argmax(np.concatenate([p, -p], axis=1), axis=1)


def lsh_scores(x, R) -> np.ndarray:
    """float64 [N, nb]: the values whose argmax is the bucket (for near-tie checks)."""
    p = np.asarray(x, np.float64) @ np.asarray(R, np.float64)
    return np.concatenate([p, -p], axis=1)


def _group(bk, nb):
    bk = np.asarray(bk, np.int64)
    return np.where((bk >= 0) & (bk < nb), bk, nb)


def hash_masked(qb, kb, nb: int) -> np.ndarray:
    """bool [N, N] in original order: True where query i does not attend key j."""
    gq, gk = _group(qb, nb), _group(kb, nb)
    N = len(gq)
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    attend = (gq[:, None] == gk[None, :]) & (gq[:, None] < nb) & (j <= i)
    return ~attend


def bucket_sort(qb, kb, nb: int):
    """One head: (qidx, qpos, kidx, kpos, lts, lte, uts, ute), all int64 [N].

    qidx[r] is the original query at sorted row r, qpos its inverse; likewise for keys; the four vectors
    are the mask of the sorted problem (run without the causal flag)."""
    gq, gk = _group(qb, nb), _group(kb, nb)
    N = len(gq)
    qidx = np.argsort(gq, kind="stable")
    kidx = np.argsort(gk, kind="stable")
    qpos = np.empty(N, np.int64)
    qpos[qidx] = np.arange(N)
    kpos = np.empty(N, np.int64)
    kpos[kidx] = np.arange(N)
    qs = np.searchsorted(gq[qidx], np.arange(nb + 1), side="left")   # first sorted row of each group
    qe = np.searchsorted(gq[qidx], np.arange(nb + 1), side="right")  # one past its last
    lts = np.full(N, N, np.int64)
    lte = np.full(N, N, np.int64)
    uts = np.zeros(N, np.int64)
    ute = np.zeros(N, np.int64)
    for c in range(N):
        p, b = int(kidx[c]), int(gk[kidx[c]])
        if b == nb:
            ute[c] = N
            continue
        rows_b = qidx[qs[b]:qe[b]]  # original positions of bucket b's queries, increasing
        lo = int(qs[b] + np.count_nonzero(rows_b < p))
        ute[c] = lo
        if qe[b] < N:
            lts[c] = int(qe[b])
    return qidx, qpos, kidx, kpos, lts, lte, uts, ute


def hash_attention_head(q, k, v, do, qb, kb, nb: int, scale: float):
    """Forward and backward of one head in original order: out [N, d], lse [N], dq, dk, dv."""
    q, k, v, do = (np.asarray(x, np.float64) for x in (q, k, v, do))
    masked = hash_masked(qb, kb, nb)
    res = attend_rows(q, k, v, do, masked, scale)
    dk = scale * (res["dS"].T @ q)
    dv = res["P"].T @ do
    return res["out"], res["lse"], res["dq"], dk, dv


def hash_attention(q, k, v, do, qb, kb, nb: int, scale: float):
    """All heads of [B, H, N, d] arrays with bucket ids qb, kb [B, H, N]."""
    B, H, N, d = q.shape
    out = np.zeros((B, H, N, d))
    lse = np.full((B, H, N), -np.inf)
    dq, dk, dv = np.zeros((B, H, N, d)), np.zeros((B, H, N, d)), np.zeros((B, H, N, d))
    for b in range(B):
        for h in range(H):
            out[b, h], lse[b, h], dq[b, h], dk[b, h], dv[b, h] = hash_attention_head(
                q[b, h], k[b, h], v[b, h], do[b, h], qb[b, h], kb[b, h], nb, scale)
    return out, lse, dq, dk, dv


def unmasked_count(qb, kb, nb: int) -> int:
    """Number of (query, key) pairs of one head that attend each other."""
    return int((~hash_masked(qb, kb, nb)).sum())


def _row_keys(gq, gk, nb, i):
    """Keys attended by query i: same group (not dropped) and position <= i."""
    if gq[i] >= nb:
        return np.zeros(0, np.int64)
    return np.flatnonzero((gk[:i + 1] == gq[i]))


def hash_rows_probe(q, k, v, do, qb, kb, nb: int, scale: float, rows):
    """out, lse, dq of selected query rows of one head (original order), each from its full row."""
    gq, gk = _group(qb, nb), _group(kb, nb)
    d = q.shape[1]
    outs, lses, dqs = [], [], []
    for i in np.asarray(rows, np.int64):
        keys = _row_keys(gq, gk, nb, int(i))
        if keys.size == 0:
            outs.append(np.zeros(d)); lses.append(-np.inf); dqs.append(np.zeros(d))
            continue
        res = attend_rows(q[i:i + 1], k[keys], v[keys], do[i:i + 1], np.zeros((1, keys.size), bool), scale)
        outs.append(res["out"][0]); lses.append(res["lse"][0]); dqs.append(res["dq"][0])
    return np.array(outs), np.array(lses), np.array(dqs)


def hash_cols_probe(q, k, v, do, qb, kb, nb: int, scale: float, cols):
    """dk, dv of selected key columns of one head: every query attending one of them is evaluated over
    its full row and its contributions to the selected columns are summed."""
    gq, gk = _group(qb, nb), _group(kb, nb)
    N, d = q.shape
    cols = np.asarray(cols, np.int64)
    dk, dv = np.zeros((cols.size, d)), np.zeros((cols.size, d))
    for n, j in enumerate(cols):
        if gk[j] >= nb:
            continue
        for i in np.flatnonzero(gq[j:] == gk[j]) + j:
            keys = _row_keys(gq, gk, nb, int(i))
            res = attend_rows(q[i:i + 1], k[keys], v[keys], do[i:i + 1], np.zeros((1, keys.size), bool), scale)
            t = int(np.searchsorted(keys, j))
            dk[n] += scale * res["dS"][0, t] * q[i]
            dv[n] += res["P"][0, t] * do[i]
    return dk, dv
