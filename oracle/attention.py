"""Float64 softmax attention under a column-wise mask: forward, backward, brute force, probes.

TEST INFRASTRUCTURE ONLY (see the package header).

The method is exact tiled attention: skipping masked work loses no accuracy (FlashMask abstract,
papers.pytorch.kr 2410.01359), and the IO-aware tiling it extends is exact too (FlashAttention-3
abstract, fugumt.com 2407.08608; the FlashAttention README on wenyanet.com). So the oracle is the plain
definition, per (batch, head) with rows i and columns j:

  S_ij = scale * q_i . k_j, and S_ij = -inf where (i, j) is masked
  P_ij = exp(S_ij - m_i) / l_i,  m_i = max_j S_ij,  l_i = sum_j exp(S_ij - m_i)
  out_i = sum_j P_ij v_j,  lse_i = m_i + ln l_i
  dV = P^T dO,  dP = dO V^T,  D_i = sum_j P_ij dP_ij,  dS = P * (dP - D),
  dQ = scale * dS K,  dK = scale * dS^T Q

A row with every column masked has P = 0, out = 0, lse = -inf and no gradient contribution (the
convention chosen where the pages are silent). Rows are processed in blocks; inside a block only the
column span that holds an unmasked entry of the block's dense mask is multiplied. That skip is read
off the dense mask itself, not from any tile bounds.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .masks import dense_masked_rows


def attend_rows(q_rows, k, v, do_rows, masked, scale):
    """Rows of one head against a column span. q_rows, do_rows [r, d]; k, v [c, d]; masked bool [r, c].

    Returns dict(out, lse, P, D, dS, dq); D, dS, dq are None when do_rows is None."""
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    S = scale * (q_rows @ k.T)
    S = np.where(masked, -np.inf, S)
    alive = ~masked.all(axis=1)
    m = np.where(alive, S.max(axis=1, initial=-np.inf), 0.0)
    E = np.where(masked, 0.0, np.exp(S - m[:, None]))
    l = E.sum(axis=1)
    safe_l = np.where(alive, l, 1.0)
    P = np.where(alive[:, None], E / safe_l[:, None], 0.0)
    out = P @ v
    lse = np.where(alive, m + np.log(safe_l), -np.inf)
    res = {"out": out, "lse": lse, "P": P, "D": None, "dS": None, "dq": None}
    if do_rows is not None:
        do_rows = np.asarray(do_rows, dtype=np.float64)
        dP = do_rows @ v.T
        D = (P * dP).sum(axis=1)
        dS = P * (dP - D[:, None])
        res.update(D=D, dS=dS, dq=scale * (dS @ k))
    return res


def _row_block(N):
    return 256 if N <= 8192 else (128 if N <= 32768 else 64)


def fwd_bwd_head_rows(q, k, v, do, vecs, causal, scale, r0, r1, row_block=None):
    """Query rows [r0, r1) of one head (q, k, v, do [N, d] float64): out, lse, dq of those rows and their
    contributions to dk, dv over [c_lo, c_hi), the column span holding every key they attend.
    Returns (out, lse, dq, c_lo, dk_part, dv_part). Summed over a partition of the rows, the parts give
    the whole dk and dv."""
    N, d = q.shape
    rb = row_block or _row_block(N)
    out = np.zeros((r1 - r0, d))
    lse = np.full(r1 - r0, -np.inf)
    dq = np.zeros((r1 - r0, d))
    dk = np.zeros((N, d))
    dv = np.zeros((N, d))
    lo, hi = N, 0
    for a in range(r0, r1, rb):
        b = min(r1, a + rb)
        masked = dense_masked_rows(*vecs, causal, N, a, b)
        live_cols = np.flatnonzero(~masked.all(axis=0))
        if live_cols.size == 0:
            continue
        c0, c1 = int(live_cols[0]), int(live_cols[-1]) + 1
        res = attend_rows(q[a:b], k[c0:c1], v[c0:c1], do[a:b], masked[:, c0:c1], scale)
        out[a - r0:b - r0] = res["out"]
        lse[a - r0:b - r0] = res["lse"]
        dq[a - r0:b - r0] = res["dq"]
        dk[c0:c1] += scale * (res["dS"].T @ q[a:b])
        dv[c0:c1] += res["P"].T @ do[a:b]
        lo, hi = min(lo, c0), max(hi, c1)
    if hi <= lo:
        return out, lse, dq, 0, dk[:0], dv[:0]
    return out, lse, dq, lo, dk[lo:hi], dv[lo:hi]


def fwd_bwd_head(q, k, v, do, vecs, causal, scale, row_block=None):
    """Full forward and backward of one head. q, k, v, do [N, d]; vecs = (lts, lte, uts, ute) 1-D or None.

    Returns out [N, d], lse [N], dq, dk, dv [N, d] (float64)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    N, d = q.shape
    out, lse, dq, lo, dkp, dvp = fwd_bwd_head_rows(q, k, v, do, vecs, causal, scale, 0, N, row_block)
    dk = np.zeros((N, d))
    dv = np.zeros((N, d))
    dk[lo:lo + dkp.shape[0]] = dkp
    dv[lo:lo + dvp.shape[0]] = dvp
    return out, lse, dq, dk, dv


def fwd_bwd_head_parallel(q, k, v, do, vecs, causal, scale, pool, chunk_rows):
    """fwd_bwd_head with the rows split into chunks of chunk_rows run on a thread pool (NumPy releases the
    GIL inside its kernels; the caller limits BLAS to one thread per call). Same result up to the order
    of the float64 sums over row chunks."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    N, d = q.shape
    out = np.zeros((N, d))
    lse = np.full(N, -np.inf)
    dq = np.zeros((N, d))
    dk = np.zeros((N, d))
    dv = np.zeros((N, d))
    starts = list(range(0, N, chunk_rows))
    futs = {pool.submit(fwd_bwd_head_rows, q, k, v, do, vecs, causal, scale, a, min(N, a + chunk_rows)): a
            for a in starts}
    from concurrent.futures import as_completed
    for f in as_completed(futs):
        a = futs[f]
        o, l_, gq, lo, dkp, dvp = f.result()
        b = a + o.shape[0]
        out[a:b], lse[a:b], dq[a:b] = o, l_, gq
        dk[lo:lo + dkp.shape[0]] += dkp
        dv[lo:lo + dvp.shape[0]] += dvp
    return out, lse, dq, dk, dv


def fwd_bwd_rows_head(q_rows, k, v, do_rows, vecs, causal, scale, q_off, row_block=None):
    """Query rows q_off .. q_off + Nq - 1 of one head against all Nk keys, the mask read in the global row
    coordinates of the vectors (the unit of work of one rank under context parallelism, FlashMask-3
    summary, readmex.ai). q_rows, do_rows [Nq, d]; k, v [Nk, d]; vecs 1-D over the Nk columns or None.

    Returns out [Nq, d], lse [Nq], dq [Nq, d] of those rows and the contributions of those rows to
    dk, dv [Nk, d]."""
    q_rows = np.asarray(q_rows, dtype=np.float64)
    do_rows = np.asarray(do_rows, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Nq, d = q_rows.shape
    Nk = k.shape[0]
    rb = row_block or _row_block(max(Nq, Nk))
    out = np.zeros((Nq, d))
    lse = np.full(Nq, -np.inf)
    dq = np.zeros((Nq, d))
    dk = np.zeros((Nk, d))
    dv = np.zeros((Nk, d))
    for r0 in range(0, Nq, rb):
        r1 = min(Nq, r0 + rb)
        masked = dense_masked_rows(*vecs, causal, Nk, q_off + r0, q_off + r1)
        res = attend_rows(q_rows[r0:r1], k, v, do_rows[r0:r1], masked, scale)
        out[r0:r1], lse[r0:r1], dq[r0:r1] = res["out"], res["lse"], res["dq"]
        dk += scale * (res["dS"].T @ q_rows[r0:r1])
        dv += res["P"].T @ do_rows[r0:r1]
    return out, lse, dq, dk, dv


def fwd_bwd(q, k, v, do, vectors, causal, scale, Hm, heads=None, workers=None):
    """Forward and backward over [B, H, N, d] arrays; vectors are the four [B, Hm, N] arrays or None.

    heads: optional list of (b, h) to compute (others are left zero / -inf). Heads run on a thread
    pool (NumPy releases the GIL inside its kernels); BLAS is limited to one thread per call.
    Returns out, lse, dq, dk, dv and the number of worker threads used."""
    B, H, N, d = q.shape
    out = np.zeros((B, H, N, d))
    lse = np.full((B, H, N), -np.inf)
    dq = np.zeros((B, H, N, d))
    dk = np.zeros((B, H, N, d))
    dv = np.zeros((B, H, N, d))
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    workers = workers or min(len(todo), os.cpu_count() or 1)

    def run(bh):
        b, h = bh
        hm = h if Hm > 1 else 0
        vecs = tuple(None if x is None else x[b, hm] for x in vectors)
        return bh, fwd_bwd_head(q[b, h], k[b, h], v[b, h], do[b, h], vecs, causal, scale)

    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=1)
    except Exception:  # pragma: no cover - threadpoolctl is present in this image
        limiter = None
    try:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            for (b, h), (o, l_, gq, gk, gv) in ex.map(run, todo):
                out[b, h], lse[b, h], dq[b, h], dk[b, h], dv[b, h] = o, l_, gq, gk, gv
    finally:
        if limiter is not None:
            limiter.restore_original_limits()
    return out, lse, dq, dk, dv, workers


def _live_span(masked):
    live = np.flatnonzero(~masked.all(axis=0))
    if live.size == 0:
        return 0, 0
    return int(live[0]), int(live[-1]) + 1


def rows_probe(q, k, v, do, vecs, causal, scale, rows):
    """out, lse, D and dq of selected query rows of one head, each from its full row of scores
    (only the span of columns holding an unmasked entry is multiplied)."""
    N, d = k.shape
    rows = np.asarray(rows, dtype=np.int64)
    outs, lses, Ds, dqs = [], [], [], []
    for i in rows:
        masked = dense_masked_rows(*vecs, causal, N, int(i), int(i) + 1)
        c0, c1 = _live_span(masked)
        if c1 == c0:
            outs.append(np.zeros(d)); lses.append(-np.inf); Ds.append(0.0); dqs.append(np.zeros(d))
            continue
        res = attend_rows(q[i:i + 1], k[c0:c1], v[c0:c1], do[i:i + 1], masked[:, c0:c1], scale)
        outs.append(res["out"][0])
        lses.append(res["lse"][0])
        Ds.append(res["D"][0])
        dqs.append(res["dq"][0])
    return np.array(outs), np.array(lses), np.array(Ds), np.array(dqs)


def attending_rows(vecs, causal, N, cols):
    """Sorted query rows that attend at least one of the given key columns."""
    rows = np.zeros(N, dtype=bool)
    for j in np.asarray(cols, dtype=np.int64):
        rows |= ~dense_masked_rows(*vecs, causal, N, 0, N, int(j), int(j) + 1)[:, 0]
    return np.flatnonzero(rows)


def cols_probe(q, k, v, do, vecs, causal, scale, cols, row_block=64):
    """dk and dv of selected key columns of one head: every row that attends one of them is evaluated
    over its full row of scores, and its contributions to the selected columns are summed."""
    q = np.asarray(q, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    N, d = q.shape
    cols = np.asarray(cols, dtype=np.int64)
    rows = attending_rows(vecs, causal, N, cols)
    dk = np.zeros((cols.size, d))
    dv = np.zeros((cols.size, d))
    for s in range(0, rows.size, row_block):
        rr = rows[s:s + row_block]
        masked = np.concatenate([dense_masked_rows(*vecs, causal, N, int(i), int(i) + 1) for i in rr])
        c0, c1 = _live_span(masked)
        res = attend_rows(q[rr], k[c0:c1], v[c0:c1], do[rr], masked[:, c0:c1], scale)
        sel = (cols >= c0) & (cols < c1)
        local = cols[sel] - c0
        dk[sel] += scale * (res["dS"][:, local].T @ q[rr])
        dv[sel] += res["P"][:, local].T @ do[rr]
    return dk, dv


def brute_force_forward(q, k, v, masked, scale):
    """Forward by explicit loops and exactly rounded sums (math.fsum), for tiny cases only."""
    N, d = len(q), len(q[0])
    Nk = len(k)
    out = [[0.0] * d for _ in range(N)]
    lse = [-math.inf] * N
    for i in range(N):
        scores = {}
        for j in range(Nk):
            if not masked[i][j]:
                scores[j] = scale * math.fsum(float(q[i][t]) * float(k[j][t]) for t in range(d))
        if not scores:
            continue
        m = max(scores.values())
        e = {j: math.exp(s - m) for j, s in scores.items()}
        total = math.fsum(e.values())
        for t in range(d):
            out[i][t] = math.fsum(e[j] / total * float(v[j][t]) for j in e)
        lse[i] = m + math.log(total)
    return np.array(out), np.array(lse)


def loss_from_out(out, do):
    """The scalar whose gradient the backward pass computes: sum(out * dO)."""
    return float(np.sum(np.asarray(out) * np.asarray(do)))
