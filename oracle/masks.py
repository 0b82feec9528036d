"""Dense expansion of the column-wise mask, dense twins of the mask families, unmasked-pair count.

TEST INFRASTRUCTURE ONLY (see the package header).

Mask definition (FlashMask abstract, papers.pytorch.kr 2410.01359, and the FlashMask-3 summary on
readmex.ai, abstract body): each key column j stores query-axis interval boundaries. Read here as the
half-open intervals [LTS_j, LTE_j) and [UTS_j, UTE_j) of masked query rows; with the causal flag the
rows i < j are masked as well; the three sets combine by union. A pair given as None is empty, an
interval with start >= end is empty, and bounds outside [0, N) are clipped by the set definition.
"""
from __future__ import annotations

import numpy as np


def dense_masked_rows(lts, lte, uts, ute, causal: bool, N: int, r0: int, r1: int,
                      c0: int = 0, c1: int | None = None) -> np.ndarray:
    """bool [r1 - r0, c1 - c0]: True where query row i is masked for key column j.

    The four vectors are 1-D (one batch/head slice) or None."""
    if c1 is None:
        c1 = N
    i = np.arange(r0, r1, dtype=np.int64)[:, None]
    j = np.arange(c0, c1, dtype=np.int64)[None, :]
    m = np.zeros((r1 - r0, c1 - c0), dtype=bool)
    if causal:
        m |= i < j
    if lts is not None:
        s = np.asarray(lts, dtype=np.int64)[c0:c1][None, :]
        e = np.asarray(lte, dtype=np.int64)[c0:c1][None, :]
        m |= (s <= i) & (i < e)
    if uts is not None:
        s = np.asarray(uts, dtype=np.int64)[c0:c1][None, :]
        e = np.asarray(ute, dtype=np.int64)[c0:c1][None, :]
        m |= (s <= i) & (i < e)
    return m


def dense_masked(lts, lte, uts, ute, causal: bool, N: int) -> np.ndarray:
    """bool [N, N] mask of one (batch, head) slice."""
    return dense_masked_rows(lts, lte, uts, ute, causal, N, 0, N)


# ---------------------------------------------------------------- dense twins (plain definitions)
# Each twin returns allowed[i, j] (True = query i attends key j) from the family's own description,
# without going through the boundary vectors. The FlashMask-3 summary names document, prefix-LM,
# share-question, sliding-window and block-sparse masks; the SCFA review names per-head key dropping.

def _grid(N):
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    return i, j


def _segment_id(bounds, x):
    return np.searchsorted(np.asarray(bounds), x, side="right") - 1


def twin_full(N):
    return np.ones((N, N), dtype=bool)


def twin_causal(N):
    i, j = _grid(N)
    return j <= i


def twin_causal_document(bounds, N):
    i, j = _grid(N)
    return (_segment_id(bounds, i) == _segment_id(bounds, j)) & (j <= i)


def twin_causal_window(w, N):
    i, j = _grid(N)
    return (i - j >= 0) & (i - j < w)


def twin_causal_document_window(bounds, w, N):
    return twin_causal_document(bounds, N) & twin_causal_window(w, N)


def twin_prefix_lm(P, N):
    i, j = _grid(N)
    return (j < P) | (j <= i)


def twin_share_question(Q, answer_bounds, N):
    i, j = _grid(N)
    a = np.asarray(answer_bounds)
    same_answer = (_segment_id(a, i) == _segment_id(a, j)) & (i >= Q) & (j >= Q)
    return (j <= i) & ((j < Q) | same_answer)


def twin_causal_key_drop(dropped, N):
    i, j = _grid(N)
    kept = ~np.isin(np.arange(N), np.asarray(dropped))
    return (j <= i) & kept[None, :]


def twin_causal_document_block_sparse(bounds, kept_blocks, block, N):
    j = np.arange(N)
    kept = np.isin(j // block, np.asarray(kept_blocks))
    return twin_causal_document(bounds, N) & kept[None, :]


def twin_bidirectional_document(bounds, N):
    i, j = _grid(N)
    return _segment_id(bounds, i) == _segment_id(bounds, j)


# ---------------------------------------------------------------- unmasked pair count U

def _clip_interval(s, e, N):
    s = np.clip(np.asarray(s, dtype=np.int64), 0, N)
    e = np.clip(np.asarray(e, dtype=np.int64), 0, N)
    e = np.maximum(e, s)
    return s, e


def unmasked_count_slice(lts, lte, uts, ute, causal: bool, N: int) -> int:
    """Number of unmasked (i, j) pairs of one slice: per column, N minus the measure of the union of
    up to three row intervals (inclusion-exclusion over intervals, whose intersections are intervals)."""
    j = np.arange(N, dtype=np.int64)
    zero = np.zeros(N, dtype=np.int64)
    ivs = [(zero, j) if causal else (zero, zero)]
    ivs.append(_clip_interval(lts, lte, N) if lts is not None else (zero, zero))
    ivs.append(_clip_interval(uts, ute, N) if uts is not None else (zero, zero))

    def length(s, e):
        return np.maximum(e - s, 0)

    def meet(a, b):
        return np.maximum(a[0], b[0]), np.minimum(a[1], b[1])

    A, Bv, C = ivs
    union = (length(*A) + length(*Bv) + length(*C)
             - length(*meet(A, Bv)) - length(*meet(A, C)) - length(*meet(Bv, C))
             + length(*meet(meet(A, Bv), C)))
    return int(N * N - int(union.sum()))


def unmasked_count(spec_vectors, causal: bool, B: int, H: int, Hm: int, N: int) -> int:
    """U summed over all (b, h); spec_vectors are the four [B, Hm, N] arrays or None."""
    total = 0
    for b in range(B):
        for h in range(H):
            hm = h if Hm > 1 else 0
            vs = [None if x is None else x[b, hm] for x in spec_vectors]
            total += unmasked_count_slice(*vs, causal, N)
    return total
