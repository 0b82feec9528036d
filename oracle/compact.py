"""Key compaction of the column-wise mask: remove the key columns that are masked for every query row.

TEST INFRASTRUCTURE ONLY (see the package header).

Per-head key dropping reduces attention work in proportion to the keys kept (SCFA review, nubint.ai,
"proposed method"). Under the column-wise mask a dropped key is a column masked for every row; it adds
nothing to out, lse or dq and its dk, dv are zero, so the problem can be solved on the kept columns
alone.

Reading (the pages give no compacted format): the kept columns are listed in increasing order. The
compacted problem runs without the causal flag; a kept column j keeps its two spans clipped to [0, N]
and its causal rows [0, j) are merged into the UT span when that span is empty or starts at or before
j, else into the LT span under the same condition. A column needing three disjoint spans marks its
(b, hm) row as not compactable (count -1). Positions past the kept count are padding: LT = [0, N)
(every row masked), UT empty. Empty spans are written canonically (LT N, N; UT 0, 0).
"""
from __future__ import annotations

import numpy as np


def _clip(s, e, N):
    return np.clip(np.asarray(s, np.int64), 0, N), np.clip(np.asarray(e, np.int64), 0, N)


def kept_columns(lts, lte, uts, ute, causal: bool, N: int) -> np.ndarray:
    """bool [N]: column j has at least one unmasked query row in [0, N).

    The masked rows of a column are a union of at most three spans. If some row is unmasked, the
    smallest one is row 0 or the end of one of the spans, so it is enough to test those candidates."""
    j = np.arange(N, dtype=np.int64)
    zero = np.zeros(N, np.int64)
    spans = [(zero, j if causal else zero)]
    if lts is not None:
        spans.append(_clip(lts, lte, N))
    if uts is not None:
        spans.append(_clip(uts, ute, N))

    def inside(x):
        hit = np.zeros(N, bool)
        for s, e in spans:
            hit |= (s <= x) & (x < e)
        return hit

    kept = np.zeros(N, bool)
    for x in [zero] + [e for _, e in spans]:
        kept |= (x < N) & ~inside(x)
    return kept


def compact_keys_slice(lts, lte, uts, ute, causal: bool, N: int):
    """(kidx, kpos, count, lts2, lte2, uts2, ute2) for one (b, hm) slice of the vectors."""
    keep = kept_columns(lts, lte, uts, ute, causal, N)
    kidx = np.full(N, -1, np.int64)
    kpos = np.full(N, -1, np.int64)
    cols = np.nonzero(keep)[0]
    count = len(cols)
    kidx[:count] = cols
    kpos[cols] = np.arange(count)
    lts2 = np.zeros(N, np.int64)
    lte2 = np.full(N, N, np.int64)
    uts2 = np.zeros(N, np.int64)
    ute2 = np.zeros(N, np.int64)
    ok = True
    for r, col in enumerate(cols):
        ls, le = (N, N) if lts is None else (int(np.clip(lts[col], 0, N)), int(np.clip(lte[col], 0, N)))
        us, ue = (0, 0) if uts is None else (int(np.clip(uts[col], 0, N)), int(np.clip(ute[col], 0, N)))
        if causal and col > 0:
            if us >= ue:
                us, ue = 0, int(col)
            elif us <= col:
                us, ue = 0, max(int(col), ue)
            elif ls >= le:
                ls, le = 0, int(col)
            elif ls <= col:
                ls, le = 0, max(int(col), le)
            else:
                ok = False
        lts2[r], lte2[r] = (N, N) if ls >= le else (ls, le)
        uts2[r], ute2[r] = (0, 0) if us >= ue else (us, ue)
    return kidx, kpos, (count if ok else -1), lts2, lte2, uts2, ute2


def compact_keys(vectors, causal: bool, B: int, Hm: int, N: int):
    """All (b, hm) slices: kidx, kpos int [B, Hm, N], counts [B, Hm], and the four compacted vectors."""
    lts, lte, uts, ute = vectors
    kidx = np.zeros((B, Hm, N), np.int64)
    kpos = np.zeros((B, Hm, N), np.int64)
    counts = np.zeros((B, Hm), np.int64)
    out = [np.zeros((B, Hm, N), np.int64) for _ in range(4)]
    for b in range(B):
        for h in range(Hm):
            sl = lambda x: None if x is None else x[b, h]  # noqa: E731
            r = compact_keys_slice(sl(lts), sl(lte), sl(uts), sl(ute), causal, N)
            kidx[b, h], kpos[b, h], counts[b, h] = r[0], r[1], r[2]
            for k in range(4):
                out[k][b, h] = r[3 + k]
    return kidx, kpos, counts, out


def gather_rows(x, idx):
    """y[..., r, :] = x[..., idx[r], :], zero where idx < 0 (x one head's [N, d] rows)."""
    y = np.zeros_like(x)
    ok = idx >= 0
    y[ok] = x[idx[ok]]
    return y
