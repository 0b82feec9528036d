"""Per-key-tile bounds of the four boundary vectors and the tile classification rule.

TEST INFRASTRUCTURE ONLY (see the package header).

The method skips tiles the mask covers completely and leaves tiles it does not touch unmasked, using
the mask's sparsity to avoid work that cannot change the result (FlashMask abstract,
papers.pytorch.kr 2410.01359). The pages give no rule for deciding this; the rule written here is the
plainest one that the per-column interval representation supports: a tile is FULL when the causal
triangle or one interval covers every (row, column) of it, NONE when no source can reach any of its
rows, and PARTIAL otherwise.
"""
from __future__ import annotations

import numpy as np

NONE, PARTIAL, FULL = 0, 1, 2
KBLOCK = 64


def tile_bounds_slice(lts, lte, uts, ute, N: int, kblock: int = KBLOCK) -> np.ndarray:
    """int32 [ceil(N/kblock), 8]: per key tile, min/max over its valid columns of LTS, LTE, UTS, UTE.

    An absent pair takes the canonical empty values (N for LT, 0 for UT)."""
    nt = -(-N // kblock)
    out = np.zeros((nt, 8), dtype=np.int64)
    for t in range(nt):
        c0, c1 = t * kblock, min(N, (t + 1) * kblock)
        row = []
        for vec, empty in ((lts, N), (lte, N), (uts, 0), (ute, 0)):
            if vec is None:
                row += [empty, empty]
            else:
                seg = np.asarray(vec[c0:c1], dtype=np.int64)
                row += [int(seg.min()), int(seg.max())]
        out[t] = row
    return out.astype(np.int32)


def tile_bounds(vectors, B: int, Hm: int, N: int, kblock: int = KBLOCK) -> np.ndarray:
    """int32 [B, Hm, ceil(N/kblock), 8] for the four [B, Hm, N] vectors (None = absent)."""
    lts, lte, uts, ute = vectors
    nt = -(-N // kblock)
    out = np.zeros((B, Hm, nt, 8), dtype=np.int32)
    for b in range(B):
        for h in range(Hm):
            def pick(x):
                return None if x is None else x[b, h]
            out[b, h] = tile_bounds_slice(pick(lts), pick(lte), pick(uts), pick(ute), N, kblock)
    return out


def classify(r0: int, r1: int, c0: int, c1: int, bnd, causal: bool) -> int:
    """Class of the tile with rows [r0, r1) and columns [c0, c1) (already clipped to N).

    bnd = (minLTS, maxLTS, minLTE, maxLTE, minUTS, maxUTS, minUTE, maxUTE) over the tile's columns."""
    mn_lts, mx_lts, mn_lte, mx_lte, mn_uts, mx_uts, mn_ute, mx_ute = (int(x) for x in bnd)
    causal_full = causal and (r1 - 1 < c0)
    causal_none = (not causal) or (r0 >= c1 - 1)
    lt_full = (r0 >= mx_lts) and (r1 <= mn_lte)
    lt_none = (r1 <= mn_lts) or (r0 >= mx_lte)
    ut_full = (r0 >= mx_uts) and (r1 <= mn_ute)
    ut_none = (r1 <= mn_uts) or (r0 >= mx_ute)
    if causal_full or lt_full or ut_full:
        return FULL
    if causal_none and lt_none and ut_none:
        return NONE
    return PARTIAL


def tile_classes(bounds: np.ndarray, N: int, causal: bool, qblock: int, kblock: int = KBLOCK) -> np.ndarray:
    """uint8 [B, Hm, ceil(N/qblock), ceil(N/kblock)] classes from int32 bounds [B, Hm, nt, 8]."""
    B, Hm, nk, _ = bounds.shape
    nq = -(-N // qblock)
    out = np.zeros((B, Hm, nq, nk), dtype=np.uint8)
    for b in range(B):
        for h in range(Hm):
            for qt in range(nq):
                r0, r1 = qt * qblock, min(N, (qt + 1) * qblock)
                for kt in range(nk):
                    c0, c1 = kt * kblock, min(N, (kt + 1) * kblock)
                    out[b, h, qt, kt] = classify(r0, r1, c0, c1, bounds[b, h, kt], causal)
    return out
