"""Plan of the stored-dS backward, and the stored tiles' contents.

TEST INFRASTRUCTURE ONLY (see the package header).

The backward may keep every dS tile that its key-parallel pass forms, so that dQ = scale * dS K is a
product over stored tiles rather than a second pass recomputing S, dP and dS. The pages do not describe
the backward's work split; what is fixed here is the bookkeeping the library's plan call writes, read
from the same tile rule the attention kernels use (oracle.tiles.classify, rows in tiles of 64, keys in
tiles of 128, bounds merged over the 128 keys):

  per (b, hm, key tile kt): first[kt] = the first 64-row query tile that is not FULL for kt (0 if none),
                            span[kt]  = last - first + 1 over the tiles that are not FULL (0 if none),
                            base[kt]  = sum of span over the earlier key tiles of the same (b, hm);
  per (b, hm):              rowtotal  = sum of span;
  per (b, h), in order:     region    = sum of rowtotal[b', hm(h')] over the earlier heads;
  total                     = sum of rowtotal over all heads.

A stored tile holds dS for 64 query rows x 128 keys in bf16; the pair (query tile qt, key tile kt) of
head (b, h) sits in slot region + base[kt] + (qt - first[kt]). Inside a tile, key 32 kg + kl and query
rows 32 ib + 16 p + 8 h + 4 g + e (p, h, g in {0, 1}, e = 0..3) are at element
((kg * 4 + 2 ib + p) * 64 + w) * 8 + 4 h + e with w = 32 g + (kl XOR (8 g + 4 p)): the library's layout,
restated here to read its cache back.
"""
from __future__ import annotations

import numpy as np

from . import masks as OM
from . import tiles as OT

QT = 64    # query rows per stored tile
KT = 128   # keys per stored tile


def spans_slice(lts, lte, uts, ute, causal: bool, N: int):
    """(first, span) int64 [ceil(N/128)] for one (b, hm) slice of the vectors."""
    b128 = OT.tile_bounds_slice(lts, lte, uts, ute, N, KT)
    nq, nk = -(-N // QT), -(-N // KT)
    first = np.zeros(nk, np.int64)
    span = np.zeros(nk, np.int64)
    for kt in range(nk):
        c0, c1 = kt * KT, min(N, (kt + 1) * KT)
        live = [qt for qt in range(nq)
                if OT.classify(qt * QT, min(N, (qt + 1) * QT), c0, c1, b128[kt], causal) != OT.FULL]
        if live:
            first[kt] = live[0]
            span[kt] = live[-1] - live[0] + 1
    return first, span


def plan(vectors, causal: bool, B: int, H: int, Hm: int, N: int):
    """dict(first, base, rowtotal [B, Hm, ...], region [B, H], total) as defined in the module header."""
    lts, lte, uts, ute = vectors
    nk = -(-N // KT)
    first = np.zeros((B, Hm, nk), np.int64)
    base = np.zeros((B, Hm, nk), np.int64)
    rowtotal = np.zeros((B, Hm), np.int64)
    for b in range(B):
        for hm in range(Hm):
            sl = lambda x: None if x is None else x[b, hm]  # noqa: E731
            f, s = spans_slice(sl(lts), sl(lte), sl(uts), sl(ute), causal, N)
            first[b, hm] = f
            base[b, hm] = np.concatenate([[0], np.cumsum(s)[:-1]])
            rowtotal[b, hm] = int(s.sum())
    region = np.zeros((B, H), np.int64)
    run = 0
    for b in range(B):
        for h in range(H):
            region[b, h] = run
            run += int(rowtotal[b, h if Hm > 1 else 0])
    return {"first": first, "base": base, "rowtotal": rowtotal, "region": region, "total": run}


def dense_spans(lts, lte, uts, ute, causal: bool, N: int):
    """(first, span) from the dense mask: the query tiles holding at least one unmasked entry of each key
    tile. Equal to spans_slice wherever the tile rule is exact (e.g. tile-aligned documents)."""
    masked = OM.dense_masked_rows(lts, lte, uts, ute, causal, N, 0, N)
    nq, nk = -(-N // QT), -(-N // KT)
    first = np.zeros(nk, np.int64)
    span = np.zeros(nk, np.int64)
    for kt in range(nk):
        blk = masked[:, kt * KT:min(N, (kt + 1) * KT)]
        live = [qt for qt in range(nq) if not blk[qt * QT:min(N, (qt + 1) * QT)].all()]
        if live:
            first[kt] = live[0]
            span[kt] = live[-1] - live[0] + 1
    return first, span


def tile_values(ds_head: np.ndarray, qt: int, kt: int) -> np.ndarray:
    """The 8192 values of stored tile (qt, kt) in storage order, from a dense float [N, N] dS of one head
    (rows = queries, columns = keys; entries past N are zero)."""
    N = ds_head.shape[0]
    blk = np.zeros((QT, KT))
    r1, c1 = min(N, (qt + 1) * QT), min(N, (kt + 1) * KT)
    blk[:r1 - qt * QT, :c1 - kt * KT] = ds_head[qt * QT:r1, kt * KT:c1]
    out = np.zeros(QT * KT)
    for kg in range(4):
        for kl in range(32):
            key = 32 * kg + kl
            for ib in range(2):
                for p in range(2):
                    for g in range(2):
                        w = 32 * g + (kl ^ (8 * g + 4 * p))
                        for h in range(2):
                            at = ((kg * 4 + 2 * ib + p) * 64 + w) * 8 + 4 * h
                            for e in range(4):
                                out[at + e] = blk[32 * ib + 16 * p + 8 * h + 4 * g + e, key]
    return out
