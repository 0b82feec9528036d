"""Longest-first order of the attention work units, from the tile classification.

TEST INFRASTRUCTURE ONLY (see the package header).

Under a sparse mask the work units of one launch (a block of query rows against its live key tiles,
or a block of key columns against its live query tiles) carry very different amounts of work, and a
fixed dispatch order leaves a tail of long units running alone at the end (the load-balancing problem
the FlashMask-3 summary, readmex.ai, raises for masked attention under parallel execution; its
balancer spreads sparsity-dependent work over workers). On one device the workers are the hardware
slots that take workgroups in launch order, so the classic longest-processing-time-first list rule
applies: dispatch units in decreasing order of work.

Reading (the pages give no single-device scheduler): the work of a unit is the number of tiles on its
row or column of the tile grid that the classification rule does not mark FULL (fully masked), with
  - query units of 128 rows against key tiles of 64 columns (forward and dq),
  - key units of 128 columns against query tiles of 64 rows (dk, dv),
the rows taken in the mask's global coordinates (local row + q_off). Units of equal work keep the
order in which they are dispatched without a schedule: latest query unit first, earliest key unit
first. Orders are per (b, hm) row of the mask.
"""
from __future__ import annotations

import numpy as np

from . import tiles as OT

QUNIT = 128  # query rows per query unit
KUNIT = 128  # key columns per key unit
QSUB = 64    # query rows per tile of a key unit
KSUB = 64    # key columns per tile of a query unit


def query_unit_work(b64, causal: bool, Nq: int, Nk: int, q_off: int, qt: int) -> int:
    """Key tiles of 64 columns (bounds b64 [ceil(Nk/64), 8]) not FULL for query unit qt."""
    r0, r1 = q_off + qt * QUNIT, q_off + min(Nq, (qt + 1) * QUNIT)
    n = 0
    for kt in range(b64.shape[0]):
        c0, c1 = kt * KSUB, min(Nk, (kt + 1) * KSUB)
        n += OT.classify(r0, r1, c0, c1, b64[kt], causal) != OT.FULL
    return n


def key_unit_work(b128, causal: bool, Nq: int, Nk: int, q_off: int, kt: int) -> int:
    """Query tiles of 64 rows not FULL for key unit kt (bounds b128 [ceil(Nk/128), 8] over 128 columns)."""
    c0, c1 = kt * KUNIT, min(Nk, (kt + 1) * KUNIT)
    n = 0
    for qt in range(-(-Nq // QSUB)):
        r0, r1 = q_off + qt * QSUB, q_off + min(Nq, (qt + 1) * QSUB)
        n += OT.classify(r0, r1, c0, c1, b128[kt], causal) != OT.FULL
    return n


def unit_bounds(lts, lte, uts, ute, Nk: int):
    """(b64, b128): per-tile min/max of the vectors over 64 and over 128 key columns."""
    return (OT.tile_bounds_slice(lts, lte, uts, ute, Nk, KSUB), OT.tile_bounds_slice(lts, lte, uts, ute, Nk, KUNIT))


def unit_costs_slice(lts, lte, uts, ute, causal: bool, Nq: int, Nk: int, q_off: int = 0):
    """(qcost [ceil(Nq/128)], kcost [ceil(Nk/128)]) for one (b, hm) slice of the [Nk] vectors."""
    b64, b128 = unit_bounds(lts, lte, uts, ute, Nk)
    qcost = np.array([query_unit_work(b64, causal, Nq, Nk, q_off, qt) for qt in range(-(-Nq // QUNIT))], np.int64)
    kcost = np.array([key_unit_work(b128, causal, Nq, Nk, q_off, kt) for kt in range(-(-Nk // KUNIT))], np.int64)
    return qcost, kcost


def longest_first(cost, default_order) -> np.ndarray:
    """Units sorted by decreasing cost; equal costs keep their place in default_order."""
    default_order = np.asarray(default_order, np.int64)
    c = np.asarray(cost, np.int64)[default_order]
    return default_order[np.argsort(-c, kind="stable")]


def schedule_slice(lts, lte, uts, ute, causal: bool, Nq: int, Nk: int, q_off: int = 0):
    """(qorder, korder, qcost, kcost) for one (b, hm) slice."""
    qcost, kcost = unit_costs_slice(lts, lte, uts, ute, causal, Nq, Nk, q_off)
    qorder = longest_first(qcost, np.arange(len(qcost))[::-1])
    korder = longest_first(kcost, np.arange(len(kcost)))
    return qorder, korder, qcost, kcost


def schedule(vectors, causal: bool, B: int, Hm: int, Nq: int, Nk: int, q_off: int = 0):
    """All (b, hm) slices of [B, Hm, Nk] vectors: qorder, qcost [B, Hm, nq]; korder, kcost [B, Hm, nk]."""
    lts, lte, uts, ute = vectors
    nq, nk = -(-Nq // QUNIT), -(-Nk // KUNIT)
    qo = np.zeros((B, Hm, nq), np.int64)
    ko = np.zeros((B, Hm, nk), np.int64)
    qc = np.zeros((B, Hm, nq), np.int64)
    kc = np.zeros((B, Hm, nk), np.int64)
    for b in range(B):
        for h in range(Hm):
            sl = lambda x: None if x is None else x[b, h]  # noqa: E731
            qo[b, h], ko[b, h], qc[b, h], kc[b, h] = schedule_slice(sl(lts), sl(lte), sl(uts), sl(ute), causal,
                                                                    Nq, Nk, q_off)
    return qo, ko, qc, kc
