"""Pins of the oracle's longest-first unit order (CPU): a hand-derived document case, the closed forms of
the plain causal and the unmasked problem, exactness against the dense mask where the classification is
exact (tile-aligned documents), soundness for any mask, and the row-block coordinates."""
import numpy as np
import pytest

import workloads as W
from oracle import masks as OM
from oracle import schedule as OS


def _vecs(spec, b=0, h=0):
    return [None if x is None else x[b, h] for x in spec.vectors()]


def test_hand_derived_document_case():
    # N = 512, causal documents [0, 128) and [128, 512). Query units of 128 rows against 64-column key
    # tiles: unit 0 sees key tiles 0-1 (its own document, causal), unit 1 the tiles 2-3 of the second
    # document up to its last row, unit 2 the tiles 2-5, unit 3 the tiles 2-7. Key units of 128 columns
    # against 64-row query tiles: unit 0 (first document) is seen by row tiles 0-1, unit 1 by row tiles
    # 2-7, unit 2 by 4-7, unit 3 by 6-7.
    spec = W.encode_causal_document(np.array([0, 128, 512]), 512)
    qo, ko, qc, kc = OS.schedule_slice(*_vecs(spec), True, 512, 512)
    assert list(qc) == [2, 2, 4, 6]
    assert list(kc) == [2, 6, 4, 2]
    assert list(qo) == [3, 2, 1, 0]   # ties (units 0 and 1) keep the latest-first default order
    assert list(ko) == [1, 2, 0, 3]   # ties (units 0 and 3) keep the earliest-first default order


@pytest.mark.parametrize("N", [1, 64, 127, 128, 129, 300, 1000])
def test_closed_forms_causal_and_unmasked(N):
    nq, nk = -(-N // 128), -(-N // 128)
    n64 = -(-N // 64)
    qo, ko, qc, kc = OS.schedule_slice(None, None, None, None, True, N, N)
    # causal: a query unit ending at row r1 - 1 reaches the key tiles with first column <= r1 - 1
    want_q = [min(n64, (min(N, 128 * (qt + 1)) - 1) // 64 + 1) for qt in range(nq)]
    # a key unit starting at column c0 is reached by the row tiles whose last row is >= c0
    want_k = [n64 - (128 * kt) // 64 for kt in range(nk)]
    assert list(qc) == want_q and list(kc) == want_k
    assert list(qo) == list(range(nq - 1, -1, -1))
    assert list(ko) == list(range(nk))
    qo, ko, qc, kc = OS.schedule_slice(None, None, None, None, False, N, N)
    assert list(qc) == [n64] * nq and list(kc) == [n64] * nk
    assert list(qo) == list(range(nq - 1, -1, -1)) and list(ko) == list(range(nk))


def _dense_live(masked, Nq, Nk, rb, cb):
    """Tiles of rb rows x cb columns holding at least one unmasked entry, counted per row / column."""
    nr, nc = -(-Nq // rb), -(-Nk // cb)
    live = np.zeros((nr, nc), bool)
    for r in range(nr):
        for c in range(nc):
            live[r, c] = not masked[r * rb:(r + 1) * rb, c * cb:(c + 1) * cb].all()
    return live


def test_exact_on_tile_aligned_documents():
    # documents on 128-row boundaries: every tile is either inside one document's block or outside all
    # of them, so the classification is exact and the cost is the count of tiles with an unmasked entry
    N = 1024
    bounds = np.array([0, 128, 512, 640, 1024])
    for spec in (W.encode_causal_document(bounds, N), W.encode_bidirectional_document(bounds, N)):
        v = _vecs(spec)
        masked = OM.dense_masked(*v, spec.causal, N)
        _, _, qc, kc = OS.schedule_slice(*v, spec.causal, N, N)
        assert list(qc) == list(_dense_live(masked, N, N, 128, 64).sum(axis=1))
        assert list(kc) == list(_dense_live(masked, N, N, 64, 128).sum(axis=0))


def test_sound_for_any_mask():
    # a tile with an unmasked entry is never counted out; random vectors exercise every interval shape
    rng = np.random.default_rng(3)
    for N in (200, 333):
        for causal in (False, True):
            v = [rng.integers(-10, N + 10, size=N) for _ in range(4)]
            masked = OM.dense_masked(*v, causal, N)
            _, _, qc, kc = OS.schedule_slice(*v, causal, N, N)
            assert np.all(qc >= _dense_live(masked, N, N, 128, 64).sum(axis=1))
            assert np.all(kc >= _dense_live(masked, N, N, 64, 128).sum(axis=0))


def test_orders_are_longest_first_permutations():
    rng = np.random.default_rng(5)
    N = 2000
    bounds = W.loguniform_doc_boundaries(rng, N, 32, 600)
    spec = W.encode_causal_document(bounds, N)
    qo, ko, qc, kc = OS.schedule_slice(*_vecs(spec), True, N, N)
    for order, cost in ((qo, qc), (ko, kc)):
        assert sorted(order) == list(range(len(cost)))
        assert np.all(np.diff(cost[order]) <= 0)


def test_row_blocks_use_global_rows():
    # a block of rows [q_off, q_off + Nq) with q_off on a 128-row boundary: its query units are the
    # whole problem's units from q_off / 128 on, and summed over a 64-aligned partition of the rows the
    # key-unit costs give the whole problem's
    rng = np.random.default_rng(9)
    N = 1100
    bounds = W.loguniform_doc_boundaries(rng, N, 40, 500)
    for spec in (W.encode_causal_document(bounds, N), W.encode_prefix_lm(300, N)):
        v = _vecs(spec)
        _, _, qc, kc = OS.schedule_slice(*v, spec.causal, N, N)
        parts = [(0, 256), (256, 640), (640, N)]
        ksum = np.zeros_like(kc)
        for a, b in parts:
            _, _, qcp, kcp = OS.schedule_slice(*v, spec.causal, b - a, N, a)
            assert list(qcp) == list(qc[a // 128:a // 128 + len(qcp)])
            ksum += kcp
        assert list(ksum) == list(kc)


def test_batched_matches_slices():
    rng = np.random.default_rng(11)
    N, B, Hm = 300, 2, 2
    drops = [np.sort(rng.choice(N, size=80, replace=False)) for _ in range(Hm)]
    spec = W.encode_causal_key_drop(drops, N, B)
    qo, ko, qc, kc = OS.schedule(spec.vectors(), True, B, Hm, N, N)
    for b in range(B):
        for h in range(Hm):
            r = OS.schedule_slice(*_vecs(spec, b, h), True, N, N)
            for got, want in zip((qo[b, h], ko[b, h], qc[b, h], kc[b, h]), r):
                assert list(got) == list(want)
