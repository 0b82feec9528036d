"""Pins of the oracle's per-key-tile bounds and tile classes (CPU): brute force over columns,
soundness against the dense mask, and the exact special cases (no mask, plain causal)."""
import numpy as np
import pytest

import workloads as W
from oracle import masks as OM
from oracle import tiles as OT


def _specs(N, rng):
    cuts = W.uniform_cuts(rng, min(4, N - 1), 1, N - 1) if N > 1 else []
    bounds = W.doc_boundaries_from_cuts(cuts, N)
    drop = np.sort(rng.choice(N, size=N // 3, replace=False))
    nblk = -(-N // 128)
    kept = np.sort(rng.choice(nblk, size=max(1, nblk // 3), replace=False))
    return [
        W.encode_full(N), W.encode_causal(N), W.encode_causal_by_vectors(N),
        W.encode_causal_document(bounds, N), W.encode_causal_window(max(1, N // 5), N),
        W.encode_causal_document_window(bounds, max(1, N // 7), N), W.encode_prefix_lm(N // 2, N),
        W.encode_share_question(max(1, N // 4), np.array([max(1, N // 4), N]), N),
        W.encode_causal_key_drop([drop], N), W.encode_bidirectional_document(bounds, N),
        W.encode_causal_document_block_sparse(bounds, kept, 128, N),
    ]


def test_bounds_brute_force():
    rng = np.random.default_rng(0)
    for N in (1, 63, 64, 65, 200):
        vecs = [rng.integers(-5, N + 5, size=N) for _ in range(4)]
        b = OT.tile_bounds_slice(*vecs, N)
        assert b.shape == (-(-N // 64), 8)
        for t in range(b.shape[0]):
            cols = [j for j in range(N) if j // 64 == t]
            want = []
            for vec in vecs:
                want += [min(int(vec[j]) for j in cols), max(int(vec[j]) for j in cols)]
            assert list(b[t]) == want
    # absent pairs take the canonical empty values
    b = OT.tile_bounds_slice(None, None, None, None, 130)
    assert np.all(b[:, :4] == 130) and np.all(b[:, 4:] == 0)


@pytest.mark.parametrize("N", [64, 100, 256, 1000])
@pytest.mark.parametrize("qblock", [64, 128])
def test_classes_sound_against_dense_mask(N, qblock):
    rng = np.random.default_rng(N + qblock)
    for spec in _specs(N, rng):
        vecs = spec.column_slice(0, 0)
        bounds = OT.tile_bounds(spec.vectors(), 1, 1, N)
        cls = OT.tile_classes(bounds, N, spec.causal, qblock)[0, 0]
        m = OM.dense_masked(*vecs, spec.causal, N)
        for qt in range(cls.shape[0]):
            for kt in range(cls.shape[1]):
                blk = m[qt * qblock:(qt + 1) * qblock, kt * 64:(kt + 1) * 64]
                if cls[qt, kt] == OT.FULL:
                    assert blk.all(), (spec.family, qt, kt)
                elif cls[qt, kt] == OT.NONE:
                    assert not blk.any(), (spec.family, qt, kt)


@pytest.mark.parametrize("N", [64, 127, 512, 1000])
def test_classes_exact_special_cases(N):
    nq, nk = -(-N // 128), -(-N // 64)
    b = OT.tile_bounds((None,) * 4, 1, 1, N)
    assert np.all(OT.tile_classes(b, N, False, 128) == OT.NONE)
    cls = OT.tile_classes(b, N, True, 128)[0, 0]
    for qt in range(nq):
        r0, r1 = qt * 128, min(N, qt * 128 + 128)
        for kt in range(nk):
            c0, c1 = kt * 64, min(N, kt * 64 + 64)
            if r1 - 1 < c0:
                assert cls[qt, kt] == OT.FULL
            elif r0 >= c1 - 1:
                assert cls[qt, kt] == OT.NONE
            else:
                assert cls[qt, kt] == OT.PARTIAL
    # plain causal by flag and by vectors classify identically
    s = W.encode_causal_by_vectors(N)
    bv = OT.tile_bounds(s.vectors(), 1, 1, N)
    assert np.array_equal(OT.tile_classes(bv, N, False, 128), OT.tile_classes(b, N, True, 128))


def test_causal_exactness_against_dense():
    # for the causal triangle alone the rule is exact: FULL iff all masked, NONE iff none masked
    for N in (100, 384):
        m = OM.dense_masked(None, None, None, None, True, N)
        cls = OT.tile_classes(OT.tile_bounds((None,) * 4, 1, 1, N), N, True, 64)[0, 0]
        for qt in range(cls.shape[0]):
            for kt in range(cls.shape[1]):
                blk = m[qt * 64:(qt + 1) * 64, kt * 64:(kt + 1) * 64]
                assert (cls[qt, kt] == OT.FULL) == bool(blk.all())
                assert (cls[qt, kt] == OT.NONE) == bool(not blk.any())


@pytest.mark.parametrize("qblock", [64, 128])
@pytest.mark.parametrize("seed", range(4))
def test_classes_exact_for_tile_aligned_documents(qblock, seed):
    """With document boundaries on the tile grid the rule is exact in both directions, the interval
    branches included: FULL exactly where the dense block is all masked, NONE exactly where it has no
    masked entry (a NONE test that is too strict, e.g. one refusing a tile that ends on the interval's
    start row, classifies such blocks PARTIAL and fails here)."""
    rng = np.random.default_rng(100 + seed)
    N = 1024
    cuts = np.sort(rng.choice(np.arange(1, N // 128), size=int(rng.integers(1, 5)), replace=False)) * 128
    bounds = np.concatenate([[0], cuts, [N]])
    for spec in (W.encode_bidirectional_document(bounds, N), W.encode_causal_document(bounds, N)):
        m = OM.dense_masked(*spec.column_slice(0, 0), spec.causal, N)
        cls = OT.tile_classes(OT.tile_bounds(spec.vectors(), 1, 1, N), N, spec.causal, qblock)[0, 0]
        n_none = 0
        for qt in range(cls.shape[0]):
            for kt in range(cls.shape[1]):
                blk = m[qt * qblock:(qt + 1) * qblock, kt * 64:(kt + 1) * 64]
                assert (cls[qt, kt] == OT.FULL) == bool(blk.all()), (spec.family, qt, kt)
                assert (cls[qt, kt] == OT.NONE) == bool(not blk.any()), (spec.family, qt, kt)
                n_none += int(cls[qt, kt] == OT.NONE)
        assert n_none > 0


def test_exactness_pin_catches_a_too_strict_none_rule(monkeypatch):
    """Plant the slip the pin above is for (an interval NONE test using r1 < min start instead of
    r1 <= min start) in the oracle's rule and check that the exactness pin then fails."""
    real = OT.classify

    def too_strict(r0, r1, c0, c1, bnd, causal):
        c = real(r0, r1, c0, c1, bnd, causal)
        mn_lts = int(bnd[0])
        if c == OT.NONE and r1 == mn_lts:
            return OT.PARTIAL
        return c

    monkeypatch.setattr(OT, "classify", too_strict)
    with pytest.raises(AssertionError):
        for seed in range(4):
            test_classes_exact_for_tile_aligned_documents(128, seed)
