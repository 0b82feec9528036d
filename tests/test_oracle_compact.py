"""Pins of the oracle's key compaction (CPU): kept columns against the dense mask, the compacted mask
against the original one column by column, and the attention results of the compacted problem against
those of the original one (SCFA review, nubint.ai, "proposed method": per-head key dropping with work
in proportion to the keys kept)."""
import math

import numpy as np
import pytest

import workloads as W
from oracle import attention as OA
from oracle import compact as OC
from oracle import masks as OM


def _specs(N, seed):
    rng = np.random.default_rng([seed, N])
    cuts = W.uniform_cuts(rng, min(3, N - 1), 1, N - 1) if N > 1 else []
    bounds = W.doc_boundaries_from_cuts(cuts, N)
    drop = np.sort(rng.choice(N, size=max(1, N // 3), replace=False))
    kept_blocks = np.sort(rng.choice(-(-N // 8), size=max(1, -(-N // 8) // 3), replace=False))
    return {
        "full": W.encode_full(N),
        "causal": W.encode_causal(N),
        "causal_document": W.encode_causal_document(bounds, N),
        "causal_window_5": W.encode_causal_window(5, N),
        "prefix_lm": W.encode_prefix_lm(N // 2, N),
        "causal_key_drop": W.encode_causal_key_drop([drop], N),
        "block_sparse": W.encode_causal_document_block_sparse(bounds, kept_blocks, 8, N),
        "bidirectional_document": W.encode_bidirectional_document(bounds, N),
    }


def _random_vectors(rng, N):
    """Arbitrary vectors, out-of-range values and empty spans included."""
    v = [rng.integers(-3, N + 4, size=N) for _ in range(4)]
    return v[0], v[1], v[2], v[3]


def _check_slice(vecs, causal, N):
    masked = OM.dense_masked(*vecs, causal, N)
    kidx, kpos, count, *vecs2 = OC.compact_keys_slice(*vecs, causal, N)
    keep = (~masked).any(axis=0)
    assert np.array_equal(OC.kept_columns(*vecs, causal, N), keep)
    if count < 0:
        return count
    assert count == keep.sum()
    assert np.array_equal(kidx[:count], np.nonzero(keep)[0]) and np.all(kidx[count:] == -1)
    assert np.all(kpos[~keep] == -1) and np.array_equal(kidx[kpos[keep]], np.nonzero(keep)[0])
    masked2 = OM.dense_masked(*vecs2, False, N)
    assert np.array_equal(masked2[:, :count], masked[:, kidx[:count]])
    assert masked2[:, count:].all()
    return count


@pytest.mark.parametrize("N", [1, 2, 3, 7, 16, 64, 97])
@pytest.mark.parametrize("seed", [0, 1])
def test_family_compaction_matches_dense_mask(N, seed):
    for name, spec in _specs(N, seed).items():
        count = _check_slice(spec.column_slice(0, 0), spec.causal, N)
        assert count >= 0, name


@pytest.mark.parametrize("N", [5, 16, 40])
@pytest.mark.parametrize("causal", [False, True])
def test_arbitrary_vectors(N, causal):
    rng = np.random.default_rng([N, int(causal)])
    for _ in range(40):
        lts, lte, uts, ute = _random_vectors(rng, N)
        for vecs in ((lts, lte, uts, ute), (lts, lte, None, None), (None, None, uts, ute)):
            _check_slice(vecs, causal, N)


def test_key_drop_keeps_exactly_the_undropped_columns():
    N = 50
    drop = np.array([0, 3, 4, 17, 49])
    spec = W.encode_causal_key_drop([drop], N)
    kidx, kpos, count, *_ = OC.compact_keys_slice(*spec.column_slice(0, 0), True, N)
    assert count == N - len(drop)
    assert set(kidx[:count]) == set(range(N)) - set(drop.tolist())


def test_three_disjoint_spans_are_not_compactable():
    # column 4 under the causal flag: rows [0, 4), LT [8, 10) and UT [12, 14) are disjoint and leave rows
    # unmasked, so the column is kept but needs three spans
    N = 16
    lts, lte = np.full(N, N), np.full(N, N)
    uts, ute = np.zeros(N, np.int64), np.zeros(N, np.int64)
    lts[4], lte[4], uts[4], ute[4] = 8, 10, 12, 14
    kidx, kpos, count, *_ = OC.compact_keys_slice(lts, lte, uts, ute, True, N)
    assert count == -1
    # without the causal flag the same column fits
    assert _check_slice((lts, lte, uts, ute), False, N) == N


@pytest.mark.parametrize("family", ["causal_key_drop", "block_sparse", "causal_document"])
def test_attention_on_the_compacted_problem_is_unchanged(family):
    N, d = 48, 8
    spec = _specs(N, 3)[family]
    rng = np.random.default_rng(7)
    q, k, v, do = (rng.standard_normal((N, d)) for _ in range(4))
    scale = 1.0 / math.sqrt(d)
    vecs = spec.column_slice(0, 0)
    out, lse, dq, dk, dv = OA.fwd_bwd_head(q, k, v, do, vecs, spec.causal, scale)
    kidx, kpos, count, *vecs2 = OC.compact_keys_slice(*vecs, spec.causal, N)
    k2, v2 = OC.gather_rows(k, kidx), OC.gather_rows(v, kidx)
    out2, lse2, dq2, dk2, dv2 = OA.fwd_bwd_head(q, k2, v2, do, vecs2, False, scale)
    assert np.max(np.abs(out2 - out)) <= 1e-12
    fin = np.isfinite(lse)
    assert np.array_equal(fin, np.isfinite(lse2))
    assert np.max(np.abs(lse2[fin] - lse[fin]), initial=0.0) <= 1e-12
    assert np.max(np.abs(dq2 - dq)) <= 1e-12
    assert np.max(np.abs(OC.gather_rows(dk2, kpos) - dk)) <= 1e-12
    assert np.max(np.abs(OC.gather_rows(dv2, kpos) - dv)) <= 1e-12
    dropped = kpos < 0
    assert np.all(dk[dropped] == 0) and np.all(dv[dropped] == 0)
