"""The benchmark's unmasked-pair count U (the FLOP count of the metric), over all rows and over row
blocks, against the dense mask of the oracle (CPU)."""
import numpy as np
import pytest

import bench
import workloads as W
from oracle import masks as OM


def _specs(N, rng):
    cuts = W.uniform_cuts(rng, min(3, N - 1), 1, N - 1)
    bounds = W.doc_boundaries_from_cuts(cuts, N)
    drop = [np.sort(rng.choice(N, size=N // 4, replace=False)) for _ in range(2)]
    return [W.encode_full(N), W.encode_causal(N), W.encode_causal_document(bounds, N),
            W.encode_prefix_lm(N // 2, N), W.encode_causal_key_drop(drop, N),
            W.encode_bidirectional_document(bounds, N), W.encode_causal_document_window(bounds, 5, N)]


@pytest.mark.parametrize("N", [1, 9, 64, 131])
def test_unmasked_pairs_match_dense(N):
    rng = np.random.default_rng(N)
    for spec in _specs(N, rng):
        H = 2
        want = 0
        for h in range(H):
            vecs = spec.column_slice(0, h if spec.Hm > 1 else 0)
            want += int((~OM.dense_masked(*vecs, spec.causal, N)).sum())
        assert bench.unmasked_pairs(spec, H) == want
        for a, b in ((0, N), (0, N // 2), (N // 3, N), (N // 4, N // 4 + max(1, N // 5))):
            if b <= a:
                continue
            want_rows = 0
            for h in range(H):
                vecs = spec.column_slice(0, h if spec.Hm > 1 else 0)
                want_rows += int((~OM.dense_masked_rows(*vecs, spec.causal, N, a, b)).sum())
            assert bench.unmasked_pairs(spec, H, rows=(a, b)) == want_rows


def test_unmasked_pairs_arbitrary_vectors():
    rng = np.random.default_rng(5)
    N = 37
    for causal in (False, True):
        v = [rng.integers(-3, N + 4, size=(1, 1, N)).astype(np.int32) for _ in range(4)]
        spec = W.MaskSpec(N, 1, 1, causal, *v)
        dense = OM.dense_masked(*spec.column_slice(0, 0), causal, N)
        assert bench.unmasked_pairs(spec, 1) == int((~dense).sum())
        assert bench.unmasked_pairs(spec, 1, rows=(5, 30)) == int((~dense[5:30]).sum())
