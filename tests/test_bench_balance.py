"""Host logic of the benchmark's balanced row blocks (CPU): per-row unmasked counts against the dense
mask, their sum against the pair count, and the balanced boundaries."""
import numpy as np

import bench
import workloads as W
from oracle import masks as OM


def _specs(N, rng):
    bounds = W.doc_boundaries_from_cuts(W.uniform_cuts(rng, 4, 1, N - 1), N)
    drop = np.sort(rng.choice(N, size=N // 4, replace=False))
    return [W.encode_causal(N), W.encode_full(N), W.encode_causal_document(bounds, N),
            W.encode_prefix_lm(N // 3, N), W.encode_share_question(N // 4, np.array([N // 4, N // 2, N]), N),
            W.encode_causal_key_drop([drop], N), W.encode_bidirectional_document(bounds, N),
            W.encode_causal_document_window(bounds, 17, N)]


def test_unmasked_per_row_against_dense_mask():
    rng = np.random.default_rng(2)
    for N in (1, 50, 257):
        for spec in _specs(max(N, 8), rng):
            n = spec.N
            want = np.zeros(n, np.int64)
            for h in range(spec.Hm):
                v = [None if x is None else x[0, h] for x in spec.vectors()]
                want += (~OM.dense_masked(*v, spec.causal, n)).sum(axis=1)
            got = bench.unmasked_per_row(spec, spec.Hm)
            assert np.array_equal(got, want), spec.family
            assert int(got.sum()) == bench.unmasked_pairs(spec, spec.Hm)


def test_balanced_boundaries():
    N = 4096
    spec = W.encode_causal(N)
    cuts = bench.balanced_row_blocks(spec, 1, 4)
    assert cuts[0] == 0 and cuts[-1] == N and all(b % 128 == 0 for b in cuts) and cuts == sorted(cuts)
    # causal: row i has i + 1 keys, so equal shares of i^2/2 put the cuts near N sqrt(r / 4)
    for r, c in enumerate(cuts[1:-1], start=1):
        assert abs(c - N * np.sqrt(r / 4)) <= 128
