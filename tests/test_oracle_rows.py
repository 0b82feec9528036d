"""Pins of the oracle's row-block form (one rank's query rows against all keys, FlashMask-3 summary,
readmex.ai) against the square oracle: over a partition of the query rows, the blocks' out, lse and dq
rows are the whole problem's rows and their dk, dv contributions sum to the whole dk, dv (CPU)."""
import math

import numpy as np
import pytest

import workloads as W
from oracle import attention as OA


def _spec(family, N, rng):
    cuts = W.uniform_cuts(rng, min(3, N - 1), 1, N - 1)
    bounds = W.doc_boundaries_from_cuts(cuts, N)
    if family == "causal_document":
        return W.encode_causal_document(bounds, N)
    if family == "prefix_lm":
        return W.encode_prefix_lm(N // 3, N)
    if family == "causal_key_drop":
        return W.encode_causal_key_drop([np.sort(rng.choice(N, size=N // 4, replace=False))], N)
    if family == "bidirectional_document":
        return W.encode_bidirectional_document(bounds, N)
    return W.encode_causal_window(7, N)


@pytest.mark.parametrize("family", ["causal_document", "prefix_lm", "causal_key_drop",
                                    "bidirectional_document", "causal_window"])
@pytest.mark.parametrize("cuts", [(0, 30, 61, 90), (0, 1, 45, 90), (0, 90)])
def test_row_blocks_reassemble_the_whole_problem(family, cuts):
    N, d = 90, 6
    rng = np.random.default_rng([N, len(cuts)])
    spec = _spec(family, N, rng)
    q, k, v, do = (rng.standard_normal((N, d)) for _ in range(4))
    scale = 1.0 / math.sqrt(d)
    vecs = spec.column_slice(0, 0)
    out, lse, dq, dk, dv = OA.fwd_bwd_head(q, k, v, do, vecs, spec.causal, scale)
    dk_sum, dv_sum = np.zeros_like(dk), np.zeros_like(dv)
    for a, b in zip(cuts[:-1], cuts[1:]):
        o, l_, gq, gk, gv = OA.fwd_bwd_rows_head(q[a:b], k, v, do[a:b], vecs, spec.causal, scale, a, row_block=13)
        assert np.max(np.abs(o - out[a:b])) <= 1e-12
        fin = np.isfinite(lse[a:b])
        assert np.array_equal(fin, np.isfinite(l_))
        assert np.max(np.abs(l_[fin] - lse[a:b][fin]), initial=0.0) <= 1e-12
        assert np.max(np.abs(gq - dq[a:b])) <= 1e-12
        dk_sum += gk
        dv_sum += gv
    assert np.max(np.abs(dk_sum - dk)) <= 1e-12
    assert np.max(np.abs(dv_sum - dv)) <= 1e-12


def test_chunked_head_equals_whole_head():
    """The row-chunked form used by the full-size checks sums the same float64 terms as fwd_bwd_head."""
    from concurrent.futures import ThreadPoolExecutor
    from oracle import attention as OA
    import workloads as W
    rng = np.random.default_rng(11)
    N, d = 700, 64
    spec = W.make_mask(2, "causal_document", 1, 1, N, 0)
    q, k, v, do = (rng.standard_normal((N, d)) for _ in range(4))
    ref = OA.fwd_bwd_head(q, k, v, do, spec.column_slice(0, 0), spec.causal, 0.125)
    with ThreadPoolExecutor(max_workers=4) as pool:
        got = OA.fwd_bwd_head_parallel(q, k, v, do, spec.column_slice(0, 0), spec.causal, 0.125, pool, 96)
    for a, b in zip(got, ref):
        assert np.allclose(a, b, rtol=1e-12, atol=1e-12, equal_nan=True)
