"""Pins of the mask encodings and of the oracle's dense expansion and unmasked-pair count (CPU)."""
import os

import numpy as np
import pytest

import workloads as W
from oracle import masks as OM

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "masks_n8.txt")


def _parse_golden():
    blocks, cur = [], None
    with open(GOLDEN) as f:
        for raw in f:
            line = raw.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("family"):
                parts = line.split()
                cur = {"family": parts[1], "params": dict(p.split("=") for p in parts[2:]), "rows": []}
                blocks.append(cur)
            elif line.startswith("causal"):
                cur["causal"] = bool(int(line.split()[1]))
            elif line.split()[0] in ("LTS", "LTE", "UTS", "UTE"):
                key, *vals = line.split()
                cur[key] = None if vals == ["NULL"] else np.array([int(x) for x in vals])
            else:
                cur["rows"].append([c == "1" for c in line])
    for b in blocks:
        b["allowed"] = np.array(b["rows"], dtype=bool)
    return blocks


def _encode_from_params(fam, params, N):
    ints = lambda s: [int(x) for x in s.split(",")]  # noqa: E731
    if fam == "causal_document":
        return W.encode_causal_document(np.array(ints(params["bounds"])), N)
    if fam == "causal_window":
        return W.encode_causal_window(int(params["w"]), N)
    if fam == "prefix_lm":
        return W.encode_prefix_lm(int(params["P"]), N)
    if fam == "share_question":
        return W.encode_share_question(int(params["Q"]), np.array(ints(params["answers"])), N)
    if fam == "bidirectional_document":
        return W.encode_bidirectional_document(np.array(ints(params["bounds"])), N)
    if fam == "causal_key_drop":
        return W.encode_causal_key_drop([np.array(ints(params["dropped"]))], N)
    if fam == "causal_by_vectors":
        return W.encode_causal_by_vectors(N)
    raise KeyError(fam)


def _twin_from_params(fam, params, N):
    ints = lambda s: [int(x) for x in s.split(",")]  # noqa: E731
    if fam == "causal_document":
        return OM.twin_causal_document(ints(params["bounds"]), N)
    if fam == "causal_window":
        return OM.twin_causal_window(int(params["w"]), N)
    if fam == "prefix_lm":
        return OM.twin_prefix_lm(int(params["P"]), N)
    if fam == "share_question":
        return OM.twin_share_question(int(params["Q"]), ints(params["answers"]), N)
    if fam == "bidirectional_document":
        return OM.twin_bidirectional_document(ints(params["bounds"]), N)
    if fam == "causal_key_drop":
        return OM.twin_causal_key_drop(ints(params["dropped"]), N)
    if fam == "causal_by_vectors":
        return OM.twin_causal(N)
    raise KeyError(fam)


@pytest.mark.parametrize("block", _parse_golden(), ids=lambda b: b["family"] + str(b["params"]))
def test_golden_hand_drawn(block):
    N = 8
    allowed = block["allowed"]
    assert allowed.shape == (N, N)
    # the hand-written vectors expand to the hand-drawn matrix
    vecs = tuple(block[k] for k in ("LTS", "LTE", "UTS", "UTE"))
    assert np.array_equal(~OM.dense_masked(*vecs, block["causal"], N), allowed)
    # the encoder writes exactly the hand-written vectors
    spec = _encode_from_params(block["family"], block["params"], N)
    assert spec.causal == block["causal"]
    for got, want in zip(spec.column_slice(0, 0), vecs):
        assert (got is None) == (want is None)
        if want is not None:
            assert np.array_equal(got, want)
    # the dense twin draws the same matrix
    assert np.array_equal(_twin_from_params(block["family"], block["params"], N), allowed)


SIZES = [1, 2, 3, 7, 16, 64, 256]


def _families(N, rng):
    """(encoded spec, dense twin allowed) pairs with seeded random parameters at size N."""
    out = []
    cuts = W.uniform_cuts(rng, int(rng.integers(0, min(N - 1, 5) + 1)), 1, N - 1) if N > 1 else []
    bounds = W.doc_boundaries_from_cuts(cuts, N)
    w = int(rng.integers(1, N + 2))
    P = int(rng.integers(0, N + 1))
    out.append((W.encode_full(N), OM.twin_full(N)))
    out.append((W.encode_causal(N), OM.twin_causal(N)))
    out.append((W.encode_causal_by_vectors(N), OM.twin_causal(N)))
    out.append((W.encode_causal_document(bounds, N), OM.twin_causal_document(bounds, N)))
    out.append((W.encode_causal_window(w, N), OM.twin_causal_window(w, N)))
    out.append((W.encode_causal_document_window(bounds, w, N), OM.twin_causal_document_window(bounds, w, N)))
    out.append((W.encode_prefix_lm(P, N), OM.twin_prefix_lm(P, N)))
    out.append((W.encode_bidirectional_document(bounds, N), OM.twin_bidirectional_document(bounds, N)))
    if N >= 2:
        Q = int(rng.integers(1, N))
        n_ans = int(rng.integers(0, min(3, N - Q - 1) + 1)) if N - Q - 1 > 0 else 0
        acuts = W.uniform_cuts(rng, n_ans, Q + 1, N - 1) if n_ans else np.zeros(0, np.int64)
        ab = np.concatenate([[Q], acuts, [N]])
        out.append((W.encode_share_question(Q, ab, N), OM.twin_share_question(Q, ab, N)))
    drop = np.sort(rng.choice(N, size=int(rng.integers(0, N + 1)), replace=False))
    out.append((W.encode_causal_key_drop([drop], N), OM.twin_causal_key_drop(drop, N)))
    blk = max(1, N // 4)
    nblk = -(-N // blk)
    kept = np.sort(rng.choice(nblk, size=int(rng.integers(0, nblk + 1)), replace=False))
    out.append((W.encode_causal_document_block_sparse(bounds, kept, blk, N),
                OM.twin_causal_document_block_sparse(bounds, kept, blk, N)))
    return out


@pytest.mark.parametrize("N", SIZES)
@pytest.mark.parametrize("seed", range(4))
def test_encodings_equal_dense_twins(N, seed):
    rng = np.random.default_rng([N, seed])
    for spec, allowed in _families(N, rng):
        got = ~OM.dense_masked(*spec.column_slice(0, 0), spec.causal, N)
        assert np.array_equal(got, allowed), spec.family


@pytest.mark.parametrize("N", SIZES)
@pytest.mark.parametrize("seed", range(3))
def test_unmasked_count_matches_dense(N, seed):
    rng = np.random.default_rng([100 + N, seed])
    for spec, allowed in _families(N, rng):
        U = OM.unmasked_count_slice(*spec.column_slice(0, 0), spec.causal, N)
        assert U == int(allowed.sum()), spec.family


def test_unmasked_count_arbitrary_vectors_matches_dense():
    # arbitrary (also empty, reversed and out-of-range) intervals with and without the causal flag
    rng = np.random.default_rng(7)
    for N in (1, 5, 33, 100):
        for _ in range(20):
            vecs = [rng.integers(-3, N + 4, size=N) for _ in range(4)]
            for causal in (False, True):
                m = OM.dense_masked(*vecs, causal, N)
                assert OM.unmasked_count_slice(*vecs, causal, N) == int((~m).sum())


@pytest.mark.parametrize("N", [1, 2, 100, 2048, 131072])
def test_unmasked_count_closed_forms(N):
    assert OM.unmasked_count_slice(None, None, None, None, False, N) == N * N
    assert OM.unmasked_count_slice(None, None, None, None, True, N) == N * (N + 1) // 2
    for w in (1, 7, 1024):
        spec = W.encode_causal_window(w, N)
        want = sum(min(i + 1, w) for i in range(N)) if N <= 4096 else \
            (w * (w + 1) // 2 + (N - w) * w if N >= w else N * (N + 1) // 2)
        assert OM.unmasked_count_slice(*spec.column_slice(0, 0), True, N) == want


def test_causal_flag_equals_vector_causal():
    for N in (1, 9, 130):
        a = OM.dense_masked(*W.encode_causal(N).column_slice(0, 0), True, N)
        s = W.encode_causal_by_vectors(N)
        b = OM.dense_masked(*s.column_slice(0, 0), False, N)
        assert np.array_equal(a, b)


def test_config_masks_are_well_formed():
    # every workload mask draws with the stated sizes; done at a reduced N for speed
    for cfg in W.CONFIGS:
        for mi, name in enumerate(cfg.masks):
            N = min(cfg.N, 2048)
            spec = W.make_mask(cfg.index, name, cfg.B, cfg.H, N, mi)
            assert spec.N == N and spec.B == cfg.B and spec.Hm in (1, cfg.H)
            for x in spec.vectors():
                if x is not None:
                    assert x.dtype == np.int32 and x.shape == (cfg.B, spec.Hm, N)


def test_key_drop_workload_drops_exactly_30_percent():
    N, H = 32768, 32
    spec = W.make_mask(3, "causal_key_drop", 1, H, N, 2)
    assert spec.Hm == H
    for h in range(H):
        assert int((spec.lts[0, h] == 0).sum()) == round(0.3 * N)


def test_block_sparse_workload_keeps_10_percent_of_blocks():
    N = 131072
    spec = W.make_mask(4, "causal_document_block_sparse", 1, 8, N, 2)
    dropped_cols = (spec.lts[0, 0] == 0)
    kept_blocks = (~dropped_cols).reshape(-1, 128).all(axis=1)
    assert int(kept_blocks.sum()) == 102
    assert np.array_equal(dropped_cols.reshape(-1, 128).all(axis=1), ~kept_blocks)
