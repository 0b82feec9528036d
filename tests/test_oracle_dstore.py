"""Pins of the oracle's stored-dS bookkeeping (oracle/dstore.py) against what the tile rule and the dense
mask fix: closed forms for the unmasked and plain causal problems, equality with spans read off the dense
mask where the tile rule is exact (tile-aligned documents), the prefix structure of base and region, and
the storage order of a tile against positions worked out by hand from the stated layout."""
import numpy as np
import pytest

from oracle import dstore as OD


def _docs_vectors(bounds, N, causal):
    """LT (and for bidirectional documents UT) vectors of documents with the given boundaries."""
    lts = np.zeros(N, np.int32)
    lte = np.full(N, N, np.int32)
    uts = np.zeros(N, np.int32)
    ute = np.zeros(N, np.int32)
    for s0, s1 in zip(bounds[:-1], bounds[1:]):
        lts[s0:s1] = s1
        ute[s0:s1] = s0
    return (lts, lte, None, None) if causal else (lts, lte, uts, ute)


@pytest.mark.parametrize("N", [128, 384, 1024])
def test_unmasked_and_causal_closed_forms(N):
    nq, nk = N // 64, N // 128
    f, s = OD.spans_slice(None, None, None, None, False, N)
    assert np.all(f == 0) and np.all(s == nq)
    f, s = OD.spans_slice(None, None, None, None, True, N)
    # key tile kt: rows below 128 kt are masked, so the first live 64-row tile is 2 kt; all later are live
    assert np.array_equal(f, 2 * np.arange(nk)) and np.array_equal(s, nq - 2 * np.arange(nk))
    p = OD.plan((None,) * 4, True, 2, 3, 1, N)
    per_head = int((nq - 2 * np.arange(nk)).sum())
    assert p["total"] == 2 * 3 * per_head
    assert np.array_equal(p["region"].ravel(), per_head * np.arange(6))


def test_ragged_causal_closed_form():
    N = 200  # tiles of 64 rows: 0..63, 64..127, 128..191, 192..199; key tiles 0..127, 128..199
    f, s = OD.spans_slice(None, None, None, None, True, N)
    assert list(f) == [0, 2] and list(s) == [4, 2]


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("bounds", [[0, 256, 384, 1024], [0, 128, 896, 1024], [0, 1024]])
def test_tile_aligned_documents_equal_dense_spans(causal, bounds):
    N = 1024
    vecs = _docs_vectors(bounds, N, causal)
    f, s = OD.spans_slice(*vecs, causal, N)
    fd, sd = OD.dense_spans(*vecs, causal, N)
    assert np.array_equal(s, sd)
    assert np.array_equal(f[s > 0], fd[sd > 0])


def test_random_vectors_never_smaller_than_dense():
    """The tile rule is sound (a FULL tile has no unmasked entry), so its span always covers the dense one."""
    rng = np.random.default_rng(7)
    N = 700
    for _ in range(5):
        a = rng.integers(-20, N + 20, size=(4, N)).astype(np.int32)
        vecs = (np.minimum(a[0], a[1]), np.maximum(a[0], a[1]), np.minimum(a[2], a[3]), np.maximum(a[2], a[3]))
        for causal in (True, False):
            f, s = OD.spans_slice(*vecs, causal, N)
            fd, sd = OD.dense_spans(*vecs, causal, N)
            live = sd > 0
            assert np.all(s[live] > 0)
            assert np.all(f[live] <= fd[live])
            assert np.all(f[live] + s[live] >= fd[live] + sd[live])


def test_plan_prefix_structure_per_head_masks():
    rng = np.random.default_rng(3)
    B, H, N = 2, 3, 512
    drop = rng.random((B, H, N)) < 0.3
    lts = np.where(drop, 0, N).astype(np.int32)
    lte = np.full((B, H, N), N, np.int32)
    p = OD.plan((lts, lte, None, None), True, B, H, H, N)
    run = 0
    for b in range(B):
        for h in range(H):
            f, s = OD.spans_slice(lts[b, h], lte[b, h], None, None, True, N)
            assert np.array_equal(p["base"][b, h], np.concatenate([[0], np.cumsum(s)[:-1]]))
            assert p["rowtotal"][b, h] == s.sum() and p["region"][b, h] == run
            run += int(s.sum())
    assert p["total"] == run


def test_tile_storage_order_by_hand():
    ds = np.arange(128 * 128, dtype=np.float64).reshape(128, 128) + 1.0  # (row r, key k): 128 r + k + 1
    out = OD.tile_values(ds, 0, 0)
    assert sorted(out.tolist()) == sorted(ds[:64].ravel().tolist())  # a permutation of the tile
    val = lambda r, k: 128 * r + k + 1  # noqa: E731
    # (row, key) -> element, from the layout: kg = k // 32, kl = k % 32, row = 32 ib + 16 p + 8 h + 4 g + e,
    # element ((kg * 4 + 2 ib + p) * 64 + 32 g + (kl ^ (8 g + 4 p))) * 8 + 4 h + e
    assert out[0] == val(0, 0) and out[3] == val(3, 0)
    assert out[4] == val(8, 0)                       # h = 1
    assert out[(32 + (0 ^ 8)) * 8] == val(4, 0)      # g = 1
    assert out[(64 + (0 ^ 4)) * 8] == val(16, 0)     # p = 1
    assert out[(128 + 0) * 8] == val(32, 0)          # ib = 1
    assert out[(4 * 64 + 5) * 8] == val(0, 37)       # kg = 1, kl = 5
    assert out[((3 * 4 + 3) * 64 + 32 + (31 ^ 12)) * 8 + 4 + 3] == val(63, 127)
