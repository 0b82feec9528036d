"""Pins of the hash-bucket oracle (CPU): the reordered problem's column-wise mask expands to exactly the
permuted hash mask, one bucket is plain causal attention, a hand-derived six-token case, the LSH
symmetries and a hand rotation, dropped tokens, brute force and float64 autograd."""
import math

import numpy as np
import pytest
import torch

from oracle import attention as OA
from oracle import hashing as OH
from oracle import masks as OM


@pytest.mark.parametrize("N", [1, 5, 64, 200])
@pytest.mark.parametrize("nb", [1, 2, 8])
def test_sorted_vectors_reproduce_permuted_mask(N, nb):
    rng = np.random.default_rng(N * 10 + nb)
    for _ in range(3):
        qb = rng.integers(-1, nb + 1, size=N)   # includes dropped tokens (-1 and nb)
        kb = rng.integers(-1, nb + 1, size=N)
        qidx, qpos, kidx, kpos, lts, lte, uts, ute = OH.bucket_sort(qb, kb, nb)
        assert sorted(qidx) == list(range(N)) and np.array_equal(qpos[qidx], np.arange(N))
        assert sorted(kidx) == list(range(N)) and np.array_equal(kpos[kidx], np.arange(N))
        want = OH.hash_masked(qb, kb, nb)[qidx][:, kidx]
        got = OM.dense_masked(lts, lte, uts, ute, False, N)
        assert np.array_equal(got, want)


def test_one_bucket_is_plain_causal():
    N = 37
    z = np.zeros(N, np.int64)
    i, j = np.meshgrid(np.arange(N), np.arange(N), indexing="ij")
    assert np.array_equal(OH.hash_masked(z, z, 1), i < j)
    qidx, qpos, kidx, kpos, lts, lte, uts, ute = OH.bucket_sort(z, z, 1)
    assert np.array_equal(qidx, np.arange(N)) and np.array_equal(kidx, np.arange(N))
    assert np.array_equal(ute, np.arange(N)) and np.all(uts == 0)   # column j: rows [0, j) masked
    assert np.all(lts == N) and np.all(lte == N)


def test_hand_derived_six_tokens():
    # buckets: queries 1 0 0 1 0 1, keys 0 1 0 0 1 1 (two buckets). Sorted queries: bucket 0 at positions
    # 1, 2, 4 (rows 0-2), bucket 1 at 0, 3, 5 (rows 3-5). Sorted keys: bucket 0 at 0, 2, 3 (columns
    # 0-2), bucket 1 at 1, 4, 5 (columns 3-5). Column c is attended by its bucket's queries at positions
    # >= the key's: key 0 by rows 0-2, key 2 by rows 1-2, key 3 by row 2; key 1 by rows 4-5, keys 4
    # and 5 by row 5.
    qb = np.array([1, 0, 0, 1, 0, 1])
    kb = np.array([0, 1, 0, 0, 1, 1])
    qidx, qpos, kidx, kpos, lts, lte, uts, ute = OH.bucket_sort(qb, kb, 2)
    assert list(qidx) == [1, 2, 4, 0, 3, 5]
    assert list(kidx) == [0, 2, 3, 1, 4, 5]
    assert list(qpos) == [3, 0, 1, 4, 2, 5]
    assert list(uts) == [0] * 6
    assert list(ute) == [0, 1, 2, 4, 5, 5]
    assert list(lts) == [3, 3, 3, 6, 6, 6]
    assert list(lte) == [6] * 6


def test_lsh_symmetries_and_hand_rotation():
    rng = np.random.default_rng(2)
    d, nb = 16, 8
    R = rng.standard_normal((d, nb // 2))
    x = rng.standard_normal((50, d))
    b = OH.lsh_buckets(x, R)
    assert np.all((b >= 0) & (b < nb))
    assert np.array_equal(OH.lsh_buckets(-x, R), (b + nb // 2) % nb)   # antipodal rows swap halves
    assert np.array_equal(OH.lsh_buckets(3.5 * x, R), b)                # positive scale does not move
    # rotation = the first two unit vectors: scores [x0, x1, -x0, -x1]
    R2 = np.eye(4)[:, :2]
    assert list(OH.lsh_buckets(np.array([[0.5, -2.0, 1.0, 0.0]]), R2)) == [3]
    assert list(OH.lsh_buckets(np.array([[1.5, -0.2, 9.0, 0.0]]), R2)) == [0]
    assert list(OH.lsh_buckets(np.zeros((1, 4)), R2)) == [0]            # ties: first index


def test_dropped_tokens():
    rng = np.random.default_rng(4)
    N, d, nb = 40, 8, 4
    q, k, v, do = (rng.standard_normal((N, d)) for _ in range(4))
    qb = rng.integers(0, nb, size=N)
    kb = rng.integers(0, nb, size=N)
    qb[[0, 7, 20]] = -1
    kb[[3, 9, 39]] = nb
    out, lse, dq, dk, dv = OH.hash_attention_head(q, k, v, do, qb, kb, nb, 0.3)
    for i in (0, 7, 20):
        assert np.all(out[i] == 0) and lse[i] == -np.inf and np.all(dq[i] == 0)
    for j in (3, 9, 39):
        assert np.all(dk[j] == 0) and np.all(dv[j] == 0)


def test_brute_force_forward():
    rng = np.random.default_rng(5)
    N, d, nb = 24, 4, 4
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    qb = rng.integers(0, nb, size=N)
    kb = rng.integers(0, nb, size=N)
    out, lse, *_ = OH.hash_attention_head(q, k, v, np.zeros((N, d)), qb, kb, nb, 0.5)
    bo, bl = OA.brute_force_forward(q, k, v, OH.hash_masked(qb, kb, nb).tolist(), 0.5)
    assert np.allclose(out, bo, atol=1e-12, rtol=0)
    fin = np.isfinite(bl)
    assert np.array_equal(fin, np.isfinite(lse)) and np.allclose(lse[fin], bl[fin], atol=1e-12, rtol=0)


def test_gradients_against_float64_autograd():
    rng = np.random.default_rng(6)
    N, d, nb = 30, 8, 3
    q, k, v, do = (rng.standard_normal((N, d)) for _ in range(4))
    qb = rng.integers(-1, nb, size=N)
    kb = rng.integers(0, nb + 1, size=N)
    scale = 1.0 / math.sqrt(d)
    out, lse, dq, dk, dv = OH.hash_attention_head(q, k, v, do, qb, kb, nb, scale)
    masked = torch.from_numpy(OH.hash_masked(qb, kb, nb))
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    s = (tq @ tk.T * scale).masked_fill(masked, float("-inf"))
    alive = ~masked.all(dim=1)
    p = torch.where(alive[:, None], torch.softmax(torch.where(alive[:, None], s, torch.zeros_like(s)), dim=1)
                    .masked_fill(masked, 0.0), torch.zeros_like(s))
    o = p @ tv
    (o * torch.from_numpy(do)).sum().backward()
    assert np.allclose(out, o.detach().numpy(), atol=1e-12)
    for got, t in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.allclose(got, t.grad.numpy(), atol=1e-11)


def test_probes_match_the_whole_head():
    rng = np.random.default_rng(8)
    N, d, nb = 60, 8, 3
    q, k, v, do = (rng.standard_normal((N, d)) for _ in range(4))
    qb = rng.integers(-1, nb, size=N)
    kb = rng.integers(0, nb + 1, size=N)
    out, lse, dq, dk, dv = OH.hash_attention_head(q, k, v, do, qb, kb, nb, 0.4)
    rows = np.arange(N)
    po, pl, pdq = OH.hash_rows_probe(q, k, v, do, qb, kb, nb, 0.4, rows)
    assert np.allclose(po, out, atol=1e-12) and np.allclose(pdq, dq, atol=1e-12)
    assert np.array_equal(np.isfinite(pl), np.isfinite(lse))
    fin = np.isfinite(lse)
    assert np.allclose(pl[fin], lse[fin], atol=1e-12)
    pdk, pdv = OH.hash_cols_probe(q, k, v, do, qb, kb, nb, 0.4, rows)
    assert np.allclose(pdk, dk, atol=1e-12) and np.allclose(pdv, dv, atol=1e-12)
