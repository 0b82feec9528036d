"""GPU checks at a large sequence length (N = 2^20), where row and column indices, tensor offsets and the
split bucket sort run far past the workloads' sizes. The mask is a causal sliding window, so the attention
work stays small; sampled rows and columns are held to the parity bars against the oracle's one-row and
one-column probes, and the tile bounds of sampled tiles are compared bit-exactly. The bucket sort of one
head is checked by its defining properties and, on sampled key columns, against the reordered mask
computed from the definition."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as OA
from tests import fmcase as C

pytestmark = pytest.mark.gpu

N = 1 << 20


@pytest.fixture(scope="module")
def fm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mask_aware_exact_amd as m
    m.load_library()
    return m


def test_window_attention_at_one_million_tokens(fm):
    print(f"\nlarge N: causal window 300, N {N}", flush=True)
    B, H, d, w = 1, 2, 128, 300
    spec = W.encode_causal_window(w, N, B)
    rng = np.random.default_rng(21)
    host = [rng.standard_normal((B, H, N, d), dtype=np.float32) for _ in range(4)]
    q, k, v, do = (torch.from_numpy(x).to(torch.bfloat16) for x in host)
    del host
    vecs = C.device_vectors(spec)
    bounds = fm.fm_tile_bounds(*vecs, B, 1, N)
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    scale = d ** -0.5
    out, lse = fm.fm_fwd(qd, kd, vd, *vecs, bounds=bounds, causal=True, scale=scale)
    dq, dk, dv = fm.fm_bwd(qd, kd, vd, out, dod, lse, *vecs, bounds=bounds, causal=True, scale=scale)
    torch.cuda.synchronize()
    bh = bounds.cpu().numpy()[0, 0]
    vcol = spec.column_slice(0, 0)
    for t in (0, 1, 7777, bh.shape[0] - 1):
        # min / max of LTS and LTE over the tile's columns (the window mask has no UT pair)
        got = bh[t]
        cols = slice(t * 64, min(N, (t + 1) * 64))
        assert got[0] == vcol[0][cols].min() and got[1] == vcol[0][cols].max()
        assert got[2] == vcol[1][cols].min() and got[3] == vcol[1][cols].max()
        assert list(got[4:]) == [0, 0, 0, 0]
    tol = C.TOL["bf16"]
    rows = np.array([0, 1, 299, 300, 123457, N // 2 + 3, N - 2, N - 1])
    cols = np.array([0, 5, N // 3, N - 300, N - 1])
    for hh in range(H):
        qh, kh, vh, doh = (C.f64(t[0, hh]) for t in (q, k, v, do))
        r_out, r_lse, _, r_dq = OA.rows_probe(qh, kh, vh, doh, vcol, True, scale, rows)
        assert np.max(np.abs(C.f64(out[0, hh, rows].cpu()) - r_out)) <= tol["out"]
        assert np.max(np.abs(lse[0, hh, rows].cpu().double().numpy() - r_lse)) <= tol["lse"]
        assert C.rel_fro(C.f64(dq[0, hh, rows].cpu()), r_dq) <= tol["grad"]
        r_dk, r_dv = OA.cols_probe(qh, kh, vh, doh, vcol, True, scale, cols)
        assert C.rel_fro(C.f64(dk[0, hh, cols].cpu()), r_dk) <= tol["grad"]
        assert C.rel_fro(C.f64(dv[0, hh, cols].cpu()), r_dv) <= tol["grad"]
        print(f"  head {hh} ok", flush=True)


def test_bucket_sort_at_one_million_tokens(fm):
    print(f"\nlarge N: bucket sort, N {N}", flush=True)
    nb = 16
    qb, kb = W.make_buckets(4, 104, 1, 1, N, nb, 0.01)
    qidx, qpos, kidx, kpos, vecs = fm.fm_bucket_sort(torch.from_numpy(qb).cuda(), torch.from_numpy(kb).cuda(), nb)
    torch.cuda.synchronize()
    qi, qp, ki, kp = (t.cpu().numpy()[0, 0].astype(np.int64) for t in (qidx, qpos, kidx, kpos))
    lts, lte, uts, ute = (t.cpu().numpy()[0, 0].astype(np.int64) for t in vecs)
    grp = lambda x: np.where((x >= 0) & (x < nb), x, nb)  # noqa: E731
    gq, gk = grp(qb[0, 0].astype(np.int64)), grp(kb[0, 0].astype(np.int64))
    # permutations, inverse of each other, stable by group
    assert np.array_equal(np.sort(qi), np.arange(N)) and np.array_equal(qp[qi], np.arange(N))
    assert np.array_equal(np.sort(ki), np.arange(N)) and np.array_equal(kp[ki], np.arange(N))
    assert np.array_equal(qi, np.argsort(gq, kind="stable")) and np.array_equal(ki, np.argsort(gk, kind="stable"))
    # the reordered mask on sampled key columns, from the definition
    qs = np.searchsorted(gq[qi], np.arange(nb + 1), side="left")
    qe = np.searchsorted(gq[qi], np.arange(nb + 1), side="right")
    rng = np.random.default_rng(5)
    for c in np.concatenate([[0, N - 1], rng.integers(0, N, size=40)]):
        p, b = int(ki[c]), int(gk[ki[c]])
        if b == nb:
            assert (uts[c], ute[c], lts[c], lte[c]) == (0, N, N, N)
            continue
        lo = qs[b] + int(np.count_nonzero(qi[qs[b]:qe[b]] < p))
        assert (uts[c], ute[c]) == (0, lo)
        assert (lts[c], lte[c]) == ((qe[b], N) if qe[b] < N else (N, N))
