"""GPU parity of hash-bucket sparse causal attention: the bucket hash (fm_lsh_buckets), the reordering
and its mask (fm_bucket_sort, bit-exact), and attention through the reordered problem against the
oracle's attention under the hash mask in original order; at the hash workloads' full sizes, sampled
rows and columns.

The hash decides an integer from float32 dot products, the oracle from float64 ones. Rows whose two
largest scores are closer than the float32 error bound d * 2^-23 * max_j sum_k |x_k R_kj| may take
either bucket; there the GPU's bucket must reach the maximum within that bound, and every other row must
match exactly. Attention parity takes its buckets from the seeded generator, never from the GPU hash."""
import os
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402
from oracle import hashing as OH  # noqa: E402
from tests import fmcase as C  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mask_aware_exact_amd as m
    m.load_library()
    return m


def _check_lsh(gpu_b, x64, R64, report=None):
    """gpu_b [N] against the float64 scores of x64 [N, d] under R64 [d, nb/2]."""
    sc = OH.lsh_scores(x64, R64)
    d = x64.shape[1]
    bound = d * 2.0 ** -23 * (np.abs(x64) @ np.abs(R64)).max(axis=1)
    srt = np.sort(sc, axis=1)
    gap = srt[:, -1] - srt[:, -2]
    want = np.argmax(sc, axis=1)
    clear = gap > 2 * bound
    assert np.array_equal(gpu_b[clear], want[clear])
    picked = sc[np.arange(len(gpu_b)), gpu_b]
    assert np.all(picked >= srt[:, -1] - 2 * bound[:])
    if report is not None:
        report["near_ties"] = int((~clear).sum())
    return clear


@pytest.mark.parametrize("dtype,d,nb,Hr", [("bf16", 128, 16, 1), ("bf16", 64, 8, 2), ("f32", 128, 64, 2),
                                           ("f32", 64, 2, 1), ("bf16", 128, 10, 2)])
def test_lsh_matches_oracle(fm, dtype, d, nb, Hr):
    print(f"\nlsh {dtype} d{d} nb{nb} Hr{Hr}", flush=True)
    B, H, N = 2, 2, 1000
    x = torch.from_numpy(W.make_tensors(2, 100 + d + nb, B, H, N, d)[0]).to(C.TORCH_DT[dtype])
    R = W.make_rotation(2, 100 + nb, Hr, d, nb)
    gb = fm.fm_lsh_buckets(x.cuda(), torch.from_numpy(R).cuda(), nb).cpu().numpy()
    assert gb.min() >= 0 and gb.max() < nb
    for b in range(B):
        for h in range(H):
            _check_lsh(gb[b, h], C.f64(x[b, h]), R[h if Hr > 1 else 0].astype(np.float64))


@pytest.mark.parametrize("d,nb,N", [(128, 64, 1), (128, 64, 31), (64, 2, 129), (128, 2, 33), (64, 64, 300),
                                    (128, 6, 128)])
def test_lsh_bf16_edges_match_oracle(fm, d, nb, N):
    """bf16 rows: every rotation width from one projection to 32, and row counts below, at and one past a
    workgroup's 128 rows."""
    print(f"\nlsh bf16 edges d{d} nb{nb} N{N}", flush=True)
    B, H = 1, 3
    x = torch.from_numpy(W.make_tensors(2, 300 + d + nb + N, B, H, N, d)[0]).to(torch.bfloat16)
    R = W.make_rotation(2, 300 + nb, H, d, nb)
    gb = fm.fm_lsh_buckets(x.cuda(), torch.from_numpy(R).cuda(), nb).cpu().numpy()
    assert gb.min() >= 0 and gb.max() < nb
    for h in range(H):
        _check_lsh(gb[0, h], C.f64(x[0, h]), R[h].astype(np.float64))


# rows of 4096 positions or more are split into segments of at least 2048, one workgroup each
SORT_CASES = [(1, 1, 1, 4), (2, 2, 63, 3), (1, 2, 1000, 16), (2, 1, 2500, 512), (1, 1, 777, 1), (1, 3, 4097, 8),
              (1, 2, 10000, 512), (2, 1, 8192, 16), (1, 1, 12345, 1)]


@pytest.mark.parametrize("B,H,N,nb", SORT_CASES)
def test_bucket_sort_matches_oracle(fm, B, H, N, nb):
    print(f"\nbucket sort B{B} H{H} N{N} nb{nb}", flush=True)
    rng = np.random.default_rng(N + nb)
    qb = rng.integers(0, nb, size=(B, H, N)).astype(np.int32)
    kb = rng.integers(0, nb, size=(B, H, N)).astype(np.int32)
    drop = rng.random((2, B, H, N)) < 0.05
    qb[drop[0]] = rng.choice(np.array([-1, nb, 1 << 30, -(1 << 30)], np.int32), size=int(drop[0].sum()))
    kb[drop[1]] = -7
    out = fm.fm_bucket_sort(torch.from_numpy(qb).cuda(), torch.from_numpy(kb).cuda(), nb)
    got = [t.cpu().numpy() for t in out[:4]] + [t.cpu().numpy() for t in out[4]]
    for b in range(B):
        for h in range(H):
            want = OH.bucket_sort(qb[b, h], kb[b, h], nb)
            for name, g, w in zip(("qidx", "qpos", "kidx", "kpos", "lts", "lte", "uts", "ute"), got, want):
                assert np.array_equal(g[b, h], w), (name, b, h)


HASH_CASES = [
    # (dtype, d, B, H, N, nb, drop)
    ("bf16", 128, 1, 2, 1000, 4, 0.0),
    ("bf16", 128, 1, 2, 1537, 8, 0.05),
    ("bf16", 64, 1, 3, 2048, 16, 0.0),
    ("f32", 64, 2, 1, 700, 3, 0.1),
    ("f32", 128, 1, 2, 129, 1, 0.0),
]


@pytest.mark.parametrize("dtype,d,B,H,N,nb,drop", HASH_CASES)
def test_hash_attention_parity(fm, dtype, d, B, H, N, nb, drop):
    print(f"\nhash attention {dtype} d{d} B{B} H{H} N{N} nb{nb} drop{drop}", flush=True)
    q, k, v, do = (torch.from_numpy(x).to(C.TORCH_DT[dtype]) for x in W.make_tensors(2, 101, B, H, N, d))
    qb, kb = W.make_buckets(2, 101 + nb, B, H, N, nb, drop)
    scale = d ** -0.5
    gpu = C.run_gpu_hash(fm, q.cuda(), k.cuda(), v.cuda(), do.cuda(), torch.from_numpy(qb).cuda(),
                         torch.from_numpy(kb).cuda(), nb, scale)
    out, lse, dq, dk, dv = OH.hash_attention(C.f64(q), C.f64(k), C.f64(v), C.f64(do), qb, kb, nb, scale)
    ref = {"out": out, "lse": lse, "dq": dq, "dk": dk, "dv": dv}
    errs = C.compare(gpu, ref, dtype)
    print(f"  {errs}", flush=True)
    # the same through the mapped entry points
    gm = C.run_gpu_hash(fm, q.cuda(), k.cuda(), v.cuda(), do.cuda(), torch.from_numpy(qb).cuda(),
                        torch.from_numpy(kb).cuda(), nb, scale, mapped=True)
    print(f"  mapped {C.compare(gm, ref, dtype)}", flush=True)


def test_hash_end_to_end_with_lsh(fm):
    """The GPU hash feeds the GPU pipeline; the oracle hashes the same inputs itself. The seed gives no
    near ties, so both sides pick the same buckets and the attention must agree."""
    print("\nhash end to end with the GPU hash", flush=True)
    B, H, N, d, nb = 1, 2, 1200, 128, 8
    q, k, v, do = (torch.from_numpy(x).to(torch.bfloat16) for x in W.make_tensors(2, 102, B, H, N, d))
    R = W.make_rotation(2, 102, H, d, nb)
    Rd = torch.from_numpy(R).cuda()
    qb_g = fm.fm_lsh_buckets(q.cuda(), Rd, nb)
    kb_g = fm.fm_lsh_buckets(k.cuda(), Rd, nb)
    qb_o = np.stack([[OH.lsh_buckets(C.f64(q[b, h]), R[h].astype(np.float64)) for h in range(H)] for b in range(B)])
    kb_o = np.stack([[OH.lsh_buckets(C.f64(k[b, h]), R[h].astype(np.float64)) for h in range(H)] for b in range(B)])
    assert np.array_equal(qb_g.cpu().numpy(), qb_o) and np.array_equal(kb_g.cpu().numpy(), kb_o)
    gpu = C.run_gpu_hash(fm, q.cuda(), k.cuda(), v.cuda(), do.cuda(), qb_g, kb_g, nb, d ** -0.5)
    ref = OH.hash_attention(C.f64(q), C.f64(k), C.f64(v), C.f64(do), qb_o, kb_o, nb, d ** -0.5)
    C.compare(gpu, dict(zip(("out", "lse", "dq", "dk", "dv"), ref)), "bf16")


@pytest.mark.parametrize("name", list(W.HASH_WORKLOADS))
def test_hash_fullsize_sampled(fm, name):
    cfg_i, nb = W.HASH_WORKLOADS[name]
    cfg = W.CONFIGS[cfg_i]
    B, H, N, d = cfg.B, cfg.H, cfg.N, cfg.d
    print(f"\nfull-size hash {name}: B{B} H{H} N{N} d{d} nb{nb}", flush=True)
    host = W.make_tensors(cfg_i, W.HASH_MASK_INDEX, B, H, N, d)
    q, k, v, do = (torch.from_numpy(x).to(torch.bfloat16) for x in host)
    del host
    R = W.make_rotation(cfg_i, W.HASH_MASK_INDEX, H, d, nb)
    qd, kd = q.cuda(), k.cuda()
    qb_g = fm.fm_lsh_buckets(qd, torch.from_numpy(R).cuda(), nb).cpu().numpy()
    rng = np.random.default_rng(11)
    heads = sorted({(0, 0), (B - 1, H - 1)})
    for (b, h) in heads:
        rows = np.sort(rng.choice(N, size=256, replace=False))
        _check_lsh(qb_g[b, h, rows], C.f64(q[b, h, rows]), R[h].astype(np.float64))
    # attention from seeded buckets (not the GPU hash)
    qb, kb = W.make_buckets(cfg_i, W.HASH_MASK_INDEX, B, H, N, nb, 0.0)
    scale = d ** -0.5
    gpu = C.run_gpu_hash(fm, qd, kd, v.cuda(), do.cuda(), torch.from_numpy(qb).cuda(),
                         torch.from_numpy(kb).cuda(), nb, scale, mapped=True)
    del qd, kd
    torch.cuda.empty_cache()
    tol = C.TOL["bf16"]
    for (b, h) in heads:
        want = OH.bucket_sort(qb[b, h], kb[b, h], nb)
        got = [gpu["qidx"][b, h], gpu["qpos"][b, h], gpu["kidx"][b, h], gpu["kpos"][b, h]] + \
            [x[b, h] for x in gpu["vecs"]]
        for g, w in zip(got, want):
            assert np.array_equal(g.numpy(), w)
        qh, kh, vh, doh = (C.f64(x[b, h]) for x in (q, k, v, do))
        rows = np.unique(np.concatenate([[0, 1, N - 1], rng.choice(N, size=10, replace=False)]))
        r_out, r_lse, r_dq = OH.hash_rows_probe(qh, kh, vh, doh, qb[b, h], kb[b, h], nb, scale, rows)
        assert np.max(np.abs(C.f64(gpu["out"][b, h, rows]) - r_out)) <= tol["out"]
        g_lse = gpu["lse"][b, h, rows].double().numpy()
        fin = np.isfinite(r_lse)
        assert np.array_equal(fin, np.isfinite(g_lse))
        assert np.max(np.abs(g_lse[fin] - r_lse[fin]), initial=0.0) <= tol["lse"]
        assert C.rel_fro(C.f64(gpu["dq"][b, h, rows]), r_dq) <= tol["grad"]
        lo = max(0, N - 1024 * nb)  # columns attended by at most about 1024 rows
        cols = np.unique(np.concatenate([[N - 1], rng.integers(lo, N, size=4)]))
        r_dk, r_dv = OH.hash_cols_probe(qh, kh, vh, doh, qb[b, h], kb[b, h], nb, scale, cols)
        assert C.rel_fro(C.f64(gpu["dk"][b, h, cols]), r_dk) <= tol["grad"]
        assert C.rel_fro(C.f64(gpu["dv"][b, h, cols]), r_dv) <= tol["grad"]
        print(f"  head ({b},{h}) ok", flush=True)


def test_hash_pipeline_graph_replays(fm):
    """The whole hash pipeline, with the gathers back and with the mapped entry points, captured in a HIP
    graph (torch.cuda.CUDAGraph; the library allocates nothing and issues no memset): every replay, with
    eager work and synchronisations between replays, equals the eager run bitwise (the pipeline has no
    atomics)."""
    print("\nhash pipeline graph replays", flush=True)
    B, H, N, d, nb = 1, 2, 1500, 128, 8
    q, k, v, do = (torch.from_numpy(x).to(torch.bfloat16).cuda() for x in W.make_tensors(2, 103, B, H, N, d))
    R = torch.from_numpy(W.make_rotation(2, 103, H, d, nb)).cuda()
    scale = d ** -0.5

    def step():
        qb = fm.fm_lsh_buckets(q, R, nb)
        kb = fm.fm_lsh_buckets(k, R, nb)
        qidx, qpos, kidx, kpos, vecs = fm.fm_bucket_sort(qb, kb, nb)
        qs, dos = fm.fm_gather_rows(q, qidx), fm.fm_gather_rows(do, qidx)
        ks, vs = fm.fm_gather_rows(k, kidx), fm.fm_gather_rows(v, kidx)
        bounds = fm.fm_tile_bounds(*vecs, B, H, N)
        outs, lse = fm.fm_fwd(qs, ks, vs, *vecs, bounds=bounds, causal=False, scale=scale)
        dqs, dks, dvs = fm.fm_bwd(qs, ks, vs, outs, dos, lse, *vecs, bounds=bounds, causal=False, scale=scale)
        out_m, lse_m = fm.fm_fwd_mapped(qs, ks, vs, qidx, *vecs, bounds=bounds, causal=False, scale=scale)
        dq_m, dk_m, dv_m = fm.fm_bwd_mapped(qs, ks, vs, out_m, dos, lse_m, qidx, kidx, *vecs, bounds=bounds,
                                            causal=False, scale=scale)
        return [fm.fm_gather_rows(outs, qpos), fm.fm_gather_rows(dqs, qpos), fm.fm_gather_rows(dks, kpos),
                fm.fm_gather_rows(dvs, kpos), lse, qb, kb, out_m, lse_m, dq_m, dk_m, dv_m]

    eager = [t.clone() for t in step()]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm the allocator on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = step()
    for rep in range(3):
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, eager):
            assert torch.equal(a, b), rep
        junk = (q.float() * 2).sum()  # eager work between replays
        torch.cuda.synchronize()
        del junk


@pytest.mark.parametrize("dtype,d,nb,drop", [("bf16", 128, 8, 0.0), ("bf16", 64, 16, 0.1), ("bf16", 128, 3, 0.05),
                                              ("f32", 64, 5, 0.1), ("f32", 128, 8, 0.0)])
def test_mapped_outputs_equal_gathered(fm, dtype, d, nb, drop):
    """fm_fwd_mapped / fm_bwd_mapped store out, dq, dk, dv straight into the original order: bitwise equal to
    fm_fwd / fm_bwd on the reordered problem followed by the gathers back, and lse equal in sorted order;
    the same with the longest-first dispatch schedule."""
    print(f"\nmapped {dtype} d{d} nb{nb} drop{drop}", flush=True)
    B, H, N = 2, 3, 1000
    q, k, v, do = (torch.from_numpy(x).to(C.TORCH_DT[dtype]).cuda() for x in W.make_tensors(2, 200 + d, B, H, N, d))
    qb, kb = (torch.from_numpy(x).cuda() for x in W.make_buckets(2, 200 + nb, B, H, N, nb, drop))
    scale = d ** -0.5
    qidx, qpos, kidx, kpos, vecs = fm.fm_bucket_sort(qb, kb, nb)
    qs, dos = fm.fm_gather_rows(q, qidx), fm.fm_gather_rows(do, qidx)
    ks, vs = fm.fm_gather_rows(k, kidx), fm.fm_gather_rows(v, kidx)
    bounds = fm.fm_tile_bounds(*vecs, B, H, N)
    outs, lse = fm.fm_fwd(qs, ks, vs, *vecs, bounds=bounds, causal=False, scale=scale)
    dqs, dks, dvs = fm.fm_bwd(qs, ks, vs, outs, dos, lse, *vecs, bounds=bounds, causal=False, scale=scale)
    ref = {"out": fm.fm_gather_rows(outs, qpos), "dq": fm.fm_gather_rows(dqs, qpos),
           "dk": fm.fm_gather_rows(dks, kpos), "dv": fm.fm_gather_rows(dvs, kpos)}
    out_m, lse_m = fm.fm_fwd_mapped(qs, ks, vs, qidx, *vecs, bounds=bounds, causal=False, scale=scale)
    dq_m, dk_m, dv_m = fm.fm_bwd_mapped(qs, ks, vs, out_m, dos, lse_m, qidx, kidx, *vecs, bounds=bounds,
                                        causal=False, scale=scale)
    # a dispatch schedule changes only the order of the work units, never a result
    sched = fm.fm_tile_schedule(bounds, B, H, N, N, False, device=q.device)
    out_s, lse_s = fm.fm_fwd_mapped(qs, ks, vs, qidx, *vecs, bounds=bounds, sched=sched, causal=False, scale=scale)
    dq_s, dk_s, dv_s = fm.fm_bwd_mapped(qs, ks, vs, out_s, dos, lse_s, qidx, kidx, *vecs, bounds=bounds,
                                        sched=sched, causal=False, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(lse_m, lse) and torch.equal(lse_s, lse)
    for name, got, got_s in (("out", out_m, out_s), ("dq", dq_m, dq_s), ("dk", dk_m, dk_s), ("dv", dv_m, dv_s)):
        assert torch.equal(got, ref[name]), name
        assert torch.equal(got_s, ref[name]), name + " (scheduled)"


def test_mapped_out_of_range_entries_write_nothing(fm):
    """A map entry outside [0, N) drops its row: the original rows it would have named keep their previous
    contents, and every other row equals the run with the full permutation."""
    print("\nmapped out-of-range entries", flush=True)
    B, H, N, d, nb = 1, 2, 700, 128, 4
    q, k, v, do = (torch.from_numpy(x).to(torch.bfloat16).cuda() for x in W.make_tensors(2, 301, B, H, N, d))
    qb, kb = (torch.from_numpy(x).cuda() for x in W.make_buckets(2, 301, B, H, N, nb, 0.0))
    qidx, qpos, kidx, kpos, vecs = fm.fm_bucket_sort(qb, kb, nb)
    qs, dos = fm.fm_gather_rows(q, qidx), fm.fm_gather_rows(do, qidx)
    ks, vs = fm.fm_gather_rows(k, kidx), fm.fm_gather_rows(v, kidx)
    bounds = fm.fm_tile_bounds(*vecs, B, H, N)
    out, lse = fm.fm_fwd_mapped(qs, ks, vs, qidx, *vecs, bounds=bounds, causal=False)
    dq, dk, dv = fm.fm_bwd_mapped(qs, ks, vs, out, dos, lse, qidx, kidx, *vecs, bounds=bounds, causal=False)
    rng = np.random.default_rng(5)
    drop_q = torch.from_numpy(rng.random((B, H, N)) < 0.2).cuda()
    drop_k = torch.from_numpy(rng.random((B, H, N)) < 0.2).cuda()
    qmap = torch.where(drop_q, torch.full_like(qidx, -1), qidx)
    qmap = torch.where(drop_q & (torch.arange(N, device="cuda") % 2 == 0), torch.full_like(qidx, N + 7), qmap)
    kmap = torch.where(drop_k, torch.full_like(kidx, -3), kidx)
    sentinel = torch.full_like(out, 7.0)
    out2, lse2 = fm.fm_fwd_mapped(qs, ks, vs, qmap, *vecs, bounds=bounds, causal=False, out=sentinel.clone())
    torch.cuda.synchronize()
    assert torch.equal(lse2, lse)
    # original rows named only by dropped entries keep the sentinel; the others equal the full run
    hit_q = torch.zeros((B, H, N + 1), dtype=torch.bool, device="cuda")  # column N collects the dropped entries
    hit_q.scatter_(2, torch.where(drop_q, torch.full_like(qidx, N), qidx).long(), True)
    hit_q = hit_q[..., :N]
    assert torch.equal(out2[hit_q], out[hit_q]) and torch.all(out2[~hit_q] == 7.0)
    # the backward with the full qmap (out as the full forward wrote it) and a kmap with dropped entries
    dq2, dk2, dv2 = fm.fm_bwd_mapped(qs, ks, vs, out, dos, lse, qidx, kmap, *vecs, bounds=bounds, causal=False,
                                     dq=torch.full_like(dq, 7.0), dk=torch.full_like(dk, 7.0),
                                     dv=torch.full_like(dv, 7.0))
    torch.cuda.synchronize()
    hit_k = torch.zeros((B, H, N + 1), dtype=torch.bool, device="cuda")
    hit_k.scatter_(2, torch.where(drop_k, torch.full_like(kidx, N), kidx).long(), True)
    hit_k = hit_k[..., :N]
    assert torch.equal(dq2, dq)
    assert torch.equal(dk2[hit_k], dk[hit_k]) and torch.all(dk2[~hit_k] == 7.0)
    assert torch.equal(dv2[hit_k], dv[hit_k]) and torch.all(dv2[~hit_k] == 7.0)
    # the backward with dropped qmap entries: a dropped query row contributes nothing to dk and dv, which
    # equal (bit for bit) the full-map run with those rows' dout set to zero; the dq rows named only by
    # dropped entries keep their previous contents and every other dq row equals the full run's
    dq3, dk3, dv3 = fm.fm_bwd_mapped(qs, ks, vs, out, dos, lse, qmap, kidx, *vecs, bounds=bounds, causal=False,
                                     dq=torch.full_like(dq, 7.0))
    dos0 = torch.where(drop_q[..., None], torch.zeros_like(dos), dos)
    dq4, dk4, dv4 = fm.fm_bwd_mapped(qs, ks, vs, out, dos0, lse, qidx, kidx, *vecs, bounds=bounds, causal=False)
    torch.cuda.synchronize()
    assert torch.equal(dk3, dk4) and torch.equal(dv3, dv4)
    assert torch.equal(dq3[hit_q], dq4[hit_q]) and torch.all(dq3[~hit_q] == 7.0)
