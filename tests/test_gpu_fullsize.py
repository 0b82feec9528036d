"""GPU parity at the workloads' full sizes, in the launch configuration bench.py times.

The oracle cannot run the whole of these sizes, so it checks sampled outputs one by one (query rows:
out, lse, dq; key columns: dk, dv, evaluated from every row that attends them) and the gradient
invariants that hold at any size on the full tensors: sum_j dV_j = sum over live rows of dO_i and
sum_j dK_j = 0 per head (sum_j P_ij = 1 and sum_j dS_ij = 0). Bounds are compared bit-exactly."""
import math
import os
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from oracle import attention as OA  # noqa: E402
from oracle import masks as OM  # noqa: E402
from oracle import tiles as OT  # noqa: E402
from tests import fmcase as C  # noqa: E402

pytestmark = pytest.mark.gpu

WORKLOADS = [name for name in bench.WORKLOADS]


@pytest.fixture(scope="module")
def fm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mask_aware_exact_amd as m
    m.load_library()
    return m


def _pick_rows(spec, b, h, N, rng):
    rows = {0, 1, N - 1, N // 2}
    p = spec.params
    for key in ("bounds", "answer_bounds"):
        if key in p:
            for s in np.asarray(p[key])[1:-1][:3]:
                rows.update({int(s) - 1, int(s)})
    rows.update(int(x) for x in rng.integers(0, N, size=6))
    return np.array(sorted(r for r in rows if 0 <= r < N))


def _pick_cols(vecs, causal, N, rng, budget=3072, want=4):
    cands = sorted(set(int(x) for x in rng.integers(0, N, size=48)) | {N - 1, N - 2, N - 100})
    picked = []
    for j in cands:
        if not (0 <= j < N):
            continue
        n = int((~OM.dense_masked_rows(*vecs, causal, N, 0, N, j, j + 1)).sum())
        if 0 < n <= budget:
            picked.append((n, j))
    picked.sort(reverse=True)  # prefer the most-attended columns within the budget
    return np.array(sorted(j for _, j in picked[:want]), dtype=np.int64)


@pytest.mark.parametrize("name", WORKLOADS)
def test_fullsize_sampled_parity(fm, name):
    print(f"\nworkload {name}", flush=True)
    dev = torch.device("cuda:0")
    wl = bench.Workload(name, dev)
    b = fm.fm_tile_bounds(*wl.vecs, wl.B, wl.spec.Hm, wl.N) if wl.has_vecs else None
    out, lse = fm.fm_fwd(wl.q, wl.k, wl.v, *wl.vecs, bounds=b, causal=wl.spec.causal, scale=wl.scale)
    dq, dk, dv = fm.fm_bwd(wl.q, wl.k, wl.v, out, wl.do, lse, *wl.vecs, bounds=b, causal=wl.spec.causal,
                           scale=wl.scale)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(dq.float()).all()
    assert torch.isfinite(dk.float()).all() and torch.isfinite(dv.float()).all()
    if b is not None:
        assert np.array_equal(b.cpu().numpy(), OT.tile_bounds(wl.spec.vectors(), wl.B, wl.spec.Hm, wl.N))

    rng = np.random.default_rng(abs(hash(name)) % (2 ** 32))
    heads = sorted({(0, 0), (wl.B - 1, wl.H - 1), (0, wl.H // 2)})
    N, tol = wl.N, C.TOL["bf16"]
    q_h, k_h, v_h, do_h = wl.host
    for (bb, hh) in heads:
        vecs = wl.spec.column_slice(bb, hh)
        f64 = lambda x: torch.from_numpy(np.ascontiguousarray(x[bb, hh])).to(torch.bfloat16).to(  # noqa: E731
            torch.float64).numpy()
        q, k, v, do = f64(q_h), f64(k_h), f64(v_h), f64(do_h)
        rows = _pick_rows(wl.spec, bb, hh, N, rng)
        r_out, r_lse, _, r_dq = OA.rows_probe(q, k, v, do, vecs, wl.spec.causal, wl.scale, rows)
        g_out = out[bb, hh, rows].double().cpu().numpy()
        g_lse = lse[bb, hh, rows].double().cpu().numpy()
        g_dq = dq[bb, hh, rows].double().cpu().numpy()
        assert np.max(np.abs(g_out - r_out)) <= tol["out"], (bb, hh)
        fin = np.isfinite(r_lse)
        assert np.array_equal(fin, np.isfinite(g_lse))
        assert np.max(np.abs(g_lse[fin] - r_lse[fin]), initial=0.0) <= tol["lse"]
        assert C.rel_fro(g_dq, r_dq) <= tol["grad"], C.rel_fro(g_dq, r_dq)
        cols = _pick_cols(vecs, wl.spec.causal, N, rng)
        if cols.size:
            r_dk, r_dv = OA.cols_probe(q, k, v, do, vecs, wl.spec.causal, wl.scale, cols)
            g_dk = dk[bb, hh, cols].double().cpu().numpy()
            g_dv = dv[bb, hh, cols].double().cpu().numpy()
            assert C.rel_fro(g_dk, r_dk) <= tol["grad"], C.rel_fro(g_dk, r_dk)
            assert C.rel_fro(g_dv, r_dv) <= tol["grad"], C.rel_fro(g_dv, r_dv)
        # invariants over the whole head
        live = np.isfinite(lse[bb, hh].double().cpu().numpy())
        dv_sum = dv[bb, hh].double().sum(dim=0).cpu().numpy()
        do_live = do[live].sum(axis=0)
        assert np.linalg.norm(dv_sum - do_live) <= 2e-2 * max(np.linalg.norm(do_live), 1.0)
        dk_full = dk[bb, hh].double()
        assert float(dk_full.sum(dim=0).norm()) <= 2e-2 * max(float(dk_full.norm()), 1e-6)
        print(f"  head ({bb},{hh}): rows {rows.size} cols {cols.size} ok", flush=True)
    del wl
    torch.cuda.empty_cache()


def test_fullsize_key_drop_compacted(fm):
    """The key-drop workload at full size through key compaction (fm_compact_keys, fm_gather_rows, the
    attention without the causal flag, fm_gather_rows back): sampled rows and columns against the
    oracle on the original problem, and the gradient invariants."""
    name = "dpo_rm_causal_key_drop"
    print(f"\nworkload {name} (compacted)", flush=True)
    dev = torch.device("cuda:0")
    wl = bench.Workload(name, dev)
    Hm = wl.spec.Hm
    kidx, kpos, counts, vecs2 = fm.fm_compact_keys(*wl.vecs, wl.B, Hm, wl.N, wl.spec.causal)
    k2, v2 = fm.fm_gather_rows(wl.k, kidx), fm.fm_gather_rows(wl.v, kidx)
    b2 = fm.fm_tile_bounds(*vecs2, wl.B, Hm, wl.N)
    out, lse = fm.fm_fwd(wl.q, k2, v2, *vecs2, bounds=b2, causal=False, scale=wl.scale)
    dq, dk2, dv2 = fm.fm_bwd(wl.q, k2, v2, out, wl.do, lse, *vecs2, bounds=b2, causal=False, scale=wl.scale)
    dk, dv = fm.fm_gather_rows(dk2, kpos), fm.fm_gather_rows(dv2, kpos)
    torch.cuda.synchronize()
    assert int(counts.min()) >= 0
    del k2, v2, dk2, dv2
    rng = np.random.default_rng(5)
    N, tol = wl.N, C.TOL["bf16"]
    q_h, k_h, v_h, do_h = wl.host
    for (bb, hh) in sorted({(0, 0), (wl.B - 1, wl.H - 1)}):
        vecs = wl.spec.column_slice(bb, hh)
        f64 = lambda x: torch.from_numpy(np.ascontiguousarray(x[bb, hh])).to(torch.bfloat16).to(  # noqa: E731
            torch.float64).numpy()
        q, k, v, do = f64(q_h), f64(k_h), f64(v_h), f64(do_h)
        rows = _pick_rows(wl.spec, bb, hh, N, rng)
        r_out, r_lse, _, r_dq = OA.rows_probe(q, k, v, do, vecs, wl.spec.causal, wl.scale, rows)
        assert np.max(np.abs(out[bb, hh, rows].double().cpu().numpy() - r_out)) <= tol["out"]
        g_lse = lse[bb, hh, rows].double().cpu().numpy()
        fin = np.isfinite(r_lse)
        assert np.array_equal(fin, np.isfinite(g_lse))
        assert np.max(np.abs(g_lse[fin] - r_lse[fin]), initial=0.0) <= tol["lse"]
        assert C.rel_fro(dq[bb, hh, rows].double().cpu().numpy(), r_dq) <= tol["grad"]
        cols = _pick_cols(vecs, wl.spec.causal, N, rng)
        if cols.size:
            r_dk, r_dv = OA.cols_probe(q, k, v, do, vecs, wl.spec.causal, wl.scale, cols)
            assert C.rel_fro(dk[bb, hh, cols].double().cpu().numpy(), r_dk) <= tol["grad"]
            assert C.rel_fro(dv[bb, hh, cols].double().cpu().numpy(), r_dv) <= tol["grad"]
        dropped = kpos[bb, hh if Hm > 1 else 0].cpu().numpy() < 0
        assert float(dk[bb, hh][torch.from_numpy(dropped).to(dev)].abs().max()) == 0.0
        live = np.isfinite(lse[bb, hh].double().cpu().numpy())
        dv_sum = dv[bb, hh].double().sum(dim=0).cpu().numpy()
        do_live = do[live].sum(axis=0)
        assert np.linalg.norm(dv_sum - do_live) <= 2e-2 * max(np.linalg.norm(do_live), 1.0)
        print(f"  head ({bb},{hh}): rows {rows.size} cols {cols.size} ok", flush=True)
    del wl
    torch.cuda.empty_cache()
