"""GPU parity of the longest-first dispatch schedule (fm_tile_schedule) and of the kernels that read it.

The schedule is integer work: orders and per-unit work are compared bit-exactly with the oracle. A
schedule only reorders independent work units, so fm_fwd / fm_bwd with it must give results bitwise
equal to the runs without it; one case is also held to the oracle's bars directly. At the workloads'
full sizes the oracle computes sampled units' work one by one, and the orders are checked by their
defining properties (a permutation, work non-increasing, equal work in the default order)."""
import os
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as W  # noqa: E402
from oracle import schedule as OS  # noqa: E402
from tests import fmcase as C  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mask_aware_exact_amd as m
    m.load_library()
    return m


CASES = [
    # (cfg, mask, B, H, N)
    (0, "causal_document", 1, 2, 256),
    (2, "causal_document", 2, 2, 1000),
    (2, "causal_window_1024", 1, 2, 2049),
    (3, "share_question", 1, 2, 1536),
    (3, "prefix_lm", 1, 2, 777),
    (3, "causal_key_drop", 2, 3, 1100),
    (4, "causal_document_block_sparse", 1, 2, 3000),
    (4, "causal_document_window_4096", 1, 2, 2500),
    (1, "causal", 2, 2, 640),
    (1, "full", 1, 2, 300),
    (2, "bidirectional_document", 1, 2, 900),
]


def _schedule(fm, spec, Nq, Nk, q_off=0):
    vecs = C.device_vectors(spec)
    bounds = fm.fm_tile_bounds(*vecs, spec.B, spec.Hm, Nk) if any(x is not None for x in vecs) else None
    s = fm.fm_tile_schedule(bounds, spec.B, spec.Hm, Nq, Nk, spec.causal, q_off)
    return vecs, bounds, s


def _check_against_oracle(fm, spec, s, Nq, Nk, q_off=0):
    qo, ko, qc, kc = (x.cpu().numpy() for x in fm.split_schedule(s, Nq, Nk))
    oqo, oko, oqc, okc = OS.schedule(spec.vectors(), spec.causal, spec.B, spec.Hm, Nq, Nk, q_off)
    assert np.array_equal(qc, oqc), "query-unit work"
    assert np.array_equal(kc, okc), "key-unit work"
    assert np.array_equal(qo, oqo), "query-unit order"
    assert np.array_equal(ko, oko), "key-unit order"


@pytest.mark.parametrize("cfg,mask,B,H,N", CASES)
def test_schedule_matches_oracle(fm, cfg, mask, B, H, N):
    print(f"\nschedule cfg{cfg} {mask} B{B} H{H} N{N}", flush=True)
    spec = W.make_mask(cfg, mask, B, H, N)
    _, _, s = _schedule(fm, spec, N, N)
    torch.cuda.synchronize()
    _check_against_oracle(fm, spec, s, N, N)


@pytest.mark.parametrize("q_off,Nq", [(0, 300), (256, 500), (700, 1348), (1983, 65)])
def test_row_block_schedule_matches_oracle(fm, q_off, Nq):
    print(f"\nrow-block schedule q_off {q_off} Nq {Nq}", flush=True)
    N = 2048
    for mask in ("causal_document", "share_question", "prefix_lm"):
        spec = W.make_mask(3 if mask != "causal_document" else 2, mask, 1, 2, N)
        _, _, s = _schedule(fm, spec, Nq, N, q_off)
        torch.cuda.synchronize()
        _check_against_oracle(fm, spec, s, Nq, N, q_off)


def _run(fm, case, bounds, sched):
    q, k, v, do = (t.cuda() for t in (case.q, case.k, case.v, case.do))
    vecs = C.device_vectors(case.spec)
    out, lse = fm.fm_fwd(q, k, v, *vecs, bounds=bounds, sched=sched, causal=case.spec.causal, scale=case.scale)
    dq, dk, dv = fm.fm_bwd(q, k, v, out, do, lse, *vecs, bounds=bounds, sched=sched, causal=case.spec.causal,
                           scale=case.scale)
    torch.cuda.synchronize()
    return {"out": out.cpu(), "lse": lse.cpu(), "dq": dq.cpu(), "dk": dk.cpu(), "dv": dv.cpu()}


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("cfg,mask,B,H,N", [c for c in CASES if c[4] <= 2100])
def test_scheduled_results_bitwise_equal(fm, cfg, mask, B, H, N, dtype):
    d = 128 if dtype == "bf16" else 64
    print(f"\nscheduled run cfg{cfg} {mask} B{B} H{H} N{N} d{d} {dtype}", flush=True)
    case = C.make_case(cfg, mask, B, H, N, d, dtype)
    _, bounds, s = _schedule(fm, case.spec, N, N)
    plain = _run(fm, case, bounds, None)
    sched = _run(fm, case, bounds, s)
    for name in plain:
        assert torch.equal(plain[name], sched[name]), name


@pytest.mark.parametrize("cfg,mask,B,H,N", [c for c in CASES if c[4] <= 2600])
def test_scheduled_stored_ds_bitwise_equal(fm, cfg, mask, B, H, N):
    """fm_bwd_ds with the schedule (its dK/dV units and the D pass in longest-first order) against the same
    call without: the stored-dS backward only reorders independent units, so dq, dk and dv are equal bit
    for bit."""
    print(f"\nscheduled stored-dS cfg{cfg} {mask} B{B} H{H} N{N}", flush=True)
    case = C.make_case(cfg, mask, B, H, N, 128, "bf16")
    vecs, bounds, s = _schedule(fm, case.spec, N, N)
    q, k, v, do = (t.cuda() for t in (case.q, case.k, case.v, case.do))
    plan = fm.fm_bwd_plan(bounds, B, H, case.spec.Hm, N, case.spec.causal, device=torch.device("cuda"))
    ws = torch.empty(fm.fm_bwd_ds_workspace_bytes(q.dtype, B, H, N, 128, fm.plan_tiles(plan)), dtype=torch.uint8,
                     device="cuda")
    out, lse = fm.fm_fwd(q, k, v, *vecs, bounds=bounds, causal=case.spec.causal, scale=case.scale)
    res = []
    for sched in (None, s):
        grads = fm.fm_bwd_ds(q, k, v, out, do, lse, plan, *vecs, bounds=bounds, sched=sched,
                             causal=case.spec.causal, scale=case.scale, workspace=ws)
        torch.cuda.synchronize()
        res.append([t.cpu() for t in grads])
    for name, a, b in zip(("dq", "dk", "dv"), res[0], res[1]):
        assert torch.equal(a, b), name


def test_scheduled_parity_against_oracle(fm):
    print("\nscheduled parity cfg2 causal_document N1000", flush=True)
    case = C.make_case(2, "causal_document", 2, 2, 1000, 128, "bf16")
    _, bounds, s = _schedule(fm, case.spec, 1000, 1000)
    C.compare(_run(fm, case, bounds, s), C.run_oracle(case), "bf16")


def test_out_of_range_schedule_does_nothing(fm):
    # every entry -1: each workgroup finds no unit and returns, leaving the outputs as they were
    print("\nout-of-range schedule", flush=True)
    case = C.make_case(2, "causal_document", 1, 2, 700, 128, "bf16")
    q, k, v = (t.cuda() for t in (case.q, case.k, case.v))
    vecs = C.device_vectors(case.spec)
    bounds = fm.fm_tile_bounds(*vecs, 1, 1, 700)
    s = torch.full((fm.fm_schedule_elems(1, 1, 700, 700),), -1, dtype=torch.int32, device="cuda")
    out = torch.full_like(q, 7.0)
    lse = torch.full((1, 2, 700), 3.0, dtype=torch.float32, device="cuda")
    fm.fm_fwd(q, k, v, *vecs, bounds=bounds, sched=s, causal=True, out=out, lse=lse)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()) and bool((lse == 3.0).all())


def _check_order_properties(order, work, key: bool):
    n = len(work)
    assert sorted(order.tolist()) == list(range(n))
    w = work[order]
    assert np.all(np.diff(w) <= 0)
    # equal work keeps the default order: key units ascending, query units descending
    same = np.diff(w) == 0
    step = np.diff(order)
    assert np.all(step[same] > 0) if key else np.all(step[same] < 0)


@pytest.mark.parametrize("name", list(bench.WORKLOADS))
def test_fullsize_schedule_sampled(fm, name):
    print(f"\nfull-size schedule {name}", flush=True)
    wl = bench.Workload(name, torch.device("cuda:0"))
    spec, N = wl.spec, wl.N
    bounds = fm.fm_tile_bounds(*wl.vecs, wl.B, spec.Hm, N) if wl.has_vecs else None
    s = fm.fm_tile_schedule(bounds, wl.B, spec.Hm, N, N, spec.causal)
    qo, ko, qc, kc = (x.cpu().numpy() for x in fm.split_schedule(s, N, N))
    rng = np.random.default_rng(7)
    rows = sorted({(0, 0), (wl.B - 1, spec.Hm - 1)})
    for b, h in rows:
        _check_order_properties(qo[b, h], qc[b, h], key=False)
        _check_order_properties(ko[b, h], kc[b, h], key=True)
        v = [None if x is None else x[b, h] for x in spec.vectors()]
        b64, b128 = OS.unit_bounds(*v, N)
        nq, nk = qc.shape[-1], kc.shape[-1]
        for qt in sorted(set(rng.integers(0, nq, size=6).tolist()) | {0, nq - 1}):
            assert qc[b, h, qt] == OS.query_unit_work(b64, spec.causal, N, N, 0, qt), ("query unit", b, h, qt)
        for kt in sorted(set(rng.integers(0, nk, size=6).tolist()) | {0, nk - 1}):
            assert kc[b, h, kt] == OS.key_unit_work(b128, spec.causal, N, N, 0, kt), ("key unit", b, h, kt)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_scheduled_row_blocks_bitwise_equal(fm, dtype, d):
    """fm_fwd_rows / fm_bwd_rows with the row block's own schedule give the results of the default order."""
    N = 1800
    case = C.make_case(2, "causal_document", 1, 2, N, d, dtype)
    print(f"\nscheduled row blocks {case.name}", flush=True)
    vecs = C.device_vectors(case.spec)
    bounds = fm.fm_tile_bounds(*vecs, 1, 1, N)
    k, v = case.k.cuda(), case.v.cuda()
    for a, b in ((0, 700), (700, 1333), (1333, N)):
        q = case.q[:, :, a:b].contiguous().cuda()
        do = case.do[:, :, a:b].contiguous().cuda()
        s = fm.fm_tile_schedule(bounds, 1, 1, b - a, N, True, a)
        runs = []
        for sc in (None, s):
            out, lse = fm.fm_fwd_rows(q, k, v, a, *vecs, bounds=bounds, sched=sc, causal=True, scale=case.scale)
            dq, dk, dv = fm.fm_bwd_rows(q, k, v, out, do, lse, a, *vecs, bounds=bounds, sched=sc, causal=True,
                                        scale=case.scale)
            torch.cuda.synchronize()
            runs.append([t.cpu() for t in (out, lse, dq, dk, dv)])
        for x, y in zip(*runs):
            assert torch.equal(x, y), (a, b)
