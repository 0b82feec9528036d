"""GPU checks of the stored-dS backward (fm_bwd_plan, fm_bwd_ds) through the C ABI: the plan bit-exact
against the oracle's bookkeeping, gradients within the bars against the fp64 oracle, dk and dv bitwise
equal to fm_bwd's (the same key-parallel pass), heads that do not fit in the workspace falling back to
fm_bwd's dq bit for bit, and the stored tiles themselves against the oracle's dS."""
import numpy as np
import pytest
import torch

from oracle import attention as OA
from oracle import dstore as OD
from oracle import masks as OM
from tests import fmcase as C

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mask_aware_exact_amd as m
    m.load_library()
    return m


def read_plan(plan: torch.Tensor, B, H, Hm, N):
    """The plan's fields, decoded from the layout the plan call writes (int64 total at byte 0, region
    [B*H] int64 at byte 16, then base [B*Hm*nkt] and rowtotal [B*Hm] int64, then first [B*Hm*nkt] int32)."""
    raw = plan.cpu().numpy()
    nkt = -(-N // 128)
    rows = B * Hm
    i64 = lambda off, n: raw[off:off + 8 * n].view(np.int64)  # noqa: E731
    total = int(i64(0, 1)[0])
    off = 16
    region = i64(off, B * H).reshape(B, H)
    off += 8 * B * H
    base = i64(off, rows * nkt).reshape(B, Hm, nkt)
    off += 8 * rows * nkt
    rowtotal = i64(off, rows).reshape(B, Hm)
    off += 8 * rows
    first = raw[off:off + 4 * rows * nkt].view(np.int32).reshape(B, Hm, nkt)
    return {"total": total, "region": region, "base": base, "rowtotal": rowtotal, "first": first}


def run_ds(case, fm, dev="cuda", cache_tiles=None):
    """fm_tile_bounds -> fm_bwd_plan -> fm_fwd -> fm_bwd_ds (and fm_bwd on the same inputs)."""
    q, k, v, do = (t.to(dev) for t in (case.q, case.k, case.v, case.do))
    vecs = C.device_vectors(case.spec, dev)
    Hm = case.spec.Hm
    bounds = fm.fm_tile_bounds(*vecs, case.B, Hm, case.N) if any(x is not None for x in vecs) else None
    plan = fm.fm_bwd_plan(bounds, case.B, case.H, Hm, case.N, case.spec.causal, device=torch.device(dev))
    tiles = fm.plan_tiles(plan) if cache_tiles is None else cache_tiles
    ws = torch.empty(fm.fm_bwd_ds_workspace_bytes(q.dtype, case.B, case.H, case.N, case.d, tiles),
                     dtype=torch.uint8, device=dev)
    out, lse = fm.fm_fwd(q, k, v, *vecs, bounds=bounds, causal=case.spec.causal, scale=case.scale)
    dq, dk, dv = fm.fm_bwd_ds(q, k, v, out, do, lse, plan, *vecs, bounds=bounds, causal=case.spec.causal,
                              scale=case.scale, workspace=ws)
    dq0, dk0, dv0 = fm.fm_bwd(q, k, v, out, do, lse, *vecs, bounds=bounds, causal=case.spec.causal,
                              scale=case.scale)
    torch.cuda.synchronize()
    res = {"out": out, "lse": lse, "dq": dq, "dk": dk, "dv": dv, "dq0": dq0, "dk0": dk0, "dv0": dv0,
           "plan": plan, "ws": ws}
    return {k_: t.cpu() for k_, t in res.items()}


CASES = [
    (0, "causal_document", 1, 2, 256, 64),
    (1, "full", 2, 3, 520, 64),
    (1, "causal", 2, 3, 520, 64),
    (2, "causal_document", 1, 4, 1000, 128),
    (2, "causal_window_1024", 1, 3, 2600, 128),
    (3, "share_question", 1, 3, 1500, 128),
    (3, "prefix_lm", 1, 3, 1100, 128),
    (3, "causal_key_drop", 1, 4, 1300, 128),
    (4, "causal_document", 1, 2, 2500, 128),
    (4, "causal_document_window_4096", 1, 2, 2500, 128),
    (4, "causal_document_block_sparse", 1, 2, 2500, 128),
    (3, "causal_key_drop", 2, 2, 777, 64),
    (1, "bidirectional_document", 2, 2, 700, 64),
    (1, "causal_by_vectors", 1, 2, 333, 128),
]


@pytest.mark.parametrize("cfg,mask,B,H,N,d", CASES, ids=lambda x: str(x))
def test_plan_and_parity(fm, cfg, mask, B, H, N, d):
    case = C.make_case(cfg, mask, B, H, N, d, "bf16")
    print(f"\ncase {case.name}", flush=True)
    gpu = run_ds(case, fm)
    spec = case.spec
    ref_plan = OD.plan(spec.vectors(), spec.causal, B, H, spec.Hm, N)
    got = read_plan(gpu["plan"], B, H, spec.Hm, N)
    assert got["total"] == ref_plan["total"]
    for key in ("region", "base", "rowtotal", "first"):
        assert np.array_equal(got[key], ref_plan[key]), key
    report = {}
    C.compare(gpu, C.run_oracle(case), "bf16", report)
    # the key-parallel pass is the same kernel as fm_bwd's, with D from the same code
    assert torch.equal(gpu["dk"], gpu["dk0"]) and torch.equal(gpu["dv"], gpu["dv0"])
    print(report, "tiles", got["total"], flush=True)


@pytest.mark.parametrize("N", [1, 63, 64, 65, 129, 200])
def test_tiny_sizes(fm, N):
    case = C.make_case(2, "causal_document", 1, 2, N, 128, "bf16")
    gpu = run_ds(case, fm)
    C.compare(gpu, C.run_oracle(case), "bf16")
    assert torch.equal(gpu["dk"], gpu["dk0"]) and torch.equal(gpu["dv"], gpu["dv0"])


@pytest.mark.parametrize("fit_heads", [0, 1, 3])
def test_partial_cache(fm, fit_heads):
    """A workspace with room for the first fit_heads heads only: those stream their dq, the others run the
    recomputing pass; every head meets the bars and the others' dq equals fm_bwd's bit for bit."""
    case = C.make_case(2, "causal_document", 1, 4, 1000, 128, "bf16")
    spec = case.spec
    ref_plan = OD.plan(spec.vectors(), spec.causal, 1, 4, spec.Hm, case.N)
    region = ref_plan["region"][0]
    cap = int(region[fit_heads]) if fit_heads < 4 else ref_plan["total"]
    gpu = run_ds(case, fm, cache_tiles=cap)
    C.compare(gpu, C.run_oracle(case), "bf16")
    for h in range(fit_heads, 4):
        assert torch.equal(gpu["dq"][0, h], gpu["dq0"][0, h]), h
    assert torch.equal(gpu["dk"], gpu["dk0"]) and torch.equal(gpu["dv"], gpu["dv0"])


def test_stored_tiles_match_oracle_ds(fm):
    """The cache of one head, tile by tile, against the oracle's dS in the documented storage order."""
    case = C.make_case(3, "share_question", 1, 2, 700, 128, "bf16")
    gpu = run_ds(case, fm)
    spec = case.spec
    N, h = case.N, 1
    p = OD.plan(spec.vectors(), spec.causal, 1, 2, spec.Hm, N)
    D_bytes = -(-(1 * 2 * N * 4) // 256) * 256
    cache = gpu["ws"][D_bytes:].view(torch.bfloat16).to(torch.float64).numpy()
    q, k, v, do = (C.f64(t[0, h]) for t in (case.q, case.k, case.v, case.do))
    masked = OM.dense_masked_rows(*spec.column_slice(0, h), spec.causal, N, 0, N)
    ds = OA.attend_rows(q, k, v, do, masked, case.scale)["dS"]
    got, ref = [], []
    for kt in range(-(-N // 128)):
        first, span = int(p["first"][0, 0, kt]), 0
        nb = int(p["base"][0, 0, kt + 1]) if kt + 1 < p["base"].shape[2] else int(p["rowtotal"][0, 0])
        span = nb - int(p["base"][0, 0, kt])
        for r in range(span):
            slot = int(p["region"][0, h] + p["base"][0, 0, kt] + r)
            qt = first + r
            if masked[qt * 64:(qt + 1) * 64, kt * 128:(kt + 1) * 128].all():
                continue  # a fully masked tile inside the span keeps an unused slot
            got.append(cache[slot * 8192:(slot + 1) * 8192])
            ref.append(OD.tile_values(ds, qt, kt))
    got, ref = np.concatenate(got), np.concatenate(ref)
    err = C.rel_fro(got, ref)
    print(f"stored dS rel-F {err:.3g} over {got.size} values", flush=True)
    assert err <= 2e-2
