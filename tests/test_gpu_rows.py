"""GPU parity of the row-block entry points (fm_fwd_rows, fm_bwd_rows): one rank's query rows against all
keys with the mask read in global row coordinates (FlashMask-3 summary, readmex.ai: zero-communication
mask localisation under context parallelism). Each block is checked against the oracle's row-block form,
and the blocks of a partition are checked to reassemble the whole problem."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as OA
from tests import fmcase as C

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mask_aware_exact_amd as m
    m.load_library()
    return m


def _oracle_rows(case, a, b):
    """Row-block oracle over every head of the case for rows [a, b)."""
    B, H, d = case.B, case.H, case.d
    Nk = case.N
    ref = {"out": np.zeros((B, H, b - a, d)), "lse": np.zeros((B, H, b - a)), "dq": np.zeros((B, H, b - a, d)),
           "dk": np.zeros((B, H, Nk, d)), "dv": np.zeros((B, H, Nk, d))}
    for bb in range(B):
        for hh in range(H):
            vecs = case.spec.column_slice(bb, hh)
            q, k, v, do = (C.f64(t[bb, hh]) for t in (case.q, case.k, case.v, case.do))
            o, l_, gq, gk, gv = OA.fwd_bwd_rows_head(q[a:b], k, v, do[a:b], vecs, case.spec.causal, case.scale, a)
            ref["out"][bb, hh], ref["lse"][bb, hh], ref["dq"][bb, hh] = o, l_, gq
            ref["dk"][bb, hh], ref["dv"][bb, hh] = gk, gv
    return ref


def _gpu_rows(fm, case, a, b, vecs, bounds):
    q = case.q[:, :, a:b].contiguous().cuda()
    do = case.do[:, :, a:b].contiguous().cuda()
    k, v = case.k.cuda(), case.v.cuda()
    out, lse = fm.fm_fwd_rows(q, k, v, a, *vecs, bounds=bounds, causal=case.spec.causal, scale=case.scale)
    dq, dk, dv = fm.fm_bwd_rows(q, k, v, out, do, lse, a, *vecs, bounds=bounds, causal=case.spec.causal,
                                scale=case.scale)
    torch.cuda.synchronize()
    return {"out": out.cpu(), "lse": lse.cpu(), "dq": dq.cpu(), "dk": dk.cpu(), "dv": dv.cpu()}


# (cfg, family, B, H, N, d, dtype, row-block boundaries)
CASES = [
    (2, "causal_document", 1, 2, 2600, 128, "bf16", (0, 700, 1999, 2600)),
    (3, "prefix_lm", 1, 2, 1500, 128, "bf16", (0, 512, 1500)),
    (3, "causal_key_drop", 1, 3, 1300, 128, "bf16", (0, 1, 640, 1300)),
    (3, "share_question", 1, 2, 1100, 64, "bf16", (0, 333, 1100)),
    (4, "causal_document_window_4096", 1, 2, 2000, 128, "bf16", (0, 1000, 2000)),
    (1, "bidirectional_document", 2, 2, 600, 64, "bf16", (0, 100, 600)),
    (1, "causal", 1, 2, 900, 128, "bf16", (0, 450, 900)),
    (2, "causal_document", 1, 2, 400, 64, "f32", (0, 129, 400)),
]


@pytest.mark.parametrize("cfg,mask,B,H,N,d,dtype,cuts", CASES, ids=lambda x: str(x))
def test_row_blocks(fm, cfg, mask, B, H, N, d, dtype, cuts):
    case = C.make_case(cfg, mask, B, H, N, d, dtype)
    print(f"\nrows {case.name} blocks {cuts}", flush=True)
    vecs = C.device_vectors(case.spec)
    bounds = fm.fm_tile_bounds(*vecs, B, case.spec.Hm, N) if any(x is not None for x in vecs) else None
    dk_sum = torch.zeros(B, H, N, d, dtype=torch.float64)
    dv_sum = torch.zeros(B, H, N, d, dtype=torch.float64)
    for a, b in zip(cuts[:-1], cuts[1:]):
        gpu = _gpu_rows(fm, case, a, b, vecs, bounds)
        ref = _oracle_rows(case, a, b)
        report = {}
        C.compare(gpu, ref, dtype, report)
        print(f"  block [{a}, {b}): {report}", flush=True)
        dk_sum += gpu["dk"].double()
        dv_sum += gpu["dv"].double()
    whole = C.run_oracle(case)
    tol = C.TOL[dtype]["grad"]
    assert C.rel_fro(dk_sum.numpy(), whole["dk"]) <= tol
    assert C.rel_fro(dv_sum.numpy(), whole["dv"]) <= tol


def test_more_query_rows_than_keys(fm):
    # rows 300 .. 999 against 500 keys with a prefix-LM mask over the keys: rows past the last key still
    # see every unmasked key
    B, H, Nk, d = 1, 2, 500, 64
    rng = np.random.default_rng(3)
    spec = W.encode_prefix_lm(200, Nk)
    q = torch.from_numpy(rng.standard_normal((B, H, 700, d)).astype(np.float32)).to(torch.bfloat16)
    k, v = (torch.from_numpy(rng.standard_normal((B, H, Nk, d)).astype(np.float32)).to(torch.bfloat16)
            for _ in range(2))
    do = torch.from_numpy(rng.standard_normal((B, H, 700, d)).astype(np.float32)).to(torch.bfloat16)
    vecs = C.device_vectors(spec)
    bounds = fm.fm_tile_bounds(*vecs, B, 1, Nk)
    out, lse = fm.fm_fwd_rows(q.cuda(), k.cuda(), v.cuda(), 300, *vecs, bounds=bounds, causal=False)
    dq, dk, dv = fm.fm_bwd_rows(q.cuda(), k.cuda(), v.cuda(), out, do.cuda(), lse, 300, *vecs, bounds=bounds,
                                causal=False)
    torch.cuda.synchronize()
    scale = d ** -0.5
    for hh in range(H):
        o, l_, gq, gk, gv = OA.fwd_bwd_rows_head(C.f64(q[0, hh]), C.f64(k[0, hh]), C.f64(v[0, hh]),
                                                 C.f64(do[0, hh]), spec.column_slice(0, 0), False, scale, 300)
        ref = {"out": o, "lse": l_, "dq": gq, "dk": gk, "dv": gv}
        gpu = {"out": out[0, hh].cpu(), "lse": lse[0, hh].cpu(), "dq": dq[0, hh].cpu(), "dk": dk[0, hh].cpu(),
               "dv": dv[0, hh].cpu()}
        C.compare(gpu, ref, "bf16")
