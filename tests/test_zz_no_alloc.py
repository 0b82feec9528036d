"""fm_bwd_noalloc (the backward whose workspace is the library's fixed device array) against fm_bwd, the
entry point it varies, through the C ABI: two calls in a row, the second on a smaller problem, each bitwise
equal to fm_bwd on the same inputs and within the parity bars of the fp64 oracle."""
import pytest
import torch

from tests import fmcase as C

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mask_aware_exact_amd as m
    m.load_library()
    return m


def _run(fm, case):
    dev = "cuda"
    q, k, v, do = (t.to(dev) for t in (case.q, case.k, case.v, case.do))
    vecs = C.device_vectors(case.spec, dev)
    bounds = fm.fm_tile_bounds(*vecs, case.B, case.spec.Hm, case.N) if any(x is not None for x in vecs) else None
    out, lse = fm.fm_fwd(q, k, v, *vecs, bounds=bounds, causal=case.spec.causal, scale=case.scale)
    ref = fm.fm_bwd(q, k, v, out, do, lse, *vecs, bounds=bounds, causal=case.spec.causal, scale=case.scale)
    sentinel = [torch.full_like(t, 7.0) for t in (q, k, v)]
    got = fm.fm_bwd_noalloc(q, k, v, out, do, lse, *vecs, bounds=bounds, causal=case.spec.causal,
                            scale=case.scale, dq=sentinel[0], dk=sentinel[1], dv=sentinel[2])
    torch.cuda.synchronize()
    return {"out": out.cpu(), "lse": lse.cpu(), "dq": got[0].cpu(), "dk": got[1].cpu(), "dv": got[2].cpu()}, \
        [t.cpu() for t in ref]


def test_noalloc_matches_fm_bwd_on_two_calls(fm):
    for case in (C.make_case(2, "causal_document", 1, 4, 1000, 128, "bf16"),
                 C.make_case(3, "causal_key_drop", 1, 2, 300, 64, "bf16")):
        print(f"\nno-alloc backward {case.name}", flush=True)
        gpu, ref = _run(fm, case)
        for name, r in zip(("dq", "dk", "dv"), ref):
            assert torch.equal(gpu[name], r), name
        print(C.compare(gpu, C.run_oracle(case), "bf16"), flush=True)
