"""GPU parity of key compaction (fm_compact_keys, fm_gather_rows) with the oracle: the index maps and
the compacted mask bit for bit, the row gather exactly, and the attention results of the compacted
pipeline against the oracle on the original problem (SCFA review, nubint.ai, "proposed method")."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import compact as OC
from tests import fmcase as C

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mask_aware_exact_amd as m
    m.load_library()
    return m


def _check_maps(fm, spec, B, Hm, N):
    vecs = C.device_vectors(spec)
    kidx, kpos, counts, vecs2 = fm.fm_compact_keys(*vecs, B, Hm, N, spec.causal)
    torch.cuda.synchronize()
    r_kidx, r_kpos, r_counts, r_vecs2 = OC.compact_keys(spec.vectors(), spec.causal, B, Hm, N)
    assert np.array_equal(counts.cpu().numpy(), r_counts)
    ok = r_counts >= 0
    assert np.array_equal(kidx.cpu().numpy()[ok], r_kidx[ok])
    assert np.array_equal(kpos.cpu().numpy()[ok], r_kpos[ok])
    for g, r in zip(vecs2, r_vecs2):
        assert np.array_equal(g.cpu().numpy()[ok], r[ok])


# (cfg, family, B, H, N) with per-head vectors where the family has them
MAP_CASES = [
    (3, "causal_key_drop", 2, 3, 1),
    (3, "causal_key_drop", 2, 3, 63),
    (3, "causal_key_drop", 1, 4, 1000),
    (3, "causal_key_drop", 1, 2, 1025),
    (3, "causal_key_drop", 1, 2, 5000),
    (4, "causal_document_block_sparse", 1, 2, 3000),
    (4, "causal_document", 2, 2, 2049),
    (3, "prefix_lm", 1, 2, 700),
    (3, "share_question", 1, 2, 900),
    (1, "bidirectional_document", 2, 2, 500),
    (1, "full", 1, 2, 300),
    (1, "causal", 1, 2, 300),
]


@pytest.mark.parametrize("cfg,mask,B,H,N", MAP_CASES, ids=lambda x: str(x))
def test_maps_and_vectors_bit_exact(fm, cfg, mask, B, H, N):
    spec = W.make_mask(cfg, mask, B, H, N)
    print(f"\ncompaction {mask} B{B} H{H} N{N} Hm{spec.Hm}", flush=True)
    _check_maps(fm, spec, B, spec.Hm, N)


@pytest.mark.parametrize("causal", [False, True])
def test_arbitrary_vectors_bit_exact(fm, causal):
    rng = np.random.default_rng([11, int(causal)])
    B, Hm, N = 2, 3, 1500
    v = [rng.integers(-5, N + 6, size=(B, Hm, N)).astype(np.int32) for _ in range(4)]
    spec = W.MaskSpec(N, B, Hm, causal, v[0], v[1], v[2], v[3])
    _check_maps(fm, spec, B, Hm, N)


def test_not_compactable_row_reports_minus_one(fm):
    N = 16
    lts, lte = np.full((1, 2, N), N, np.int32), np.full((1, 2, N), N, np.int32)
    uts, ute = np.zeros((1, 2, N), np.int32), np.zeros((1, 2, N), np.int32)
    lts[0, 1, 4], lte[0, 1, 4], uts[0, 1, 4], ute[0, 1, 4] = 8, 10, 12, 14
    spec = W.MaskSpec(N, 1, 2, True, lts, lte, uts, ute)
    vecs = C.device_vectors(spec)
    _, _, counts, _ = fm.fm_compact_keys(*vecs, 1, 2, N, True)
    assert counts.cpu().numpy().tolist() == [[N, -1]]


@pytest.mark.parametrize("dtype,d,Hm", [("bf16", 128, 1), ("bf16", 64, 3), ("f32", 64, 3), ("f32", 128, 1)])
def test_gather_rows_exact(fm, dtype, d, Hm):
    B, H, N = 2, 3, 333
    rng = np.random.default_rng([d, Hm])
    x = torch.from_numpy(rng.standard_normal((B, H, N, d)).astype(np.float32)).to(C.TORCH_DT[dtype])
    idx = rng.integers(-1, N, size=(B, Hm, N)).astype(np.int32)
    y = fm.fm_gather_rows(x.cuda(), torch.from_numpy(idx).cuda()).cpu()
    xn = x.float().numpy()
    for b in range(B):
        for h in range(H):
            ref = OC.gather_rows(xn[b, h], idx[b, h if Hm > 1 else 0].astype(np.int64))
            assert np.array_equal(y[b, h].float().numpy(), ref)


# (cfg, family, B, H, N, d, dtype)
PIPE_CASES = [
    (3, "causal_key_drop", 1, 4, 1300, 128, "bf16"),
    (3, "causal_key_drop", 2, 2, 777, 64, "bf16"),
    (3, "causal_key_drop", 1, 2, 300, 64, "f32"),
    (4, "causal_document_block_sparse", 1, 2, 2500, 128, "bf16"),
    (3, "prefix_lm", 1, 2, 600, 128, "bf16"),
    (1, "bidirectional_document", 1, 2, 400, 64, "bf16"),
    (2, "causal_document", 1, 2, 1000, 128, "bf16"),
]


@pytest.mark.parametrize("cfg,mask,B,H,N,d,dtype", PIPE_CASES, ids=lambda x: str(x))
def test_compacted_pipeline_parity(fm, cfg, mask, B, H, N, d, dtype):
    case = C.make_case(cfg, mask, B, H, N, d, dtype)
    print(f"\ncompacted {case.name}", flush=True)
    gpu = C.run_gpu_compacted(case, fm)
    ref = C.run_oracle(case)
    report = {}
    C.compare(gpu, ref, dtype, report)
    print(report, flush=True)
    dropped = gpu["kpos"].numpy() < 0
    for name in ("dk", "dv"):
        g = gpu[name].float().numpy()
        for b in range(B):
            for h in range(H):
                assert np.all(g[b, h][dropped[b, h if case.spec.Hm > 1 else 0]] == 0.0)
