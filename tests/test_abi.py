"""The C-ABI library loads, exports every symbol include/fm.h declares, and rejects bad arguments on
the host before any launch (CPU: no call here reaches a kernel)."""
import ctypes
import os
import re

import pytest

import mask_aware_exact_amd as fm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "fm.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fm_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fm.LIB_PATH):
        fm_build = __import__("mask_aware_exact_amd.build", fromlist=["build"])
        fm_build.build()
    return fm.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert set(names) == set(fm.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_size_queries(lib):
    assert lib.fm_kblock() == 64
    assert lib.fm_fwd_qblock(64) == 128 and lib.fm_fwd_qblock(128) == 128 and lib.fm_fwd_qblock(96) == 0
    assert lib.fm_bounds_elems(1, 1, 1) == 8
    assert lib.fm_bounds_elems(2, 3, 130) == 2 * 3 * 3 * 8
    assert lib.fm_bounds_elems(0, 1, 10) == 0 and lib.fm_bounds_elems(1, 1, (1 << 24) + 1) == 0
    n = lib.fm_bwd_workspace_bytes(fm.FM_BF16, 1, 2, 100, 64)
    assert n >= 1 * 2 * 100 * 4 and n % 256 == 0
    assert lib.fm_bwd_workspace_bytes(fm.FM_BF16, 1, 2, 100, 96) == 0
    assert lib.fm_bwd_workspace_bytes(7, 1, 2, 100, 64) == 0


def test_status_strings(lib):
    for s in range(5):
        assert isinstance(fm.status_str(s), str) and fm.status_str(s)
    assert fm.status_str(42) == "unknown status"


P = ctypes.c_void_p
A = P(0x100000)  # an aligned stand-in address: every call below is rejected before it is used
B_ = P(0x200000)


def _fwd(lib, **kw):
    args = dict(q=A, k=A, v=A, dtype=fm.FM_BF16, B=1, H=2, N=100, d=64, lts=None, lte=None, uts=None,
                ute=None, Hm=1, bounds=None, sched=None, causal=1, scale=0.125, out=B_, lse=B_)
    args.update(kw)
    return lib.fm_fwd(args["q"], args["k"], args["v"], args["dtype"], args["B"], args["H"], args["N"],
                      args["d"], args["lts"], args["lte"], args["uts"], args["ute"], args["Hm"], args["bounds"],
                      args["sched"], args["causal"], args["scale"], args["out"], args["lse"], None)


def test_fwd_validation(lib):
    assert _fwd(lib, q=None) == fm.FM_ERR_INVALID
    assert _fwd(lib, out=None) == fm.FM_ERR_INVALID
    assert _fwd(lib, lse=None) == fm.FM_ERR_INVALID
    assert _fwd(lib, B=0) == fm.FM_ERR_INVALID
    assert _fwd(lib, N=-5) == fm.FM_ERR_INVALID
    assert _fwd(lib, N=(1 << 24) + 1) == fm.FM_ERR_INVALID
    assert _fwd(lib, scale=float("inf")) == fm.FM_ERR_INVALID
    assert _fwd(lib, scale=float("nan")) == fm.FM_ERR_INVALID
    assert _fwd(lib, scale=0.0) == fm.FM_ERR_INVALID
    assert _fwd(lib, scale=-0.5) == fm.FM_ERR_INVALID
    assert _fwd(lib, lts=A) == fm.FM_ERR_INVALID                      # half-NULL pair
    assert _fwd(lib, ute=A) == fm.FM_ERR_INVALID
    assert _fwd(lib, lts=A, lte=A) == fm.FM_ERR_INVALID               # vectors without bounds
    assert _fwd(lib, lts=A, lte=A, bounds=A, Hm=3) == fm.FM_ERR_INVALID  # Hm not in {1, H}
    assert _fwd(lib, d=96) == fm.FM_ERR_UNSUPPORTED
    assert _fwd(lib, d=256) == fm.FM_ERR_UNSUPPORTED
    assert _fwd(lib, dtype=5) == fm.FM_ERR_UNSUPPORTED
    assert _fwd(lib, q=P(0x100002)) == fm.FM_ERR_INVALID              # misaligned


def _bwd(lib, **kw):
    args = dict(q=A, k=A, v=A, out=A, dout=A, lse=A, dtype=fm.FM_BF16, B=1, H=2, N=100, d=64, lts=None,
                lte=None, uts=None, ute=None, Hm=1, bounds=None, sched=None, causal=1, scale=0.125, dq=B_, dk=B_,
                dv=B_,
                ws=P(0x300000), ws_bytes=1 << 30)
    args.update(kw)
    return lib.fm_bwd(args["q"], args["k"], args["v"], args["out"], args["dout"], args["lse"], args["dtype"],
                      args["B"], args["H"], args["N"], args["d"], args["lts"], args["lte"], args["uts"],
                      args["ute"], args["Hm"], args["bounds"], args["sched"], args["causal"], args["scale"], args["dq"],
                      args["dk"], args["dv"], args["ws"], args["ws_bytes"], None)


def test_bwd_validation(lib):
    for name in ("q", "k", "v", "out", "dout", "lse", "dq", "dk", "dv"):
        assert _bwd(lib, **{name: None}) == fm.FM_ERR_INVALID, name
    assert _bwd(lib, H=0) == fm.FM_ERR_INVALID
    assert _bwd(lib, scale=-1.0) == fm.FM_ERR_INVALID
    assert _bwd(lib, uts=A) == fm.FM_ERR_INVALID
    assert _bwd(lib, uts=A, ute=A) == fm.FM_ERR_INVALID
    assert _bwd(lib, d=32) == fm.FM_ERR_UNSUPPORTED
    assert _bwd(lib, ws=None) == fm.FM_ERR_WORKSPACE
    need = lib.fm_bwd_workspace_bytes(fm.FM_BF16, 1, 2, 100, 64)
    assert _bwd(lib, ws_bytes=need - 1) == fm.FM_ERR_WORKSPACE
    assert _bwd(lib, dk=P(0x200008)) == fm.FM_ERR_INVALID


def test_mapped_validation(lib):
    """fm_fwd_mapped / fm_bwd_mapped: the fm_fwd / fm_bwd checks (an unknown dtype refused), plus NULL maps."""
    M = P(0x400000)

    def fwdm(omap=M, dtype=fm.FM_BF16, B=1, q=A, scale=0.125):
        return lib.fm_fwd_mapped(q, A, A, dtype, B, 2, 100, 64, None, None, None, None, 1, None, None, 0, scale,
                                 omap, B_, B_, None)

    def bwdm(qmap=M, kmap=M, dtype=fm.FM_BF16, ws_bytes=1 << 30, dq=B_):
        return lib.fm_bwd_mapped(A, A, A, A, A, A, dtype, 1, 2, 100, 64, None, None, None, None, 1, None, None, 0,
                                 0.125, qmap, kmap, dq, B_, B_, P(0x300000), ws_bytes, None)

    assert fwdm(omap=None) == fm.FM_ERR_INVALID
    assert fwdm(dtype=7) == fm.FM_ERR_UNSUPPORTED
    assert fwdm(B=0) == fm.FM_ERR_INVALID
    assert fwdm(q=None) == fm.FM_ERR_INVALID
    assert fwdm(scale=-1.0) == fm.FM_ERR_INVALID
    assert bwdm(qmap=None) == fm.FM_ERR_INVALID
    assert bwdm(kmap=None) == fm.FM_ERR_INVALID
    assert bwdm(dtype=7) == fm.FM_ERR_UNSUPPORTED
    assert bwdm(dq=None) == fm.FM_ERR_INVALID
    assert bwdm(ws_bytes=16) == fm.FM_ERR_WORKSPACE


def test_bounds_and_classes_validation(lib):
    assert lib.fm_tile_bounds(A, A, None, None, 1, 1, 10, None, None) == fm.FM_ERR_INVALID
    assert lib.fm_tile_bounds(A, None, None, None, 1, 1, 10, B_, None) == fm.FM_ERR_INVALID
    assert lib.fm_tile_bounds(None, None, None, None, 0, 1, 10, B_, None) == fm.FM_ERR_INVALID
    assert lib.fm_tile_classes(A, 1, 1, 10, 1, 0, B_, None) == fm.FM_ERR_INVALID
    assert lib.fm_tile_classes(A, 1, 1, 10, 1, 64, None, None) == fm.FM_ERR_INVALID


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fm.fm_fwd(q, q, q)


def _compact(lib, **kw):
    args = dict(lts=A, lte=A, uts=None, ute=None, B=1, Hm=2, N=100, causal=1, kidx=A, kpos=A, counts=A,
                lts2=A, lte2=A, uts2=A, ute2=A)
    args.update(kw)
    return lib.fm_compact_keys(args["lts"], args["lte"], args["uts"], args["ute"], args["B"], args["Hm"],
                               args["N"], args["causal"], args["kidx"], args["kpos"], args["counts"],
                               args["lts2"], args["lte2"], args["uts2"], args["ute2"], None)


def test_compact_validation(lib):
    for name in ("kidx", "kpos", "counts", "lts2", "lte2", "uts2", "ute2"):
        assert _compact(lib, **{name: None}) == fm.FM_ERR_INVALID, name
    assert _compact(lib, lte=None) == fm.FM_ERR_INVALID          # half-NULL pair
    assert _compact(lib, uts=A) == fm.FM_ERR_INVALID
    assert _compact(lib, B=0) == fm.FM_ERR_INVALID
    assert _compact(lib, N=(1 << 24) + 1) == fm.FM_ERR_INVALID


def _gather(lib, **kw):
    args = dict(x=A, dtype=fm.FM_BF16, B=1, H=2, N=100, d=64, idx=A, Hm=1, y=P(0x200000))
    args.update(kw)
    return lib.fm_gather_rows(args["x"], args["dtype"], args["B"], args["H"], args["N"], args["d"], args["idx"],
                              args["Hm"], args["y"], None)


def test_gather_validation(lib):
    assert _gather(lib, x=None) == fm.FM_ERR_INVALID
    assert _gather(lib, idx=None) == fm.FM_ERR_INVALID
    assert _gather(lib, y=None) == fm.FM_ERR_INVALID
    assert _gather(lib, y=A) == fm.FM_ERR_INVALID                 # aliases x
    assert _gather(lib, Hm=3) == fm.FM_ERR_INVALID
    assert _gather(lib, d=96) == fm.FM_ERR_UNSUPPORTED
    assert _gather(lib, dtype=5) == fm.FM_ERR_UNSUPPORTED
    assert _gather(lib, y=P(0x200004)) == fm.FM_ERR_INVALID       # misaligned
    assert _gather(lib, H=0) == fm.FM_ERR_INVALID


def test_rows_validation(lib):
    # (q, k, v, dtype, B, H, Nq, Nk, q_off, d, lts, lte, uts, ute, Hm, bounds, sched, causal, scale, out, lse,
    #  stream)
    def fwd_rows(Nq=100, Nk=100, q_off=0):
        return lib.fm_fwd_rows(A, A, A, fm.FM_BF16, 1, 2, Nq, Nk, q_off, 64, None, None, None, None, 1, None, None,
                               1, 0.125, B_, B_, None)
    assert fwd_rows(q_off=-1) == fm.FM_ERR_INVALID
    assert fwd_rows(Nk=0) == fm.FM_ERR_INVALID
    assert fwd_rows(Nq=0) == fm.FM_ERR_INVALID
    assert fwd_rows(q_off=(1 << 24) - 50) == fm.FM_ERR_INVALID    # rows past FM_MAX_N
    ws = lib.fm_bwd_workspace_bytes(fm.FM_BF16, 1, 2, 100, 64)

    def bwd_rows(q_off=0, wsb=ws):
        return lib.fm_bwd_rows(A, A, A, A, A, A, fm.FM_BF16, 1, 2, 100, 100, q_off, 64, None, None, None, None, 1,
                               None, None, 1, 0.125, B_, B_, B_, A, wsb, None)
    assert bwd_rows(q_off=-3) == fm.FM_ERR_INVALID
    assert bwd_rows(wsb=ws - 256) == fm.FM_ERR_WORKSPACE


def test_schedule_validation(lib):
    assert lib.fm_schedule_elems(1, 1, 1, 1) == 4
    assert lib.fm_schedule_elems(2, 3, 300, 129) == 2 * 3 * 2 * (3 + 2)
    assert lib.fm_schedule_elems(0, 1, 10, 10) == 0 and lib.fm_schedule_elems(1, 1, (1 << 24) + 1, 10) == 0
    # (bounds, B, Hm, Nq, Nk, q_off, causal, sched, stream)
    assert lib.fm_tile_schedule(A, 1, 1, 100, 100, 0, 1, None, None) == fm.FM_ERR_INVALID
    assert lib.fm_tile_schedule(A, 0, 1, 100, 100, 0, 1, B_, None) == fm.FM_ERR_INVALID
    assert lib.fm_tile_schedule(A, 1, 1, 100, 0, 0, 1, B_, None) == fm.FM_ERR_INVALID
    assert lib.fm_tile_schedule(A, 1, 1, 100, 100, -1, 1, B_, None) == fm.FM_ERR_INVALID
    assert lib.fm_tile_schedule(A, 1, 1, 100, 100, (1 << 24) - 50, 1, B_, None) == fm.FM_ERR_INVALID


def test_hash_validation(lib):
    # fm_lsh_buckets(x, dtype, B, H, N, d, rot, Hr, nb, buckets, stream)
    def lsh(**kw):
        a = dict(x=A, dtype=fm.FM_BF16, B=1, H=2, N=100, d=128, rot=A, Hr=2, nb=16, out=B_)
        a.update(kw)
        return lib.fm_lsh_buckets(a["x"], a["dtype"], a["B"], a["H"], a["N"], a["d"], a["rot"], a["Hr"], a["nb"],
                                  a["out"], None)
    for name in ("x", "rot", "out"):
        assert lsh(**{name: None}) == fm.FM_ERR_INVALID, name
    assert lsh(nb=15) == fm.FM_ERR_INVALID          # odd
    assert lsh(nb=0) == fm.FM_ERR_INVALID
    assert lsh(nb=66) == fm.FM_ERR_INVALID          # above 64
    assert lsh(Hr=3) == fm.FM_ERR_INVALID           # not 1 or H
    assert lsh(x=P(0x100004)) == fm.FM_ERR_INVALID  # misaligned
    assert lsh(d=96) == fm.FM_ERR_UNSUPPORTED
    assert lsh(dtype=9) == fm.FM_ERR_UNSUPPORTED
    assert lsh(N=0) == fm.FM_ERR_INVALID

    # fm_bucket_sort(qb, kb, B, H, N, nb, qidx, qpos, kidx, kpos, lts, lte, uts, ute, stream)
    def srt(nb=16, N=100, **kw):
        p = dict(qb=A, kb=A, qidx=B_, qpos=B_, kidx=B_, kpos=B_, lts=B_, lte=B_, uts=B_, ute=B_)
        p.update(kw)
        return lib.fm_bucket_sort(p["qb"], p["kb"], 1, 2, N, nb, p["qidx"], p["qpos"], p["kidx"], p["kpos"],
                                  p["lts"], p["lte"], p["uts"], p["ute"], None)
    for name in ("qb", "kb", "qidx", "qpos", "kidx", "kpos", "lts", "lte", "uts", "ute"):
        assert srt(**{name: None}) == fm.FM_ERR_INVALID, name
    assert srt(nb=0) == fm.FM_ERR_INVALID
    assert srt(nb=513) == fm.FM_ERR_INVALID
    assert srt(N=(1 << 24) + 1) == fm.FM_ERR_INVALID


def test_noalloc_rejects_problems_past_its_array(lib):
    """fm_bwd_noalloc holds D (4 bytes per query row) in a fixed array of FM_NOALLOC_SCRATCH_BYTES: a larger
    problem is FM_ERR_WORKSPACE, decided on the host before anything is launched."""
    limit_rows = (16 << 20) // 4
    args = lambda H, N: (A, A, A, A, A, A, fm.FM_BF16, 1, H, N, 64, None, None, None, None, 1, None, None, 1,  # noqa
                         ctypes.c_float(0.125), B_, B_, B_, None)
    assert lib.fm_bwd_noalloc(*args(64, 131072)) == fm.FM_ERR_WORKSPACE   # 2^23 rows
    assert lib.fm_bwd_noalloc(*args(32, limit_rows // 32 + 1)) == fm.FM_ERR_WORKSPACE
    assert lib.fm_bwd_noalloc(*args(2, 0)) == fm.FM_ERR_INVALID            # bad sizes as fm_bwd reports them
    assert lib.fm_bwd_noalloc(*args(2, 100)[:10] + (96,) + args(2, 100)[11:]) == fm.FM_ERR_UNSUPPORTED
