"""Thin Python binding of libfm.so, the column-wise-mask (FlashMask) exact attention library for MI355X.

Argument marshalling only: torch supplies device memory and the current stream, every step of the
path runs in the HIP kernels behind the C ABI declared in include/fm.h. The entry points keep the C
names: fm_tile_bounds, fm_tile_schedule, fm_fwd, fm_bwd, their row-block forms fm_fwd_rows and
fm_bwd_rows, the key-compaction pair fm_compact_keys and fm_gather_rows, the hash-bucket pair
fm_lsh_buckets and fm_bucket_sort (plus fm_tile_classes, a test hook). There is no fallback:
if libfm.so is missing or cannot be loaded, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfm.so")

FM_OK, FM_ERR_INVALID, FM_ERR_UNSUPPORTED, FM_ERR_WORKSPACE, FM_ERR_LAUNCH = 0, 1, 2, 3, 4
FM_BF16, FM_F32 = 0, 1
NONE, PARTIAL, FULL = 0, 1, 2

EXPORTED = ("fm_kblock", "fm_fwd_qblock", "fm_bounds_elems", "fm_tile_bounds", "fm_schedule_elems",
            "fm_tile_schedule", "fm_fwd",
            "fm_bwd_workspace_bytes", "fm_bwd", "fm_fwd_rows", "fm_bwd_rows", "fm_tile_classes",
            "fm_compact_keys", "fm_gather_rows", "fm_lsh_buckets", "fm_bucket_sort", "fm_fwd_mapped",
            "fm_bwd_mapped", "fm_bwd_plan_bytes", "fm_bwd_plan", "fm_bwd_ds_workspace_bytes", "fm_bwd_ds",
            "fm_bwd_noalloc", "fm_status_str")


class FmError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_str(status)} (status {status})")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libfm.so and declare its signatures; raises if the library is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m mask_aware_exact_amd.build`")
    lib = ctypes.CDLL(path)
    P, I, F, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fm_kblock.restype = I
    lib.fm_kblock.argtypes = []
    lib.fm_fwd_qblock.restype = I
    lib.fm_fwd_qblock.argtypes = [I]
    lib.fm_bounds_elems.restype = S
    lib.fm_bounds_elems.argtypes = [I, I, I]
    lib.fm_tile_bounds.restype = I
    lib.fm_tile_bounds.argtypes = [P, P, P, P, I, I, I, P, P]
    lib.fm_fwd.restype = I
    lib.fm_schedule_elems.restype = S
    lib.fm_schedule_elems.argtypes = [I, I, I, I]
    lib.fm_tile_schedule.restype = I
    lib.fm_tile_schedule.argtypes = [P, I, I, I, I, I, I, P, P]
    lib.fm_fwd.argtypes = [P, P, P, I, I, I, I, I, P, P, P, P, I, P, P, I, F, P, P, P]
    lib.fm_bwd_workspace_bytes.restype = S
    lib.fm_bwd_workspace_bytes.argtypes = [I, I, I, I, I]
    lib.fm_bwd.restype = I
    lib.fm_bwd.argtypes = [P, P, P, P, P, P, I, I, I, I, I, P, P, P, P, I, P, P, I, F, P, P, P, P, S, P]
    lib.fm_bwd_plan_bytes.restype = S
    lib.fm_bwd_plan_bytes.argtypes = [I, I, I, I]
    lib.fm_bwd_plan.restype = I
    lib.fm_bwd_plan.argtypes = [P, I, I, I, I, I, P, P]
    lib.fm_bwd_ds_workspace_bytes.restype = S
    lib.fm_bwd_ds_workspace_bytes.argtypes = [I, I, I, I, I, ctypes.c_int64]
    lib.fm_bwd_ds.restype = I
    lib.fm_bwd_ds.argtypes = [P, P, P, P, P, P, I, I, I, I, I, P, P, P, P, I, P, P, P, I, F, P, P, P, P, S, P]
    lib.fm_bwd_noalloc.restype = I
    lib.fm_bwd_noalloc.argtypes = [P, P, P, P, P, P, I, I, I, I, I, P, P, P, P, I, P, P, I, F, P, P, P, P]
    lib.fm_tile_classes.restype = I
    lib.fm_tile_classes.argtypes = [P, I, I, I, I, I, P, P]
    lib.fm_fwd_mapped.restype = I
    lib.fm_fwd_mapped.argtypes = [P, P, P, I, I, I, I, I, P, P, P, P, I, P, P, I, F, P, P, P, P]
    lib.fm_bwd_mapped.restype = I
    lib.fm_bwd_mapped.argtypes = [P, P, P, P, P, P, I, I, I, I, I, P, P, P, P, I, P, P, I, F, P, P, P, P, P, P, S, P]
    lib.fm_fwd_rows.restype = I
    lib.fm_fwd_rows.argtypes = [P, P, P, I, I, I, I, I, I, I, P, P, P, P, I, P, P, I, F, P, P, P]
    lib.fm_bwd_rows.restype = I
    lib.fm_bwd_rows.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, P, P, P, P, I, P, P, I, F, P, P, P, P, S,
                                P]
    lib.fm_compact_keys.restype = I
    lib.fm_compact_keys.argtypes = [P, P, P, P, I, I, I, I, P, P, P, P, P, P, P, P]
    lib.fm_gather_rows.restype = I
    lib.fm_gather_rows.argtypes = [P, I, I, I, I, I, P, I, P, P]
    lib.fm_lsh_buckets.restype = I
    lib.fm_lsh_buckets.argtypes = [P, I, I, I, I, I, P, I, I, P, P]
    lib.fm_bucket_sort.restype = I
    lib.fm_bucket_sort.argtypes = [P, P, I, I, I, I, P, P, P, P, P, P, P, P, P]
    lib.fm_status_str.restype = ctypes.c_char_p
    lib.fm_status_str.argtypes = [I]
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load_library().fm_status_str(int(status)).decode()


def _check(status: int, where: str):
    if status != FM_OK:
        raise FmError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return FM_BF16
    if t.dtype == torch.float32:
        return FM_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _need_cuda(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("tensors must live on the GPU")
            if not t.is_contiguous():
                raise ValueError("tensors must be contiguous")


def _vec(t):
    if t is None:
        return None
    if t.dtype != torch.int32:
        raise TypeError("mask vectors must be int32")
    return t


def fm_kblock() -> int:
    return load_library().fm_kblock()


def fm_fwd_qblock(d: int) -> int:
    return load_library().fm_fwd_qblock(int(d))


def fm_bounds_elems(B: int, Hm: int, N: int) -> int:
    return load_library().fm_bounds_elems(B, Hm, N)


def fm_bwd_workspace_bytes(dtype: torch.dtype, B: int, H: int, N: int, d: int) -> int:
    code = FM_BF16 if dtype == torch.bfloat16 else FM_F32 if dtype == torch.float32 else 99
    return load_library().fm_bwd_workspace_bytes(code, B, H, N, d)


def fm_tile_bounds(lts, lte, uts, ute, B: int, Hm: int, N: int, bounds=None, stream=None):
    """int32 [B, Hm, ceil(N/64), 8] per-key-tile min/max of the four vectors (None pairs allowed)."""
    lib = load_library()
    vecs = [_vec(x) for x in (lts, lte, uts, ute)]
    _need_cuda(*vecs)
    if bounds is None:
        dev = next((x.device for x in vecs if x is not None), torch.device("cuda"))
        bounds = torch.empty(fm_bounds_elems(B, Hm, N), dtype=torch.int32, device=dev)
    _check(lib.fm_tile_bounds(*[_ptr(x) for x in vecs], B, Hm, N, _ptr(bounds), _stream(stream)),
           "fm_tile_bounds")
    return bounds.view(B, Hm, -1, 8)


def fm_schedule_elems(B: int, Hm: int, Nq: int, Nk: int) -> int:
    return load_library().fm_schedule_elems(B, Hm, Nq, Nk)


def fm_tile_schedule(bounds, B: int, Hm: int, Nq: int, Nk: int, causal: bool, q_off: int = 0, sched=None,
                     device=None, stream=None):
    """int32 [B, Hm, 2 (nq + nk)] longest-first dispatch schedule (nq = ceil(Nq/128), nk = ceil(Nk/128)):
    query-unit order, key-unit order, then the work of each query unit and of each key unit."""
    lib = load_library()
    _need_cuda(bounds)
    n = fm_schedule_elems(B, Hm, Nq, Nk)
    if sched is None:
        dev = bounds.device if bounds is not None else (device or torch.device("cuda"))
        sched = torch.empty(max(n, 1), dtype=torch.int32, device=dev)
    _check(lib.fm_tile_schedule(_ptr(bounds), B, Hm, Nq, Nk, int(q_off), int(bool(causal)), _ptr(sched),
                                _stream(stream)), "fm_tile_schedule")
    return sched[:n].view(B, Hm, -1)


def split_schedule(sched, Nq: int, Nk: int):
    """(query order, key order, query work, key work) views of a [B, Hm, 2 (nq + nk)] schedule."""
    nq, nk = -(-Nq // 128), -(-Nk // 128)
    return sched[..., :nq], sched[..., nq:nq + nk], sched[..., nq + nk:2 * nq + nk], sched[..., 2 * nq + nk:]


def fm_fwd(q, k, v, lts=None, lte=None, uts=None, ute=None, bounds=None, causal=False, scale=None,
           out=None, lse=None, stream=None, sched=None):
    """(out, lse) for q, k, v of shape [B, H, N, d]; vectors int32 [B, Hm, N] or None."""
    lib = load_library()
    B, H, N, d = q.shape
    vecs = [_vec(x) for x in (lts, lte, uts, ute)]
    Hm = next((x.shape[1] for x in vecs if x is not None), 1)
    _need_cuda(q, k, v, bounds, sched, *vecs)
    if scale is None:
        scale = d ** -0.5
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _check(lib.fm_fwd(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), B, H, N, d, *[_ptr(x) for x in vecs], Hm,
                      _ptr(bounds), _ptr(sched), int(bool(causal)), float(scale), _ptr(out), _ptr(lse), _stream(stream)),
           "fm_fwd")
    return out, lse


def fm_bwd(q, k, v, out, dout, lse, lts=None, lte=None, uts=None, ute=None, bounds=None, causal=False,
           scale=None, dq=None, dk=None, dv=None, workspace=None, stream=None, sched=None):
    """(dq, dk, dv): gradients of sum(out * dout)."""
    lib = load_library()
    B, H, N, d = q.shape
    vecs = [_vec(x) for x in (lts, lte, uts, ute)]
    Hm = next((x.shape[1] for x in vecs if x is not None), 1)
    _need_cuda(q, k, v, out, dout, lse, bounds, sched, *vecs)
    if scale is None:
        scale = d ** -0.5
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = fm_bwd_workspace_bytes(q.dtype, B, H, N, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib.fm_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _dtype_code(q), B, H, N, d,
                      *[_ptr(x) for x in vecs], Hm, _ptr(bounds), _ptr(sched), int(bool(causal)), float(scale), _ptr(dq),
                      _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel(), _stream(stream)), "fm_bwd")
    return dq, dk, dv


def fm_bwd_plan_bytes(B: int, H: int, Hm: int, N: int) -> int:
    return load_library().fm_bwd_plan_bytes(B, H, Hm, N)


def fm_bwd_plan(bounds, B: int, H: int, Hm: int, N: int, causal: bool, plan=None, stream=None, device=None):
    """Plan of the stored-dS backward (uint8 device tensor); plan_tiles() reads its tile count."""
    lib = load_library()
    _need_cuda(bounds, plan)
    if plan is None:
        dev = bounds.device if bounds is not None else (device or torch.device("cuda"))
        plan = torch.empty(max(fm_bwd_plan_bytes(B, H, Hm, N), 8), dtype=torch.uint8, device=dev)
    _check(lib.fm_bwd_plan(_ptr(bounds), B, H, Hm, N, int(bool(causal)), _ptr(plan), _stream(stream)),
           "fm_bwd_plan")
    return plan


def plan_tiles(plan) -> int:
    """Stored-dS tiles of the whole problem (the plan's first 8 bytes; synchronises with the device)."""
    return int(plan[:8].view(torch.int64).item())


def fm_bwd_ds_workspace_bytes(dtype: torch.dtype, B: int, H: int, N: int, d: int, tiles: int) -> int:
    code = FM_BF16 if dtype == torch.bfloat16 else FM_F32
    return load_library().fm_bwd_ds_workspace_bytes(code, B, H, N, d, int(tiles))


def fm_bwd_ds(q, k, v, out, dout, lse, plan, lts=None, lte=None, uts=None, ute=None, bounds=None, causal=False,
              scale=None, dq=None, dk=None, dv=None, workspace=None, stream=None, sched=None):
    """(dq, dk, dv) as fm_bwd, with dq formed from stored dS tiles for the heads that fit in the workspace
    (without a workspace, one sized from the plan's tile count is allocated)."""
    lib = load_library()
    B, H, N, d = q.shape
    vecs = [_vec(x) for x in (lts, lte, uts, ute)]
    Hm = next((x.shape[1] for x in vecs if x is not None), 1)
    _need_cuda(q, k, v, out, dout, lse, bounds, sched, plan, *vecs)
    if scale is None:
        scale = d ** -0.5
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if workspace is None:
        need = fm_bwd_ds_workspace_bytes(q.dtype, B, H, N, d, plan_tiles(plan))
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib.fm_bwd_ds(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _dtype_code(q), B, H, N, d,
                         *[_ptr(x) for x in vecs], Hm, _ptr(bounds), _ptr(sched), _ptr(plan), int(bool(causal)),
                         float(scale), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel(),
                         _stream(stream)), "fm_bwd_ds")
    return dq, dk, dv


def fm_bwd_noalloc(q, k, v, out, dout, lse, lts=None, lte=None, uts=None, ute=None, bounds=None, causal=False,
                   scale=None, dq=None, dk=None, dv=None, stream=None, sched=None):
    """(dq, dk, dv) as fm_bwd, with the workspace in the library's fixed device array (no allocation
    inside the call; outputs are allocated here only when not given)."""
    lib = load_library()
    B, H, N, d = q.shape
    vecs = [_vec(x) for x in (lts, lte, uts, ute)]
    Hm = next((x.shape[1] for x in vecs if x is not None), 1)
    _need_cuda(q, k, v, out, dout, lse, bounds, sched, *vecs)
    if scale is None:
        scale = d ** -0.5
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check(lib.fm_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _dtype_code(q), B, H, N,
                              d, *[_ptr(x) for x in vecs], Hm, _ptr(bounds), _ptr(sched), int(bool(causal)),
                              float(scale), _ptr(dq), _ptr(dk), _ptr(dv), _stream(stream)), "fm_bwd_noalloc")
    return dq, dk, dv


def fm_fwd_mapped(q, k, v, omap, lts=None, lte=None, uts=None, ute=None, bounds=None, causal=False, scale=None,
                  out=None, lse=None, stream=None, sched=None):
    """fm_fwd on a reordered problem with out stored in the original order: out row omap[b, h, r] receives
    result row r (omap int32 [B, H, N]); lse stays in the reordered order."""
    lib = load_library()
    B, H, N, d = q.shape
    vecs = [_vec(x) for x in (lts, lte, uts, ute)]
    Hm = next((x.shape[1] for x in vecs if x is not None), 1)
    _need_cuda(q, k, v, omap, bounds, sched, *vecs)
    if scale is None:
        scale = d ** -0.5
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _check(lib.fm_fwd_mapped(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), B, H, N, d, *[_ptr(x) for x in vecs], Hm,
                             _ptr(bounds), _ptr(sched), int(bool(causal)), float(scale), _ptr(_vec(omap)),
                             _ptr(out), _ptr(lse), _stream(stream)), "fm_fwd_mapped")
    return out, lse


def fm_bwd_mapped(q, k, v, out, dout, lse, qmap, kmap, lts=None, lte=None, uts=None, ute=None, bounds=None,
                  causal=False, scale=None, dq=None, dk=None, dv=None, workspace=None, stream=None, sched=None):
    """fm_bwd on a reordered problem: out (original order, as fm_fwd_mapped wrote it) is read through qmap;
    dq is stored at rows qmap, dk and dv at rows kmap (int32 [B, H, N] each)."""
    lib = load_library()
    B, H, N, d = q.shape
    vecs = [_vec(x) for x in (lts, lte, uts, ute)]
    Hm = next((x.shape[1] for x in vecs if x is not None), 1)
    _need_cuda(q, k, v, out, dout, lse, qmap, kmap, bounds, sched, *vecs)
    if scale is None:
        scale = d ** -0.5
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = fm_bwd_workspace_bytes(q.dtype, B, H, N, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib.fm_bwd_mapped(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _dtype_code(q), B, H, N,
                             d, *[_ptr(x) for x in vecs], Hm, _ptr(bounds), _ptr(sched), int(bool(causal)),
                             float(scale), _ptr(_vec(qmap)), _ptr(_vec(kmap)), _ptr(dq), _ptr(dk), _ptr(dv),
                             _ptr(workspace), workspace.numel(), _stream(stream)), "fm_bwd_mapped")
    return dq, dk, dv


def fm_tile_classes(bounds, B: int, Hm: int, N: int, causal: bool, qblock: int, classes=None, stream=None):
    """uint8 [B, Hm, ceil(N/qblock), ceil(N/64)] tile classes (0 NONE, 1 PARTIAL, 2 FULL)."""
    lib = load_library()
    _need_cuda(bounds)
    if qblock <= 0:
        raise FmError(FM_ERR_INVALID, "fm_tile_classes")
    nq, nk = -(-N // qblock), -(-N // 64)
    if classes is None:
        dev = bounds.device if bounds is not None else torch.device("cuda")
        classes = torch.empty(B * Hm * nq * nk, dtype=torch.uint8, device=dev)
    _check(lib.fm_tile_classes(_ptr(bounds), B, Hm, N, int(bool(causal)), qblock, _ptr(classes),
                               _stream(stream)), "fm_tile_classes")
    return classes.view(B, Hm, nq, nk)


def fm_compact_keys(lts, lte, uts, ute, B: int, Hm: int, N: int, causal: bool, stream=None):
    """Kept-column compaction of the mask (see include/fm.h). Returns (kidx, kpos, counts, vectors) with
    kidx, kpos int32 [B, Hm, N], counts int32 [B, Hm] and vectors the four int32 [B, Hm, N] arrays of
    the compacted problem (to be run with causal = False). Asynchronous: counts of -1 (a column the
    compacted mask cannot hold) are the caller's to check."""
    lib = load_library()
    vecs = [_vec(x) for x in (lts, lte, uts, ute)]
    _need_cuda(*vecs)
    dev = next((x.device for x in vecs if x is not None), torch.device("cuda"))
    new = lambda *shape: torch.empty(shape, dtype=torch.int32, device=dev)  # noqa: E731
    kidx, kpos, counts = new(B, Hm, N), new(B, Hm, N), new(B, Hm)
    out = [new(B, Hm, N) for _ in range(4)]
    _check(lib.fm_compact_keys(*[_ptr(x) for x in vecs], B, Hm, N, int(bool(causal)), _ptr(kidx), _ptr(kpos),
                               _ptr(counts), *[_ptr(x) for x in out], _stream(stream)), "fm_compact_keys")
    return kidx, kpos, counts, out


def fm_gather_rows(x, idx, y=None, stream=None):
    """y[b, h, r] = x[b, h, idx[b, hm, r]] (zero where idx < 0) for x of shape [B, H, N, d]."""
    lib = load_library()
    B, H, N, d = x.shape
    idx = _vec(idx)
    _need_cuda(x, idx)
    y = torch.empty_like(x) if y is None else y
    _check(lib.fm_gather_rows(_ptr(x), _dtype_code(x), B, H, N, d, _ptr(idx), idx.shape[1], _ptr(y),
                              _stream(stream)), "fm_gather_rows")
    return y


def fm_fwd_rows(q, k, v, q_off: int, lts=None, lte=None, uts=None, ute=None, bounds=None, causal=False,
                scale=None, out=None, lse=None, stream=None, sched=None):
    """(out, lse) for the query rows q_off .. q_off + Nq - 1 (q: [B, H, Nq, d]) against all keys
    (k, v: [B, H, Nk, d]); vectors int32 [B, Hm, Nk] in global row coordinates."""
    lib = load_library()
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    vecs = [_vec(x) for x in (lts, lte, uts, ute)]
    Hm = next((x.shape[1] for x in vecs if x is not None), 1)
    _need_cuda(q, k, v, bounds, sched, *vecs)
    if scale is None:
        scale = d ** -0.5
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if lse is None else lse
    _check(lib.fm_fwd_rows(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), B, H, Nq, Nk, int(q_off), d,
                           *[_ptr(x) for x in vecs], Hm, _ptr(bounds), _ptr(sched), int(bool(causal)), float(scale),
                           _ptr(out),
                           _ptr(lse), _stream(stream)), "fm_fwd_rows")
    return out, lse


def fm_bwd_rows(q, k, v, out, dout, lse, q_off: int, lts=None, lte=None, uts=None, ute=None, bounds=None,
                causal=False, scale=None, dq=None, dk=None, dv=None, workspace=None, stream=None, sched=None):
    """(dq, dk, dv) of the row block: dq for its rows, dk / dv the contributions of its rows."""
    lib = load_library()
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    vecs = [_vec(x) for x in (lts, lte, uts, ute)]
    Hm = next((x.shape[1] for x in vecs if x is not None), 1)
    _need_cuda(q, k, v, out, dout, lse, bounds, sched, *vecs)
    if scale is None:
        scale = d ** -0.5
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = fm_bwd_workspace_bytes(q.dtype, B, H, Nq, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib.fm_bwd_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _dtype_code(q), B, H, Nq,
                           Nk, int(q_off), d, *[_ptr(x) for x in vecs], Hm, _ptr(bounds), _ptr(sched),
                           int(bool(causal)),
                           float(scale), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel(),
                           _stream(stream)), "fm_bwd_rows")
    return dq, dk, dv


def fm_lsh_buckets(x, rot, nb: int, out=None, stream=None):
    """int32 [B, H, N] bucket of each row of x [B, H, N, d]: argmax of [x R, -x R] for rot float32
    [Hr, d, nb / 2] (Hr = 1 or H)."""
    lib = load_library()
    B, H, N, d = x.shape
    _need_cuda(x, rot)
    if rot.dtype != torch.float32:
        raise TypeError("rot must be float32")
    out = torch.empty((B, H, N), dtype=torch.int32, device=x.device) if out is None else out
    _check(lib.fm_lsh_buckets(_ptr(x), _dtype_code(x), B, H, N, d, _ptr(rot), rot.shape[0], nb, _ptr(out),
                              _stream(stream)), "fm_lsh_buckets")
    return out


def fm_bucket_sort(qbucket, kbucket, nb: int, stream=None):
    """(qidx, qpos, kidx, kpos, vectors): stable reordering of queries and keys by bucket (int32 [B, H, N]
    inputs; values outside [0, nb) are dropped tokens) and the sorted problem's four int32 [B, H, N] mask
    vectors, to be run with causal = False and Hm = H."""
    lib = load_library()
    qbucket, kbucket = _vec(qbucket), _vec(kbucket)
    _need_cuda(qbucket, kbucket)
    B, H, N = qbucket.shape
    new = lambda: torch.empty((B, H, N), dtype=torch.int32, device=qbucket.device)  # noqa: E731
    qidx, qpos, kidx, kpos = new(), new(), new(), new()
    vecs = [new() for _ in range(4)]
    _check(lib.fm_bucket_sort(_ptr(qbucket), _ptr(kbucket), B, H, N, nb, _ptr(qidx), _ptr(qpos), _ptr(kidx),
                              _ptr(kpos), *[_ptr(x) for x in vecs], _stream(stream)), "fm_bucket_sort")
    return qidx, qpos, kidx, kpos, vecs
