"""Shared helpers for the GPU parity tests: seeded cases, the HIP path through the C ABI, the oracle,
and the comparison bars (bf16: out max-abs 1e-2, lse max-abs 1e-3, dq/dk/dv relative Frobenius 2e-2;
float32: 1e-4, 1e-5 and 1e-4)."""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch

import workloads as W
from oracle import attention as OA
from oracle import tiles as OT

TOL = {
    "bf16": {"out": 1e-2, "lse": 1e-3, "grad": 2e-2},
    "f32": {"out": 1e-4, "lse": 1e-5, "grad": 1e-4},
}
TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


@dataclass
class Case:
    name: str
    spec: W.MaskSpec
    B: int
    H: int
    N: int
    d: int
    dtype: str
    q: torch.Tensor  # CPU, in the compute dtype
    k: torch.Tensor
    v: torch.Tensor
    do: torch.Tensor

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.d)


def make_case(cfg, mask, B, H, N, d, dtype="bf16", mask_index=None, spec=None, name=None) -> Case:
    if spec is None:
        spec = W.make_mask(cfg, mask, B, H, N, mask_index)
    mi = mask_index if mask_index is not None else 0
    ts = W.make_tensors(cfg, mi, B, H, N, d)
    q, k, v, do = (torch.from_numpy(x).to(TORCH_DT[dtype]) for x in ts)
    return Case(name or f"cfg{cfg}-{mask}-B{B}H{H}N{N}d{d}-{dtype}", spec, B, H, N, d, dtype, q, k, v, do)


def device_vectors(spec: W.MaskSpec, dev="cuda"):
    return [None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in spec.vectors()]


def run_gpu(case: Case, fm, dev="cuda", sched=False):
    """fm_tile_bounds -> (fm_tile_schedule if sched) -> fm_fwd -> fm_bwd through the C ABI; returns CPU
    tensors."""
    q, k, v, do = (t.to(dev) for t in (case.q, case.k, case.v, case.do))
    vecs = device_vectors(case.spec, dev)
    bounds = None
    if any(x is not None for x in vecs):
        bounds = fm.fm_tile_bounds(*vecs, case.B, case.spec.Hm, case.N)
    s = fm.fm_tile_schedule(bounds, case.B, case.spec.Hm, case.N, case.N, case.spec.causal,
                            device=torch.device(dev)) if sched else None
    out, lse = fm.fm_fwd(q, k, v, *vecs, bounds=bounds, sched=s, causal=case.spec.causal, scale=case.scale)
    dq, dk, dv = fm.fm_bwd(q, k, v, out, do, lse, *vecs, bounds=bounds, sched=s, causal=case.spec.causal,
                           scale=case.scale)
    torch.cuda.synchronize()
    res = {"out": out, "lse": lse, "dq": dq, "dk": dk, "dv": dv, "bounds": bounds}
    return {k_: (None if t is None else t.cpu()) for k_, t in res.items()}


def f64(t: torch.Tensor) -> np.ndarray:
    return t.to(torch.float64).numpy()


def run_oracle(case: Case):
    out, lse, dq, dk, dv, _ = OA.fwd_bwd(f64(case.q), f64(case.k), f64(case.v), f64(case.do),
                                         case.spec.vectors(), case.spec.causal, case.scale, case.spec.Hm)
    return {"out": out, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


def rel_fro(a: np.ndarray, ref: np.ndarray) -> float:
    """||a - ref||_F / ||ref||_F, the denominator floored at an RMS of 1e-4 so that an identically
    zero reference (a single-key row has dS = 0 exactly) compares rounding noise absolutely."""
    den = max(float(np.linalg.norm(ref)), 1e-4 * math.sqrt(max(ref.size, 1)))
    return float(np.linalg.norm(a - ref) / den)


def compare(gpu: dict, ref: dict, dtype: str, report: dict | None = None):
    """Assert the bars; returns the measured errors."""
    tol = TOL[dtype]
    errs = {}
    out_g = f64(gpu["out"])
    errs["out_maxabs"] = float(np.max(np.abs(out_g - ref["out"]), initial=0.0))
    lse_g = gpu["lse"].numpy().astype(np.float64)
    fin_g, fin_r = np.isfinite(lse_g), np.isfinite(ref["lse"])
    assert np.array_equal(fin_g, fin_r), "rows without any unmasked key differ"
    assert np.all(lse_g[~fin_g] == -np.inf) and np.all(ref["lse"][~fin_r] == -np.inf)
    errs["lse_maxabs"] = float(np.max(np.abs(lse_g[fin_g] - ref["lse"][fin_r]), initial=0.0))
    for name in ("dq", "dk", "dv"):
        errs[f"{name}_relF"] = rel_fro(f64(gpu[name]), ref[name])
    if report is not None:
        report.update(errs)
    assert errs["out_maxabs"] <= tol["out"], errs
    assert errs["lse_maxabs"] <= tol["lse"], errs
    for name in ("dq", "dk", "dv"):
        assert errs[f"{name}_relF"] <= tol["grad"], errs
    # rows without any key: out row and dq row exactly zero
    dead = ~fin_r
    if dead.any():
        assert np.all(out_g[dead] == 0.0) and np.all(f64(gpu["dq"])[dead] == 0.0)
    return errs


def oracle_bounds(spec: W.MaskSpec):
    return OT.tile_bounds(spec.vectors(), spec.B, spec.Hm, spec.N)


def run_gpu_compacted(case: Case, fm, dev="cuda"):
    """The same results through key compaction: fm_compact_keys -> fm_gather_rows (K, V) ->
    fm_tile_bounds -> fm_fwd / fm_bwd without the causal flag -> fm_gather_rows (dK, dV back)."""
    q, k, v, do = (t.to(dev) for t in (case.q, case.k, case.v, case.do))
    vecs = device_vectors(case.spec, dev)
    Hm = case.spec.Hm
    kidx, kpos, counts, vecs2 = fm.fm_compact_keys(*vecs, case.B, Hm, case.N, case.spec.causal)
    k2, v2 = fm.fm_gather_rows(k, kidx), fm.fm_gather_rows(v, kidx)
    bounds = fm.fm_tile_bounds(*vecs2, case.B, Hm, case.N)
    out, lse = fm.fm_fwd(q, k2, v2, *vecs2, bounds=bounds, causal=False, scale=case.scale)
    dq, dk2, dv2 = fm.fm_bwd(q, k2, v2, out, do, lse, *vecs2, bounds=bounds, causal=False, scale=case.scale)
    dk, dv = fm.fm_gather_rows(dk2, kpos), fm.fm_gather_rows(dv2, kpos)
    torch.cuda.synchronize()
    assert int(counts.min()) >= 0, "mask not compactable"
    res = {"out": out, "lse": lse, "dq": dq, "dk": dk, "dv": dv, "kidx": kidx, "kpos": kpos, "counts": counts,
           "vecs2": vecs2}
    return {k_: ([x.cpu() for x in t] if isinstance(t, list) else t.cpu()) for k_, t in res.items()}


def run_gpu_hash(fm, q, k, v, do, qb, kb, nb: int, scale: float, mapped: bool = False):
    """Hash-bucket attention through the C ABI on device tensors: fm_bucket_sort, fm_gather_rows of Q, dO
    (by qidx) and K, V (by kidx), fm_tile_bounds, fm_fwd / fm_bwd without the causal flag on the sorted
    problem, then fm_gather_rows of out, dq (by qpos) and dk, dv (by kpos) back to the original order.
    With `mapped` the attention runs as fm_fwd_mapped / fm_bwd_mapped, which store out, dq, dk, dv
    straight into the original order through qidx and kidx, as the benchmark's hash step does.
    lse stays in sorted order in the library; it is put back in original order here, on the host side
    of the comparison. Returns CPU tensors."""
    B, H, N, d = q.shape
    qidx, qpos, kidx, kpos, vecs = fm.fm_bucket_sort(qb, kb, nb)
    qs, dos = fm.fm_gather_rows(q, qidx), fm.fm_gather_rows(do, qidx)
    ks, vs = fm.fm_gather_rows(k, kidx), fm.fm_gather_rows(v, kidx)
    bounds = fm.fm_tile_bounds(*vecs, B, H, N)
    if mapped:
        out, lse_s = fm.fm_fwd_mapped(qs, ks, vs, qidx, *vecs, bounds=bounds, causal=False, scale=scale)
        dq, dk, dv = fm.fm_bwd_mapped(qs, ks, vs, out, dos, lse_s, qidx, kidx, *vecs, bounds=bounds,
                                      causal=False, scale=scale)
    else:
        outs, lse_s = fm.fm_fwd(qs, ks, vs, *vecs, bounds=bounds, causal=False, scale=scale)
        dqs, dks, dvs = fm.fm_bwd(qs, ks, vs, outs, dos, lse_s, *vecs, bounds=bounds, causal=False,
                                  scale=scale)
        out, dq = fm.fm_gather_rows(outs, qpos), fm.fm_gather_rows(dqs, qpos)
        dk, dv = fm.fm_gather_rows(dks, kpos), fm.fm_gather_rows(dvs, kpos)
    torch.cuda.synchronize()
    lse = torch.gather(lse_s.cpu(), 2, qpos.cpu().long())
    res = {"out": out, "dq": dq, "dk": dk, "dv": dv, "qidx": qidx, "qpos": qpos, "kidx": kidx, "kpos": kpos}
    res = {k_: t.cpu() for k_, t in res.items()}
    res["lse"] = lse
    res["vecs"] = [x.cpu() for x in vecs]
    return res
