"""Pins of the fp64 attention oracle against brute force, closed forms, an independent autograd
library, finite differences and invariants of the softmax-attention gradient (CPU)."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as OA
from oracle import masks as OM


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _case(seed, N, d, family="causal_document"):
    rng = np.random.default_rng([seed, N, d])
    q, k, v, do = (_rand(rng, N, d) for _ in range(4))
    if family == "causal_document":
        cuts = W.uniform_cuts(rng, min(3, N - 1), 1, N - 1) if N > 1 else []
        spec = W.encode_causal_document(W.doc_boundaries_from_cuts(cuts, N), N)
    elif family == "key_drop":
        spec = W.encode_causal_key_drop([np.sort(rng.choice(N, size=N // 3, replace=False))], N)
    elif family == "prefix_lm":
        spec = W.encode_prefix_lm(N // 2, N)
    elif family == "bidirectional_document":
        spec = W.encode_bidirectional_document(W.doc_boundaries_from_cuts([N // 3], N), N)
    else:
        raise KeyError(family)
    return q, k, v, do, spec


FAMILIES = ["causal_document", "key_drop", "prefix_lm", "bidirectional_document"]


# ------------------------------------------------------------------ forward

@pytest.mark.parametrize("family", FAMILIES)
@pytest.mark.parametrize("N,d", [(1, 3), (5, 2), (17, 4), (64, 8)])
def test_forward_matches_brute_force(family, N, d):
    q, k, v, do, spec = _case(1, N, d, family)
    vecs = spec.column_slice(0, 0)
    scale = 1.0 / math.sqrt(d)
    masked = OM.dense_masked(*vecs, spec.causal, N)
    out, lse, *_ = OA.fwd_bwd_head(q, k, v, do, vecs, spec.causal, scale, row_block=7)
    bout, blse = OA.brute_force_forward(q, k, v, masked, scale)
    assert np.max(np.abs(out - bout)) <= 1e-12
    fin = np.isfinite(blse)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.max(np.abs(lse[fin] - blse[fin]), initial=0.0) <= 1e-12


@pytest.mark.parametrize("family", FAMILIES)
def test_softmax_rows(family):
    N, d = 96, 16
    q, k, v, do, spec = _case(2, N, d, family)
    vecs = spec.column_slice(0, 0)
    masked = OM.dense_masked(*vecs, spec.causal, N)
    res = OA.attend_rows(q, k, v, do, masked, 0.3)
    P = res["P"]
    alive = ~masked.all(axis=1)
    assert np.all(P >= 0)
    assert np.all(P[masked] == 0)
    assert np.max(np.abs(P[alive].sum(axis=1) - 1.0)) <= 1e-12
    assert np.all(P[~alive] == 0)


def test_fully_masked_rows_convention():
    # dropping key 0 under causal leaves query 0 with no key at all
    N, d = 12, 4
    rng = np.random.default_rng(3)
    q, k, v, do = (_rand(rng, N, d) for _ in range(4))
    spec = W.encode_causal_key_drop([np.array([0, 5])], N)
    vecs = spec.column_slice(0, 0)
    out, lse, dq, dk, dv = OA.fwd_bwd_head(q, k, v, do, vecs, True, 0.5)
    assert np.all(out[0] == 0) and lse[0] == -np.inf and np.all(dq[0] == 0)
    # the dead row contributes nothing: zeroing its q / dO changes no gradient of the keys
    q2, do2 = q.copy(), do.copy()
    q2[0] = 123.0
    do2[0] = -77.0
    _, _, _, dk2, dv2 = OA.fwd_bwd_head(q2, k, v, do2, vecs, True, 0.5)
    assert np.array_equal(dk, dk2) and np.array_equal(dv, dv2)
    # a dropped key receives no gradient
    assert np.all(dk[5] == 0) and np.all(dv[5] == 0)


def test_closed_form_zero_query_is_mean():
    # q = 0 makes every unmasked score equal: out = mean of the unmasked values, lse = ln(count)
    N, d = 40, 6
    rng = np.random.default_rng(4)
    k, v, do = (_rand(rng, N, d) for _ in range(3))
    q = np.zeros((N, d))
    spec = W.encode_causal_window(9, N)
    vecs = spec.column_slice(0, 0)
    out, lse, *_ = OA.fwd_bwd_head(q, k, v, do, vecs, True, 0.7)
    for i in range(N):
        js = [j for j in range(N) if 0 <= i - j < 9]
        assert np.allclose(out[i], v[js].mean(axis=0), atol=1e-13, rtol=0)
        assert abs(lse[i] - math.log(len(js))) <= 1e-13


def test_closed_form_single_key_and_constant_values():
    N, d = 10, 3
    rng = np.random.default_rng(5)
    q, k, v, do = (_rand(rng, N, d) for _ in range(4))
    # under the causal document mask with every token its own document, row i sees only key i
    spec = W.encode_causal_document(np.arange(N + 1), N)
    vecs = spec.column_slice(0, 0)
    out, lse, dq, dk, dv = OA.fwd_bwd_head(q, k, v, do, vecs, True, 0.9)
    assert np.allclose(out, v, atol=1e-14, rtol=0)
    assert np.allclose(lse, 0.9 * np.sum(q * k, axis=1), atol=1e-13, rtol=0)
    assert np.allclose(dq, 0, atol=1e-14) and np.allclose(dk, 0, atol=1e-14)
    assert np.allclose(dv, do, atol=1e-14, rtol=0)
    # constant values: every row's output is that constant
    vc = np.tile(rng.standard_normal(d), (N, 1))
    out2, *_ = OA.fwd_bwd_head(q, k, vc, do, W.encode_causal(N).column_slice(0, 0), True, 0.9)
    assert np.allclose(out2, vc, atol=1e-13, rtol=0)


def test_hand_computed_two_token_example():
    # N = 2, d = 1, scale 1, causal: q = (0, ln 3), k = (1, 0), v = (4, 8), dO = (1, 1).
    # row 0 sees key 0 only: out 4, lse 0. row 1: scores (ln 3, 0) -> P = (3/4, 1/4), out = 5, lse = ln 4.
    # backward: dP_1 = (4, 8), D_1 = 5, dS_1 = (-3/4, 3/4), dq_1 = -3/4; dq_0 = 0;
    # dk = (-3/4 ln 3, 3/4 ln 3), dv = (7/4, 1/4).
    l3 = math.log(3.0)
    q = np.array([[0.0], [l3]])
    k = np.array([[1.0], [0.0]])
    v = np.array([[4.0], [8.0]])
    do = np.array([[1.0], [1.0]])
    out, lse, dq, dk, dv = OA.fwd_bwd_head(q, k, v, do, (None,) * 4, True, 1.0)
    assert np.allclose(out[:, 0], [4.0, 5.0], atol=1e-14)
    assert np.allclose(lse, [0.0, math.log(4.0)], atol=1e-14)
    assert np.allclose(dq[:, 0], [0.0, -0.75], atol=1e-14)
    assert np.allclose(dk[:, 0], [-0.75 * l3, 0.75 * l3], atol=1e-14)
    assert np.allclose(dv[:, 0], [1.75, 0.25], atol=1e-14)


# ------------------------------------------------------------------ backward

def _torch_reference(q, k, v, do, masked, scale):
    """Independent gradient: torch CPU float64 autograd of masked softmax attention (live rows only)."""
    alive = torch.from_numpy(~masked.all(axis=1))
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    tm = torch.from_numpy(masked)
    s = (tq @ tk.T) * scale
    s = s.masked_fill(tm, float("-inf"))
    s = torch.where(alive[:, None], s, torch.zeros_like(s))
    p = torch.softmax(s, dim=-1)
    p = torch.where(alive[:, None], p, torch.zeros_like(p))
    out = p @ tv
    (out * torch.from_numpy(do)).sum().backward()
    return out.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("family", FAMILIES)
@pytest.mark.parametrize("N,d", [(7, 3), (50, 8), (130, 16)])
def test_backward_matches_torch_autograd(family, N, d):
    q, k, v, do, spec = _case(6, N, d, family)
    vecs = spec.column_slice(0, 0)
    scale = 1.0 / math.sqrt(d)
    masked = OM.dense_masked(*vecs, spec.causal, N)
    out, lse, dq, dk, dv = OA.fwd_bwd_head(q, k, v, do, vecs, spec.causal, scale, row_block=32)
    tout, tdq, tdk, tdv = _torch_reference(q, k, v, do, masked, scale)
    for a, b in ((out, tout), (dq, tdq), (dk, tdk), (dv, tdv)):
        assert np.max(np.abs(a - b)) <= 1e-12


@pytest.mark.parametrize("family", FAMILIES)
def test_backward_matches_finite_differences(family):
    N, d, h = 9, 3, 1e-6
    q, k, v, do, spec = _case(7, N, d, family)
    vecs = spec.column_slice(0, 0)
    scale = 0.8

    def loss(q_, k_, v_):
        out, *_ = OA.fwd_bwd_head(q_, k_, v_, do, vecs, spec.causal, scale)
        return OA.loss_from_out(out, do)

    _, _, dq, dk, dv = OA.fwd_bwd_head(q, k, v, do, vecs, spec.causal, scale)
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        args = [q, k, v]
        fd = np.zeros_like(grad)
        for idx in np.ndindex(*grad.shape):
            plus = [a.copy() for a in args]
            minus = [a.copy() for a in args]
            plus[which][idx] += h
            minus[which][idx] -= h
            fd[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        assert np.max(np.abs(fd - grad)) <= 1e-7, which


@pytest.mark.parametrize("family", FAMILIES)
def test_backward_invariants(family):
    N, d = 150, 8
    q, k, v, do, spec = _case(8, N, d, family)
    vecs = spec.column_slice(0, 0)
    masked = OM.dense_masked(*vecs, spec.causal, N)
    alive = ~masked.all(axis=1)
    out, lse, dq, dk, dv = OA.fwd_bwd_head(q, k, v, do, vecs, spec.causal, 0.4, row_block=64)
    # sum_j P_ij = 1 makes the key-sum of dV the sum of dO over live rows
    assert np.allclose(dv.sum(axis=0), do[alive].sum(axis=0), atol=1e-11)
    # sum_j dS_ij = 0 makes the key-sum of dK vanish
    assert np.allclose(dk.sum(axis=0), 0.0, atol=1e-11)
    # the D identity: sum_j P_ij dP_ij = dO_i . out_i
    res = OA.attend_rows(q, k, v, do, masked, 0.4)
    assert np.allclose(res["D"], np.sum(do * out, axis=1), atol=1e-12)
    # with all keys equal, every score in a row is equal, so dS rows vanish and dQ = 0
    k_eq = np.tile(k[:1], (N, 1))
    _, _, dq_eq, _, _ = OA.fwd_bwd_head(q, k_eq, v, do, vecs, spec.causal, 0.4)
    assert np.allclose(dq_eq, 0.0, atol=1e-12)


def test_probes_equal_full_computation():
    N, d = 300, 8
    q, k, v, do, spec = _case(9, N, d, "key_drop")
    vecs = spec.column_slice(0, 0)
    out, lse, dq, dk, dv = OA.fwd_bwd_head(q, k, v, do, vecs, True, 0.35, row_block=64)
    rows = np.array([0, 1, 77, 128, 299])
    po, pl, pD, pdq = OA.rows_probe(q, k, v, do, vecs, True, 0.35, rows)
    assert np.allclose(po, out[rows], atol=1e-12) and np.allclose(pdq, dq[rows], atol=1e-12)
    assert np.array_equal(np.isfinite(pl), np.isfinite(lse[rows]))
    fin = np.isfinite(pl)
    assert np.allclose(pl[fin], lse[rows][fin], atol=1e-12)
    cols = np.array([0, 3, 150, 299])
    pdk, pdv = OA.cols_probe(q, k, v, do, vecs, True, 0.35, cols)
    assert np.allclose(pdk, dk[cols], atol=1e-12) and np.allclose(pdv, dv[cols], atol=1e-12)


def test_multihead_driver_matches_per_head():
    B, H, N, d = 2, 3, 70, 4
    spec = W.make_mask(3, "causal_key_drop", B, H, N, 2)
    q, k, v, do = (np.random.default_rng(i).standard_normal((B, H, N, d)) for i in range(4))
    out, lse, dq, dk, dv, used = OA.fwd_bwd(q, k, v, do, spec.vectors(), True, 0.5, spec.Hm, workers=3)
    assert used == 3
    for b in range(B):
        for h in range(H):
            o, l_, gq, gk, gv = OA.fwd_bwd_head(q[b, h], k[b, h], v[b, h], do[b, h],
                                                spec.column_slice(b, h), True, 0.5)
            assert np.array_equal(o, out[b, h]) and np.array_equal(gk, dk[b, h])


# ------------------------------------------------------------------ the pins catch planted mistakes

def test_pins_catch_planted_mistakes(monkeypatch):
    """Plant plausible slips in the oracle and check a pin above would fail for each."""
    N, d = 17, 4
    q, k, v, do, spec = _case(10, N, d, "causal_document")
    vecs = spec.column_slice(0, 0)
    masked = OM.dense_masked(*vecs, True, N)
    bout, _ = OA.brute_force_forward(q, k, v, masked, 0.5)
    _, tdq, tdk, tdv = _torch_reference(q, k, v, do, masked, 0.5)
    real = OA.attend_rows

    def flipped_mask(q_rows, k_, v_, do_rows, m, scale):
        return real(q_rows, k_, v_, do_rows, ~m if m.shape[0] == m.shape[1] else m, scale)

    def missing_d(q_rows, k_, v_, do_rows, m, scale):
        r = real(q_rows, k_, v_, do_rows, m, scale)
        r["dS"] = r["P"] * (np.asarray(do_rows) @ np.asarray(v_).T)  # dropped the -D term
        return r

    def transposed_scores(q_rows, k_, v_, do_rows, m, scale):
        return real(k_[: len(q_rows)], q_rows[: len(k_)], v_, do_rows, m, scale)

    for planted, check in ((flipped_mask, "fwd"), (missing_d, "dk"), (transposed_scores, "fwd")):
        monkeypatch.setattr(OA, "attend_rows", planted)
        out, _, dq, dk, dv = OA.fwd_bwd_head(q, k, v, do, vecs, True, 0.5, row_block=N)
        if check == "fwd":
            assert np.max(np.abs(out - bout)) > 1e-6
        else:
            assert np.max(np.abs(dk - tdk)) > 1e-6
        monkeypatch.setattr(OA, "attend_rows", real)
