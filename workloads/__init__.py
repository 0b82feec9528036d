"""Seeded synthetic inputs for column-wise-mask (FlashMask) attention.

This module is shared by the tests, the benchmark and the smoke check. It holds no attention, softmax
or tile arithmetic: only seeded random draws (document cuts, answer cuts, dropped keys, kept blocks,
Q/K/V/dO tensors) and the caller-side encoding of each mask family into the four per-key-column
query-axis boundary vectors.

Mask semantics (FlashMask abstract, papers.pytorch.kr 2410.01359; FlashMask-3 summary, readmex.ai):
each key column j carries four int32 query-axis bounds LTS_j, LTE_j, UTS_j, UTE_j. Query row i is
masked for column j when LTS_j <= i < LTE_j or UTS_j <= i < UTE_j, or, with the causal flag, i < j.
A vector pair left as None is the empty interval. The FlashMask-3 summary names the families encoded
here: document, prefix-LM, share-question, sliding-window and block-sparse; per-head key dropping is
the sparse causal attention of the SCFA review (nubint.ai), section "proposed method".

Seeds: ``np.random.default_rng([cfg, mask, purpose])`` with purpose 0 = mask draws, 1 = Q, 2 = K,
3 = V, 4 = dO. Tensors are N(0, 1) float32; the bf16 runs round them to bf16 (round to nearest even)
and the oracle consumes exactly the rounded values.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

PURPOSE_MASK, PURPOSE_Q, PURPOSE_K, PURPOSE_V, PURPOSE_DO = 0, 1, 2, 3, 4
PURPOSE_ROT, PURPOSE_BUCKET = 5, 6


@dataclass
class MaskSpec:
    """Column-wise mask: causal flag plus up to two interval pairs, each int32 [B, Hm, N] or None."""

    N: int
    B: int
    Hm: int
    causal: bool
    lts: Optional[np.ndarray] = None
    lte: Optional[np.ndarray] = None
    uts: Optional[np.ndarray] = None
    ute: Optional[np.ndarray] = None
    family: str = ""
    params: dict = field(default_factory=dict)

    def vectors(self):
        return self.lts, self.lte, self.uts, self.ute

    def column_slice(self, b: int, h: int):
        """The four vectors for batch b, head h (Hm = 1 broadcasts over heads); None stays None."""
        hm = h if self.Hm > 1 else 0
        return tuple(None if x is None else x[b, hm] for x in self.vectors())


def _full(B, Hm, N, value):
    return np.full((B, Hm, N), value, dtype=np.int32)


def _as_bhn(row, B, Hm):
    row = np.asarray(row, dtype=np.int64)
    return np.ascontiguousarray(np.broadcast_to(row, (B, Hm, row.shape[-1])).astype(np.int32))


# ---------------------------------------------------------------- documents and cuts (seeded draws)

def uniform_cuts(rng: np.random.Generator, n_cuts: int, lo: int, hi: int) -> np.ndarray:
    """``n_cuts`` distinct integers drawn uniformly from [lo, hi], sorted."""
    if n_cuts <= 0:
        return np.zeros(0, dtype=np.int64)
    return np.sort(rng.choice(np.arange(lo, hi + 1), size=n_cuts, replace=False)).astype(np.int64)


def doc_boundaries_from_cuts(cuts: Sequence[int], N: int) -> np.ndarray:
    """0 = s_0 < s_1 < ... < s_K = N from the interior cut points."""
    return np.concatenate([[0], np.asarray(cuts, dtype=np.int64), [N]]).astype(np.int64)


def loguniform_doc_boundaries(rng: np.random.Generator, N: int, lo: int, hi: int) -> np.ndarray:
    """Document lengths round(exp(U(ln lo, ln hi))) drawn until they cover N; the last is truncated."""
    bounds = [0]
    while bounds[-1] < N:
        length = int(round(float(np.exp(rng.uniform(np.log(lo), np.log(hi))))))
        bounds.append(min(N, bounds[-1] + max(1, length)))
    return np.asarray(bounds, dtype=np.int64)


def doc_end_per_column(bounds: np.ndarray, N: int) -> np.ndarray:
    """For each column j, the end s_{doc(j)+1} of the document holding j."""
    j = np.arange(N)
    k = np.searchsorted(bounds, j, side="right") - 1
    return bounds[k + 1]


def doc_start_per_column(bounds: np.ndarray, N: int) -> np.ndarray:
    j = np.arange(N)
    k = np.searchsorted(bounds, j, side="right") - 1
    return bounds[k]


# ---------------------------------------------------------------- family encoders (caller side)

def encode_full(N, B=1, Hm=1) -> MaskSpec:
    return MaskSpec(N, B, Hm, False, family="full")


def encode_causal(N, B=1, Hm=1) -> MaskSpec:
    """Plain causal mask as the causal flag with every vector pair empty."""
    return MaskSpec(N, B, Hm, True, family="causal")


def encode_causal_by_vectors(N, B=1, Hm=1) -> MaskSpec:
    """The same causal mask with the flag off: UT masks rows [0, j) of column j."""
    j = np.arange(N)
    return MaskSpec(N, B, Hm, False, uts=_as_bhn(np.zeros(N), B, Hm), ute=_as_bhn(j, B, Hm),
                    family="causal_by_vectors")


def encode_causal_document(bounds, N, B=1, Hm=1) -> MaskSpec:
    """Causal packing of documents: column j is hidden from every row at or past its document's end."""
    end = doc_end_per_column(np.asarray(bounds), N)
    return MaskSpec(N, B, Hm, True, lts=_as_bhn(end, B, Hm), lte=_full(B, Hm, N, N),
                    family="causal_document", params={"bounds": np.asarray(bounds)})


def encode_causal_window(w, N, B=1, Hm=1) -> MaskSpec:
    """Causal sliding window of width w: row i sees keys j with 0 <= i - j < w."""
    j = np.arange(N)
    return MaskSpec(N, B, Hm, True, lts=_as_bhn(np.minimum(j + w, N), B, Hm), lte=_full(B, Hm, N, N),
                    family="causal_window", params={"w": w})


def encode_causal_document_window(bounds, w, N, B=1, Hm=1) -> MaskSpec:
    end = doc_end_per_column(np.asarray(bounds), N)
    j = np.arange(N)
    return MaskSpec(N, B, Hm, True, lts=_as_bhn(np.minimum(end, j + w), B, Hm), lte=_full(B, Hm, N, N),
                    family="causal_document_window", params={"bounds": np.asarray(bounds), "w": w})


def encode_prefix_lm(P, N, B=1, Hm=1) -> MaskSpec:
    """Prefix-LM: keys in [0, P) are seen by every row; later keys only causally (no causal flag)."""
    j = np.arange(N)
    return MaskSpec(N, B, Hm, False, uts=_as_bhn(np.zeros(N), B, Hm),
                    ute=_as_bhn(np.where(j >= P, j, 0), B, Hm), family="prefix_lm", params={"P": P})


def encode_share_question(Q, answer_bounds, N, B=1, Hm=1) -> MaskSpec:
    """One question [0, Q) then answers [a_k, a_{k+1}); each answer sees the question and itself."""
    a = np.asarray(answer_bounds, dtype=np.int64)
    j = np.arange(N)
    k = np.searchsorted(a, j, side="right") - 1
    ans_end = a[np.minimum(k + 1, len(a) - 1)]
    lts = np.where(j < Q, N, ans_end)
    return MaskSpec(N, B, Hm, True, lts=_as_bhn(lts, B, Hm), lte=_full(B, Hm, N, N),
                    family="share_question", params={"Q": Q, "answer_bounds": a})


def encode_causal_key_drop(dropped_per_head: Sequence[np.ndarray], N, B=1) -> MaskSpec:
    """Causal attention with a per-head set of dropped key columns (each dropped column fully masked)."""
    H = len(dropped_per_head)
    lts = np.full((B, H, N), N, dtype=np.int32)
    lte = np.full((B, H, N), N, dtype=np.int32)
    for h, drop in enumerate(dropped_per_head):
        lts[:, h, drop] = 0
    return MaskSpec(N, B, H, True, lts=lts, lte=lte, family="causal_key_drop",
                    params={"dropped": [np.asarray(x) for x in dropped_per_head]})


def encode_causal_document_block_sparse(bounds, kept_blocks, block, N, B=1, Hm=1) -> MaskSpec:
    """Causal documents where only the listed 'block'-wide key-column blocks are kept."""
    end = doc_end_per_column(np.asarray(bounds), N)
    j = np.arange(N)
    kept = np.isin(j // block, np.asarray(kept_blocks))
    lts = np.where(kept, end, 0)
    return MaskSpec(N, B, Hm, True, lts=_as_bhn(lts, B, Hm), lte=_full(B, Hm, N, N),
                    family="causal_document_block_sparse",
                    params={"bounds": np.asarray(bounds), "kept_blocks": np.asarray(kept_blocks),
                            "block": block})


def encode_bidirectional_document(bounds, N, B=1, Hm=1) -> MaskSpec:
    """Documents with full attention inside each document and none across (no causal flag)."""
    b = np.asarray(bounds)
    return MaskSpec(N, B, Hm, False, lts=_as_bhn(doc_end_per_column(b, N), B, Hm),
                    lte=_full(B, Hm, N, N), uts=_as_bhn(np.zeros(N), B, Hm),
                    ute=_as_bhn(doc_start_per_column(b, N), B, Hm), family="bidirectional_document",
                    params={"bounds": b})


# ---------------------------------------------------------------- the five synthetic workloads

@dataclass(frozen=True)
class Config:
    index: int
    name: str
    B: int
    H: int
    N: int
    d: int
    masks: tuple
    dtypes: tuple = ("bf16",)


CONFIGS = (
    Config(0, "tiny_causal_document", 1, 2, 256, 64, ("causal_document",), ("f32", "bf16")),
    Config(1, "bert_base", 8, 12, 2048, 64, ("full", "causal")),
    Config(2, "sft_packing", 1, 32, 8192, 128, ("causal_document", "causal_window_1024")),
    Config(3, "dpo_rm_share_question", 1, 32, 32768, 128,
           ("share_question", "prefix_lm", "causal_key_drop")),
    Config(4, "long_context", 1, 8, 131072, 128,
           ("causal_document", "causal_document_window_4096", "causal_document_block_sparse")),
)


def rng_for(cfg: int, mask: int, purpose: int) -> np.random.Generator:
    return np.random.default_rng([cfg, mask, purpose])


def make_mask(cfg: int, mask_name: str, B: int, H: int, N: int, mask_index: Optional[int] = None) -> MaskSpec:
    """Seeded mask of one family at the given shape. The defaults follow the five workloads; a smaller
    N keeps the same recipe scaled to N (question N/4, prefix N/2, 30% key drop, 10% block density)."""
    if mask_index is None:
        mask_index = CONFIGS[cfg].masks.index(mask_name) if cfg < len(CONFIGS) and \
            mask_name in CONFIGS[cfg].masks else 0
    rng = rng_for(cfg, mask_index, PURPOSE_MASK)
    if mask_name == "full":
        return encode_full(N, B)
    if mask_name == "causal":
        return encode_causal(N, B)
    if mask_name == "causal_by_vectors":
        return encode_causal_by_vectors(N, B)
    if mask_name == "causal_document":
        if cfg == 4:
            lo, hi = (1024, 32768) if N >= 32768 else (max(1, N // 128), max(2, N // 4))
            bounds = loguniform_doc_boundaries(rng, N, lo, hi)
        elif cfg == 0:
            bounds = doc_boundaries_from_cuts(uniform_cuts(rng, min(2, N - 1), 1, N - 1), N)
        else:
            K = int(rng.integers(2, 13))
            bounds = doc_boundaries_from_cuts(uniform_cuts(rng, min(K - 1, N - 1), 1, N - 1), N)
        return encode_causal_document(bounds, N, B)
    if mask_name.startswith("causal_window_"):
        w = int(mask_name.rsplit("_", 1)[1])
        return encode_causal_window(min(w, N), N, B)
    if mask_name.startswith("causal_document_window_"):
        w = int(mask_name.rsplit("_", 1)[1])
        lo, hi = (1024, 32768) if N >= 32768 else (max(1, N // 128), max(2, N // 4))
        bounds = loguniform_doc_boundaries(rng, N, lo, hi)
        return encode_causal_document_window(bounds, w if N >= 32768 else max(1, N // 32), N, B)
    if mask_name == "causal_document_block_sparse":
        lo, hi = (1024, 32768) if N >= 32768 else (max(1, N // 128), max(2, N // 4))
        bounds = loguniform_doc_boundaries(rng, N, lo, hi)
        nblk = -(-N // 128)
        keep = max(1, int(round(0.1 * nblk))) if N >= 32768 or nblk >= 10 else max(1, nblk // 3)
        kept = np.sort(rng.choice(nblk, size=keep, replace=False))
        return encode_causal_document_block_sparse(bounds, kept, 128, N, B)
    if mask_name == "prefix_lm":
        return encode_prefix_lm(N // 2, N, B)
    if mask_name == "share_question":
        Q = N // 4
        cuts = uniform_cuts(rng, 3, Q + 1, N - 1)
        return encode_share_question(Q, np.concatenate([[Q], cuts, [N]]), N, B)
    if mask_name == "causal_key_drop":
        n_drop = int(round(0.3 * N))
        drops = [np.sort(rng.choice(N, size=n_drop, replace=False)) for _ in range(H)]
        return encode_causal_key_drop(drops, N, B)
    if mask_name == "bidirectional_document":
        K = int(rng.integers(2, 6))
        bounds = doc_boundaries_from_cuts(uniform_cuts(rng, min(K - 1, N - 1), 1, N - 1), N)
        return encode_bidirectional_document(bounds, N, B)
    raise ValueError(f"unknown mask family {mask_name!r}")


def make_tensors(cfg: int, mask_index: int, B: int, H: int, N: int, d: int):
    """Q, K, V, dO as float32 N(0, 1) arrays [B, H, N, d], one seeded stream per tensor."""
    out = []
    for purpose in (PURPOSE_Q, PURPOSE_K, PURPOSE_V, PURPOSE_DO):
        rng = rng_for(cfg, mask_index, purpose)
        out.append(rng.standard_normal((B, H, N, d), dtype=np.float32))
    return tuple(out)


# ---------------------------------------------------------------- hash-bucket attention inputs
# The hash needs a random matrix per head; it is drawn here and passed in, like Q, K, V and dO. The
# hash-bucket workloads use the SFT shape (8192 tokens) with 8 and 16 buckets, the setting of the SCFA
# review's hash-attention timings, and the long-context shape with 16 buckets.

HASH_WORKLOADS = {
    # name: (config index, buckets)
    "sft_packing_hash_8": (2, 8),
    "sft_packing_hash_16": (2, 16),
    "long_context_hash_16": (4, 16),
}
HASH_MASK_INDEX = 100  # seed stream of the hash workloads, apart from the mask families'


def make_rotation(cfg: int, mask_index: int, H: int, d: int, nb: int) -> np.ndarray:
    """float32 N(0, 1) [H, d, nb / 2]: one random rotation per head for the bucket hash."""
    return rng_for(cfg, mask_index, PURPOSE_ROT).standard_normal((H, d, nb // 2), dtype=np.float32)


def make_buckets(cfg: int, mask_index: int, B: int, H: int, N: int, nb: int, drop: float = 0.0):
    """int32 [B, H, N] query and key bucket ids, uniform in [0, nb), with a fraction `drop` of each set
    to -1 (dropped token): inputs for the reordering and the attention independent of any hash."""
    rng = rng_for(cfg, mask_index, PURPOSE_BUCKET)
    out = []
    for _ in range(2):
        bk = rng.integers(0, nb, size=(B, H, N)).astype(np.int32)
        if drop > 0:
            bk[rng.random((B, H, N)) < drop] = -1
        out.append(bk)
    return tuple(out)
