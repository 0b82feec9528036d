"""CPU oracle for column-wise-mask (FlashMask) attention, forward and backward.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package. It shares no code with the HIP path (``mask_aware_exact_amd``) and never imports
it; the product path never imports this package.

What it computes is the plain definition that the method reaches exactly, since its tile skipping
costs no accuracy (FlashMask abstract, papers.pytorch.kr 2410.01359): the four per-column
query-axis boundary vectors are expanded into a dense boolean mask, and softmax attention with its
gradients is evaluated in float64 with library matrix products and elementwise NumPy operations.

Modules:
  masks     dense mask expansion, hand-written dense twins of each mask family, unmasked-pair count
  tiles     per-key-tile min/max of the four vectors and the FULL/PARTIAL/NONE tile rule
  attention fp64 forward/backward (row-blocked), brute force for tiny cases, one-row/one-column probes
  compact   removal of the key columns masked for every row, and the compacted problem's mask
  schedule  longest-first order of the work units by their count of tiles that are not fully masked
  hashing   LSH buckets, reordering by bucket with the reordered problem's mask, hash-bucket attention
"""
from . import masks, tiles, attention, compact, schedule, hashing  # noqa: F401
