// Longest-first dispatch order of the attention work units (gfx950).
//
// Under a sparse mask the units of one launch carry very different amounts of work, and a fixed
// dispatch order can leave a few long units running alone at the end of the launch (the
// load-balancing problem of masked attention that the FlashMask-3 summary, readmex.ai, addresses across
// workers with a sparsity-aware balancer). On one GPU the hardware dispatcher hands workgroups to free
// slots in launch order, so it already is a list scheduler: giving it the units in decreasing order of
// work is the longest-processing-time-first rule, with no persistent grid and no work queue.
//
// Units and their work (tiles not classified fully masked, rows in the mask's global coordinates):
//   query unit qt: rows [128 qt, 128 qt + 128) against the 64-column key tiles (forward, dq);
//   key unit kt:   columns [128 kt, 128 kt + 128) against 64-row query tiles (dk, dv).
// Schedule layout per (b, hm) row of the mask, stride 2 (nq + nk) int32:
//   [0, nq)                query units, longest first (ties: latest unit first)
//   [nq, nq + nk)          key units, longest first (ties: earliest unit first)
//   [nq + nk, 2 nq + nk)   work of each query unit
//   [2 nq + nk, 2 (nq+nk)) work of each key unit
// The ties keep the order the kernels use without a schedule, so a schedule never reorders units of
// equal work.
#include "fm_common.h"

namespace fm {

namespace {

constexpr int UNIT = SCHED_UNIT;  // rows of a query unit, columns of a key unit
constexpr int SUB = 64;    // rows of the query tiles a key unit is classified against

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

}  // namespace

// One wave per unit: lanes stride over the tiles of the unit's row or column of the tile grid.
__global__ __launch_bounds__(256) void unit_work_kernel(const int* __restrict__ bounds, int Nq, int Nk, int q_off,
                                                        int causal, int nq, int nk, int* __restrict__ sched) {
  const int bpr = (nq + nk + 3) / 4;  // blocks per mask row
  const int row = (int)(blockIdx.x / bpr);
  const int u = (int)(blockIdx.x % bpr) * 4 + (threadIdx.x >> 6);
  if (u >= nq + nk) return;  // whole waves exit together
  const int lane = threadIdx.x & 63;
  const int nkb = (Nk + KBLOCK - 1) / KBLOCK;
  const int* brow = bounds == nullptr ? nullptr : bounds + (size_t)row * nkb * 8;
  const bool cz = causal != 0;
  int live = 0;
  if (u < nq) {
    const int g0 = q_off + u * UNIT, g1 = q_off + min(Nq, u * UNIT + UNIT);
    for (int t = lane; t < nkb; t += 64) {
      const TileBounds b = merged_bounds(brow, t, t + 1, Nk);
      live += classify_tile(g0, g1, t * KBLOCK, min(Nk, t * KBLOCK + KBLOCK), b, cz) != CLS_FULL;
    }
  } else {
    const int kt = u - nq;
    const int c0 = kt * UNIT, c1 = min(Nk, c0 + UNIT);
    const TileBounds b = merged_bounds(brow, kt * (UNIT / KBLOCK), min(nkb, (kt + 1) * (UNIT / KBLOCK)), Nk);
    const int nsub = (Nq + SUB - 1) / SUB;
    for (int t = lane; t < nsub; t += 64)
      live += classify_tile(q_off + t * SUB, q_off + min(Nq, t * SUB + SUB), c0, c1, b, cz) != CLS_FULL;
  }
  live = wave_sum(live);
  if (lane == 0) sched[(size_t)row * 2 * (nq + nk) + nq + nk + u] = live;
}

// Rank of each unit among the units of its kind: those with more work, and those with equal work that
// come earlier in the default order, go first. The ranks are a permutation, so every slot of the order
// is written exactly once. Per mask row, blocks [0, ceil(nq / 256)) take query units, the rest key units.
__global__ __launch_bounds__(256) void unit_order_kernel(int nq, int nk, int* __restrict__ sched) {
  __shared__ int work_lds[256];
  const int nqb = (nq + 255) / 256;
  const int bpr = nqb + (nk + 255) / 256;  // blocks per mask row
  const int row = (int)(blockIdx.x / bpr);
  const int blk = (int)(blockIdx.x % bpr);
  const bool key = blk >= nqb;
  const int n = key ? nk : nq;
  const int u = (blk - (key ? nqb : 0)) * 256 + (int)threadIdx.x;
  int* srow = sched + (size_t)row * 2 * (nq + nk);
  const int* work = srow + nq + nk + (key ? nq : 0);
  // default position: key units earliest first, query units latest first
  auto dpos = [&](int x) { return key ? x : n - 1 - x; };
  const int mine = u < n ? work[u] : 0;
  const int mypos = dpos(u);
  int rank = 0;
  for (int v0 = 0; v0 < n; v0 += 256) {
    __syncthreads();
    if (v0 + (int)threadIdx.x < n) work_lds[threadIdx.x] = work[v0 + threadIdx.x];
    __syncthreads();
    const int cnt = min(256, n - v0);
    for (int i = 0; i < cnt; ++i) {
      const int w = work_lds[i];
      rank += (w > mine) || (w == mine && dpos(v0 + i) < mypos);
    }
  }
  if (u < n) srow[(key ? nq : 0) + rank] = u;
}

hipError_t launch_tile_schedule(const int* bounds, int rows, int Nq, int Nk, int q_off, int causal, int* sched,
                                hipStream_t stream) {
  const int nq = (Nq + UNIT - 1) / UNIT, nk = (Nk + UNIT - 1) / UNIT;
  const long work_blocks = (long)rows * ((nq + nk + 3) / 4);
  const long order_blocks = (long)rows * ((nq + 255) / 256 + (nk + 255) / 256);
  hipLaunchKernelGGL(unit_work_kernel, dim3((unsigned)work_blocks), dim3(256), 0, stream, bounds, Nq, Nk, q_off,
                     causal, nq, nk, sched);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(unit_order_kernel, dim3((unsigned)order_blocks), dim3(256), 0, stream, nq, nk, sched);
  return hipGetLastError();
}

}  // namespace fm
