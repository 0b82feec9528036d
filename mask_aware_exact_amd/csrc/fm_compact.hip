// Key compaction for masks that drop whole key columns, and the row gather that moves tensors between
// the full and the compacted key order (gfx950).
//
// Per-head key dropping reduces attention compute in proportion to the keys kept (SCFA review,
// nubint.ai, "proposed method"). Under the column-wise mask a dropped key is a column that is masked
// for every query row. Such columns contribute nothing to out, lse or dq, and their dk, dv are zero, so
// they can be removed before the attention kernels run:
//   1. fm_compact_keys lists, per (b, hm) row of the mask, the kept columns in increasing order and
//      writes the mask of the compacted problem. A kept column keeps its intervals; its causal
//      condition (rows i < j, j its original index) becomes the interval [0, j), folded into the upper
//      or the lower interval, so the compacted problem runs with causal = 0. Positions past the kept
//      count are padding, masked for every row, so their tiles are skipped as fully masked.
//   2. fm_gather_rows copies K and V rows into the compacted order, runs of the same call scatter dK and
//      dV back (dropped rows zero).
// The attention kernels themselves are unchanged.
#include "fm_common.h"

namespace fm {

namespace {

struct Span {
  int s, e;  // [s, e) clipped to [0, N]; empty when s >= e
};

__device__ __forceinline__ Span clip_span(int s, int e, int N) { return Span{min(max(s, 0), N), min(max(e, 0), N)}; }
__device__ __forceinline__ bool span_empty(Span a) { return a.s >= a.e; }

// Whether the union of up to three clipped spans covers [0, N).
__device__ __forceinline__ bool covers_all(Span a, Span b, Span c, int N) {
  // order by start (three elements), then sweep
  if (b.s < a.s) { const Span t = a; a = b; b = t; }
  if (c.s < b.s) { const Span t = b; b = c; c = t; }
  if (b.s < a.s) { const Span t = a; a = b; b = t; }
  int reach = 0;
  const Span v[3] = {a, b, c};
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    if (span_empty(v[k])) continue;
    if (v[k].s > reach) return false;
    reach = max(reach, v[k].e);
  }
  return reach >= N;
}

constexpr int CT = 1024;  // threads of the compaction kernel (16 waves)

}  // namespace

// One workgroup per (b, hm) mask row. Columns are taken CT at a time; the kept ones get consecutive
// positions (wave ballots, then a prefix over the 16 wave totals). counts[row] is the number kept, or -1
// if a kept column needs three disjoint intervals (causal plus both spans), which the compacted mask
// cannot hold.
__global__ __launch_bounds__(CT) void compact_keys_kernel(const int* __restrict__ lts, const int* __restrict__ lte,
                                                          const int* __restrict__ uts, const int* __restrict__ ute,
                                                          int N, int causal, int* __restrict__ kidx,
                                                          int* __restrict__ kpos, int* __restrict__ counts,
                                                          int* __restrict__ lts2, int* __restrict__ lte2,
                                                          int* __restrict__ uts2, int* __restrict__ ute2) {
  __shared__ int wave_tot[CT / 64];
  __shared__ int bad_any;
  const int row = blockIdx.x;
  const size_t base = (size_t)row * N;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) bad_any = 0;
  int kept_before = 0;  // kept columns in earlier chunks
  for (int c0 = 0; c0 < N; c0 += CT) {
    const int j = c0 + tid;
    bool keep = false;
    Span lt{N, N}, ut{0, 0};
    if (j < N) {
      if (lts != nullptr) lt = clip_span(lts[base + j], lte[base + j], N);
      if (uts != nullptr) ut = clip_span(uts[base + j], ute[base + j], N);
      const Span cz = causal ? Span{0, j} : Span{0, 0};
      keep = !covers_all(cz, lt, ut, N);
    }
    const uint64_t bal = __ballot(keep);
    const int in_wave = __builtin_popcountll(bal & ((1ull << lane) - 1ull));
    __syncthreads();  // every wave is past the previous chunk's reads of wave_tot
    if (lane == 0) wave_tot[wave] = __builtin_popcountll(bal);
    __syncthreads();
    int before = kept_before;
    int total = kept_before;
#pragma unroll
    for (int w = 0; w < CT / 64; ++w) {
      before += w < wave ? wave_tot[w] : 0;
      total += wave_tot[w];
    }
    if (j < N) {
      if (keep) {
        const int r = before + in_wave;
        kidx[base + r] = j;
        kpos[base + j] = r;
        // fold the causal rows [0, j) into one of the two spans
        Span nl = lt, nu = ut;
        bool ok = true;
        if (causal && j > 0) {
          if (span_empty(ut)) {
            nu = Span{0, j};
          } else if (ut.s <= j) {
            nu = Span{0, max(j, ut.e)};
          } else if (span_empty(lt)) {
            nl = Span{0, j};
          } else if (lt.s <= j) {
            nl = Span{0, max(j, lt.e)};
          } else {
            ok = false;
          }
        }
        if (!ok) atomicOr(&bad_any, 1);
        lts2[base + r] = span_empty(nl) ? N : nl.s;
        lte2[base + r] = span_empty(nl) ? N : nl.e;
        uts2[base + r] = span_empty(nu) ? 0 : nu.s;
        ute2[base + r] = span_empty(nu) ? 0 : nu.e;
      } else {
        kpos[base + j] = -1;
      }
    }
    kept_before = total;
  }
  // padding positions: no source column, masked for every row
  for (int r = kept_before + tid; r < N; r += CT) {
    kidx[base + r] = -1;
    lts2[base + r] = 0;
    lte2[base + r] = N;
    uts2[base + r] = 0;
    ute2[base + r] = 0;
  }
  __syncthreads();
  if (tid == 0) counts[row] = bad_any ? -1 : kept_before;
}

// y[b, h, r, :] = x[b, h, idx[b, hm, r], :], or zero where idx is outside [0, N). A task is RPB rows of one
// (b, h); thread t moves 16-byte chunk t % CPR of rows t / CPR + k * (256 / CPR), k < GK, loading the GK
// indices, then the GK chunks, then storing them, so each thread has GK independent copies in flight.
// CPR (chunks per row) is 8, 16 or 32, so the row and chunk of a thread are shifts, not divisions.
constexpr int GK = 4;

template <int CPR>
__global__ __launch_bounds__(256) void gather_rows_kernel(const char* __restrict__ x, const int* __restrict__ idx,
                                                          int H, int Hm, int N, int nrb, long ntask,
                                                          char* __restrict__ y) {
  constexpr int RPS = 256 / CPR;  // rows per step of the workgroup
  constexpr int RPB = RPS * GK;   // rows per task
  const int piece = threadIdx.x % CPR, rl = threadIdx.x / CPR;
  for (long t = blockIdx.x; t < ntask; t += gridDim.x) {
    const long bh = t / nrb;
    const int r0 = (int)(t - bh * nrb) * RPB + rl;
    const int b = (int)(bh / H), h = (int)(bh % H);
    const int* ih = idx + ((size_t)b * Hm + (Hm > 1 ? h : 0)) * N;
    const char* xh = x + (size_t)bh * N * (CPR * 16);
    char* yh = y + (size_t)bh * N * (CPR * 16);
    int src[GK];
#pragma unroll
    for (int k = 0; k < GK; ++k) {
      const int r = r0 + k * RPS;
      src[k] = r < N ? ih[r] : -1;
    }
    i32x4 v[GK];
#pragma unroll
    for (int k = 0; k < GK; ++k) {
      v[k] = i32x4{0, 0, 0, 0};
      if (src[k] >= 0 && src[k] < N) v[k] = *reinterpret_cast<const i32x4*>(xh + ((size_t)src[k] * CPR + piece) * 16);
    }
#pragma unroll
    for (int k = 0; k < GK; ++k) {
      const int r = r0 + k * RPS;
      if (r < N) *reinterpret_cast<i32x4*>(yh + ((size_t)r * CPR + piece) * 16) = v[k];
    }
  }
}

hipError_t launch_compact_keys(const int* lts, const int* lte, const int* uts, const int* ute, int rows, int N,
                               int causal, int* kidx, int* kpos, int* counts, int* lts2, int* lte2, int* uts2,
                               int* ute2, hipStream_t stream) {
  hipLaunchKernelGGL(compact_keys_kernel, dim3((unsigned)rows), dim3(CT), 0, stream, lts, lte, uts, ute, N, causal,
                     kidx, kpos, counts, lts2, lte2, uts2, ute2);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* x, const int* idx, int B, int H, int Hm, int N, int row_bytes, void* y,
                              hipStream_t stream) {
  const int cpr = row_bytes / 16;
  const int rpb = 256 / cpr * GK;
  const int nrb = (N + rpb - 1) / rpb;
  const long ntask = (long)B * H * nrb;
  const unsigned blocks = (unsigned)min(ntask, 1L << 20);
  const char* xs = static_cast<const char*>(x);
  char* ys = static_cast<char*>(y);
  if (cpr == 8)
    hipLaunchKernelGGL(gather_rows_kernel<8>, dim3(blocks), dim3(256), 0, stream, xs, idx, H, Hm, N, nrb, ntask, ys);
  else if (cpr == 16)
    hipLaunchKernelGGL(gather_rows_kernel<16>, dim3(blocks), dim3(256), 0, stream, xs, idx, H, Hm, N, nrb, ntask, ys);
  else if (cpr == 32)
    hipLaunchKernelGGL(gather_rows_kernel<32>, dim3(blocks), dim3(256), 0, stream, xs, idx, H, Hm, N, nrb, ntask, ys);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace fm
