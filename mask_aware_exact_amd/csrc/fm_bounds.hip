// Per-key-tile bounds pre-pass and the test-only tile classifier (gfx950).
//
// The bounds pass streams the int32 [B, Hm, N] vectors once and writes 32 bytes per key tile of
// KBLOCK = 64 columns, so it is HBM-bound. A wave takes 256 consecutive columns of one (b, hm) row, four
// key tiles: lane l reads columns 4 l .. 4 l + 3 of each present vector (one 16-byte load per vector when
// the rows are 16-byte aligned), reduces them in registers, and the 16 lanes of a tile finish the eight
// min/max values with four DPP lane moves. Each wave keeps TPW chunks of loads in flight. The tile
// classification is read from these bounds (FlashMask abstract, papers.pytorch.kr 2410.01359: skip
// computation where the mask is known).
#include <climits>

#include "fm_common.h"

namespace fm {

template <int CTRL>
__device__ __forceinline__ int dpp_int(int x) {
  return __builtin_amdgcn_mov_dpp(x, CTRL, 0xF, 0xF, false);
}
// min / max over the 16 lanes of a DPP row: quad swaps, then the half-row and row mirrors
__device__ __forceinline__ int row16_min(int v) {
  v = min(v, dpp_int<0xB1>(v));   // quad_perm [1, 0, 3, 2]
  v = min(v, dpp_int<0x4E>(v));   // quad_perm [2, 3, 0, 1]
  v = min(v, dpp_int<0x141>(v));  // row_half_mirror
  return min(v, dpp_int<0x140>(v));  // row_mirror
}
__device__ __forceinline__ int row16_max(int v) {
  v = max(v, dpp_int<0xB1>(v));
  v = max(v, dpp_int<0x4E>(v));
  v = max(v, dpp_int<0x141>(v));
  return max(v, dpp_int<0x140>(v));
}

constexpr int BOUNDS_CHUNK = 256;  // columns per wave and chunk: four key tiles

// Column values 4 l .. 4 l + 3 of one vector row; columns at or past n take `fill`.
template <bool VEC>
__device__ __forceinline__ i32x4 load_cols4(const int* __restrict__ row, int j0, int n, int fill) {
  i32x4 v = {fill, fill, fill, fill};
  if constexpr (VEC) {
    // n is a multiple of 4 here, so the four columns are all valid or all past n
    if (j0 < n) v = *reinterpret_cast<const i32x4*>(row + j0);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (j0 + e < n) v[e] = row[j0 + e];
  }
  return v;
}

// TPW chunks per wave, their loads issued together (more bytes in flight per wave for large inputs).
template <bool VEC, int TPW>
__global__ __launch_bounds__(256) void tile_bounds_kernel(const int* __restrict__ lts, const int* __restrict__ lte,
                                                          const int* __restrict__ uts, const int* __restrict__ ute,
                                                          int N, int nkt, int nchunks,
                                                          int* __restrict__ bounds) {
  const int lane = threadIdx.x & 63;
  const int cpr = (N + BOUNDS_CHUNK - 1) / BOUNDS_CHUNK;  // chunks per row
  const int first = (int)(blockIdx.x * 4 + (threadIdx.x >> 6)) * TPW;
  i32x4 ls[TPW][4];  // per chunk: LTS, LTE, UTS, UTE values of this lane's four columns
#pragma unroll
  for (int k = 0; k < TPW; ++k) {
    const int ch = first + k;
    const int chc = ch < nchunks ? ch : 0;  // past the end: any valid chunk, not written
    const int row = chc / cpr;
    const int j0 = (chc - row * cpr) * BOUNDS_CHUNK + 4 * lane;
    const size_t rb = (size_t)row * N;
    if (lts != nullptr) {
      ls[k][0] = load_cols4<VEC>(lts + rb, j0, N, INT_MAX);
      ls[k][1] = load_cols4<VEC>(lte + rb, j0, N, INT_MAX);
    }
    if (uts != nullptr) {
      ls[k][2] = load_cols4<VEC>(uts + rb, j0, N, INT_MAX);
      ls[k][3] = load_cols4<VEC>(ute + rb, j0, N, INT_MAX);
    }
  }
#pragma unroll
  for (int k = 0; k < TPW; ++k) {
    const int ch = first + k;
    if (ch >= nchunks) break;  // whole waves take the same branch
    const int row = ch / cpr;
    const int cw = ch - row * cpr;  // chunk within the row
    const int t = cw * (BOUNDS_CHUNK / KBLOCK) + lane / 16;  // this lane's key tile
    const int j0 = cw * BOUNDS_CHUNK + 4 * lane;
    int out[8];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const bool present = v < 2 ? lts != nullptr : uts != nullptr;
      if (present) {
        // columns past N hold INT_MAX: neutral for min; for max use INT_MIN instead
        const i32x4 x = ls[k][v];
        int mn = min(min(x[0], x[1]), min(x[2], x[3]));
        int mx = INT_MIN;
#pragma unroll
        for (int e = 0; e < 4; ++e) mx = max(mx, j0 + e < N ? x[e] : INT_MIN);
        out[2 * v] = row16_min(mn);
        out[2 * v + 1] = row16_max(mx);
      } else {
        out[2 * v] = out[2 * v + 1] = v < 2 ? N : 0;  // canonical empty interval of a missing pair
      }
    }
    if ((lane & 15) == 0 && t < nkt) {
      i32x4* dst = reinterpret_cast<i32x4*>(bounds + ((size_t)row * nkt + t) * 8);
      dst[0] = i32x4{out[0], out[1], out[2], out[3]};
      dst[1] = i32x4{out[4], out[5], out[6], out[7]};
    }
  }
}

__global__ __launch_bounds__(256) void tile_classes_kernel(const int* __restrict__ bounds, int rows, int N,
                                                           int causal, int qblock, int nq, int nkt,
                                                           uint8_t* __restrict__ classes) {
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long)rows * nq * nkt) return;
  const int kt = (int)(idx % nkt);
  const int qt = (int)((idx / nkt) % nq);
  const int row = (int)(idx / ((long)nkt * nq));
  const TileBounds b = merged_bounds(bounds == nullptr ? nullptr : bounds + (size_t)row * nkt * 8, kt, kt + 1, N);
  const int r0 = qt * qblock, r1 = min(N, r0 + qblock);
  const int c0 = kt * KBLOCK, c1 = min(N, c0 + KBLOCK);
  classes[idx] = (uint8_t)classify_tile(r0, r1, c0, c1, b, causal != 0);
}

hipError_t launch_tile_bounds(const int* lts, const int* lte, const int* uts, const int* ute, int rows, int N,
                              int* bounds, hipStream_t stream) {
  const int nkt = (N + KBLOCK - 1) / KBLOCK;
  const long nchunks_l = (long)rows * ((N + BOUNDS_CHUNK - 1) / BOUNDS_CHUNK);
  if (nchunks_l > INT_MAX / 2) return hipErrorInvalidValue;  // 2^38 columns: beyond any device memory
  const int nchunks = (int)nchunks_l;
  // 16-byte loads need every row start 16-byte aligned: aligned bases and N a multiple of 4
  const uintptr_t bases = reinterpret_cast<uintptr_t>(lts) | reinterpret_cast<uintptr_t>(lte) |
                          reinterpret_cast<uintptr_t>(uts) | reinterpret_cast<uintptr_t>(ute);
  const bool vec = (bases & 15u) == 0 && N % 4 == 0;
  // small inputs: one chunk per wave for more waves; large ones: two, for more loads in flight
  const bool two = nchunks >= 8192;
  const int waves = two ? (nchunks + 1) / 2 : nchunks;
  const unsigned grid = (unsigned)((waves + 3) / 4);
  auto kern = vec ? (two ? tile_bounds_kernel<true, 2> : tile_bounds_kernel<true, 1>)
                  : (two ? tile_bounds_kernel<false, 2> : tile_bounds_kernel<false, 1>);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), 0, stream, lts, lte, uts, ute, N, nkt, nchunks, bounds);
  return hipGetLastError();
}

hipError_t launch_tile_classes(const int* bounds, int rows, int N, int causal, int qblock, uint8_t* classes,
                               hipStream_t stream) {
  const int nkt = (N + KBLOCK - 1) / KBLOCK;
  const int nq = (N + qblock - 1) / qblock;
  const long total = (long)rows * nq * nkt;
  const unsigned grid = (unsigned)((total + 255) / 256);
  hipLaunchKernelGGL(tile_classes_kernel, dim3(grid), dim3(256), 0, stream, bounds, rows, N, causal, qblock, nq,
                     nkt, classes);
  return hipGetLastError();
}

}  // namespace fm
