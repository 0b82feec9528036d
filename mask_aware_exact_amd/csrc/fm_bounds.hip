// Per-key-tile bounds pre-pass and the test-only tile classifier (gfx950).
//
// The bounds pass streams the four int32 [B, Hm, N] vectors once and writes 32 bytes per key tile of
// KBLOCK = 64 columns, so it is HBM-bound. One wave owns one key tile: lane c reads column
// t * 64 + c of each vector (four coalesced 256-byte reads), and butterfly shuffles reduce the
// eight min/max values across the wave. The tile classification is read from these bounds
// (FlashMask abstract, papers.pytorch.kr 2410.01359: skip computation where the mask is known).
#include <climits>

#include "fm_common.h"

namespace fm {

__device__ __forceinline__ int wave_min(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = min(v, __shfl_xor(v, m, 64));
  return v;
}
__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = max(v, __shfl_xor(v, m, 64));
  return v;
}

__global__ __launch_bounds__(256) void tile_bounds_kernel(const int* __restrict__ lts, const int* __restrict__ lte,
                                                          const int* __restrict__ uts, const int* __restrict__ ute,
                                                          int rows, int N, int nkt, int* __restrict__ bounds) {
  const long tile = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tile >= (long)rows * nkt) return;  // whole waves exit together
  const int lane = threadIdx.x & 63;
  const int row = (int)(tile / nkt);
  const int t = (int)(tile % nkt);
  const int j = t * KBLOCK + lane;
  const bool valid = j < N;
  const size_t off = (size_t)row * N + (valid ? j : 0);
  int out[8];
  if (lts != nullptr) {
    const int s = lts[off], e = lte[off];
    out[0] = wave_min(valid ? s : INT_MAX);
    out[1] = wave_max(valid ? s : INT_MIN);
    out[2] = wave_min(valid ? e : INT_MAX);
    out[3] = wave_max(valid ? e : INT_MIN);
  } else {
    out[0] = out[1] = out[2] = out[3] = N;
  }
  if (uts != nullptr) {
    const int s = uts[off], e = ute[off];
    out[4] = wave_min(valid ? s : INT_MAX);
    out[5] = wave_max(valid ? s : INT_MIN);
    out[6] = wave_min(valid ? e : INT_MAX);
    out[7] = wave_max(valid ? e : INT_MIN);
  } else {
    out[4] = out[5] = out[6] = out[7] = 0;
  }
  if (lane == 0) {
    i32x4* dst = reinterpret_cast<i32x4*>(bounds + (size_t)tile * 8);
    dst[0] = i32x4{out[0], out[1], out[2], out[3]};
    dst[1] = i32x4{out[4], out[5], out[6], out[7]};
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
  const long tiles = (long)rows * nkt;
  const unsigned grid = (unsigned)((tiles + 3) / 4);
  hipLaunchKernelGGL(tile_bounds_kernel, dim3(grid), dim3(256), 0, stream, lts, lte, uts, ute, rows, N, nkt,
                     bounds);
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
