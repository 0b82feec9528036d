// Host-side interface between the C ABI (fm_api.hip) and the kernel files: the launch functions each
// kernel file defines, the limits the argument checks use, and the layout of the stored-dS plan. Plain
// C++ over the HIP runtime's types, so that the argument checks can also be built for the host alone.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace fm {

constexpr int LSH_NB_LIMIT = 64;    // largest bucket count of the hash (rotation staged in LDS)
constexpr int SORT_NB_LIMIT = 512;  // largest bucket count of the sort (per-wave group counts in LDS)

// View of a stored-dS plan (written by the plan pass of the stored-dS backward): per (b, hm, 128-key
// tile) the first live 64-row query tile and the tile's first slot inside its head's region, per (b, hm)
// the slots of one head, and per (b, h) the region's first slot. Slots are counted in 16 KB tiles.
constexpr int DS_QROWS = 64;                         // query rows of a stored dS tile
constexpr int DS_KEYS = 128;                         // keys of a stored dS tile
constexpr int DS_TILE_BYTES = DS_QROWS * DS_KEYS * 2;  // bf16

struct DsPlan {
  long long* total;     // [1]: slots of the whole problem
  long long* region;    // [B * H]
  long long* base;      // [B * Hm * nkt]
  long long* rowtotal;  // [B * Hm]
  int* first;           // [B * Hm * nkt]
  int nkt;              // 128-key tiles per row
};

// Plan layout in bytes: total (int64) at 0, region [B * H] int64 at 16, then base [B * Hm * nkt] and
// rowtotal [B * Hm] int64, then first [B * Hm * nkt] int32; nkt = ceil(N / DS_KEYS).
inline size_t ds_plan_bytes(int B, int H, int Hm, int N) {
  const size_t nkt = (size_t)(N + DS_KEYS - 1) / DS_KEYS;
  const size_t rows = (size_t)B * Hm;
  const size_t bytes = 16 + 8 * ((size_t)B * H + rows * nkt + rows) + 4 * rows * nkt;
  return (bytes + 255) / 256 * 256;
}

inline DsPlan ds_plan_view(const void* plan, int B, int H, int Hm, int N) {
  const size_t nkt = (size_t)(N + DS_KEYS - 1) / DS_KEYS;
  const size_t rows = (size_t)B * Hm;
  char* p = static_cast<char*>(const_cast<void*>(plan));
  DsPlan v;
  v.total = reinterpret_cast<long long*>(p);
  v.region = reinterpret_cast<long long*>(p + 16);
  v.base = v.region + (size_t)B * H;
  v.rowtotal = v.base + rows * nkt;
  v.first = reinterpret_cast<int*>(v.rowtotal + rows);
  v.nkt = (int)nkt;
  return v;
}

hipError_t launch_tile_bounds(const int* lts, const int* lte, const int* uts, const int* ute, int rows, int N,
                              int* bounds, hipStream_t stream);
hipError_t launch_tile_classes(const int* bounds, int rows, int N, int causal, int qblock, uint8_t* classes,
                               hipStream_t stream);
hipError_t launch_fwd(bool bf16_in, int d, const void* q, const void* k, const void* v, void* out, float* lse,
                      const int* lts, const int* lte, const int* uts, const int* ute, const int* bounds, int B, int H,
                      int Nq, int Nk, int q_off, int Hm, const int* sched, int causal, float scale,
                      hipStream_t stream, const int* omap);
hipError_t launch_bwd(bool bf16_in, int d, const void* q, const void* k, const void* v, const void* out,
                      const void* dout, const float* lse, void* dq, void* dk, void* dv, float* dd, const int* lts,
                      const int* lte, const int* uts, const int* ute, const int* bounds, int B, int H, int Nq,
                      int Nk, int q_off, int Hm, const int* sched, int causal, float scale,
                      hipStream_t stream, const int* qmap, const int* kmap, void* ds_cache, long long ds_cap,
                      const DsPlan* ds_plan);
hipError_t launch_ds_plan(const int* bounds, int B, int H, int Hm, int N, int causal, void* plan,
                          hipStream_t stream);
int fwd_qblock();
hipError_t launch_tile_schedule(const int* bounds, int rows, int Nq, int Nk, int q_off, int causal, int* sched,
                                hipStream_t stream);
hipError_t launch_compact_keys(const int* lts, const int* lte, const int* uts, const int* ute, int rows, int N,
                               int causal, int* kidx, int* kpos, int* counts, int* lts2, int* lte2, int* uts2,
                               int* ute2, hipStream_t stream);
hipError_t launch_gather_rows(const void* x, const int* idx, int B, int H, int Hm, int N, int row_bytes, void* y,
                              hipStream_t stream);
int lsh_max_nb();
int sort_max_nb();
hipError_t launch_lsh_buckets(bool bf16_in, int d, const void* x, const float* rot, int B, int H, int N, int Hr,
                              int nb, int* out, hipStream_t stream);
hipError_t launch_bucket_sort(const int* qb, const int* kb, int rows, int N, int nb, int* qidx, int* qpos,
                              int* kidx, int* kpos, int* lts, int* lte, int* uts, int* ute, hipStream_t stream);

}  // namespace fm
