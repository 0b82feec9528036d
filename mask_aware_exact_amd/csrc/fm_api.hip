// C ABI of the column-wise-mask attention library: argument validation and kernel launches.
// Every argument check runs on the host before any HIP call, so a rejected call touches no device
// state and launches nothing. See include/fm.h for the contract of each entry point.
#include <cmath>
#include <cstdint>

#include "fm.h"
#include "fm_common.h"
#include "fm_launch.h"


namespace {

constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool sizes_ok(int B, int H, int N) {
  if (B <= 0 || H <= 0 || N <= 0 || N > FM_MAX_N) return false;
  // flattened grids and row counts stay far inside 32-bit launch limits
  return (long long)B * H <= (1LL << 20) && (long long)B * H * ((N + 63) / 64) < (1LL << 31);
}

bool pair_ok(const int32_t* s, const int32_t* e) { return (s == nullptr) == (e == nullptr); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

fm_status dtype_d_ok(fm_dtype dtype, int d) {
  if (dtype != FM_BF16 && dtype != FM_F32) return FM_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return FM_ERR_UNSUPPORTED;
  return FM_OK;
}

fm_status mask_args_ok(const int32_t* lts, const int32_t* lte, const int32_t* uts, const int32_t* ute, int Hm,
                       int H, const int32_t* bounds) {
  if (!pair_ok(lts, lte) || !pair_ok(uts, ute)) return FM_ERR_INVALID;
  if (Hm != 1 && Hm != H) return FM_ERR_INVALID;
  const bool any_vec = lts != nullptr || uts != nullptr;
  if (any_vec && bounds == nullptr) return FM_ERR_INVALID;
  return FM_OK;
}

fm_status from_hip(hipError_t e) { return e == hipSuccess ? FM_OK : FM_ERR_LAUNCH; }

// A row block [q_off, q_off + Nq) of a problem with Nk keys: both sizes in range and global row indices
// inside int32 arithmetic.
bool rows_ok(int B, int H, int Nq, int Nk, int q_off) {
  return sizes_ok(B, H, Nq) && sizes_ok(B, H, Nk) && q_off >= 0 && (long long)q_off + Nq <= FM_MAX_N;
}

}  // namespace

extern "C" {

int fm_kblock(void) { return fm::KBLOCK; }

int fm_fwd_qblock(int d) { return (d == 64 || d == 128) ? fm::fwd_qblock() : 0; }

size_t fm_bounds_elems(int B, int Hm, int N) {
  if (B <= 0 || Hm <= 0 || N <= 0 || N > FM_MAX_N) return 0;
  return (size_t)B * Hm * ((N + fm::KBLOCK - 1) / fm::KBLOCK) * 8;
}

fm_status fm_tile_bounds(const int32_t* lts, const int32_t* lte, const int32_t* uts, const int32_t* ute, int B,
                         int Hm, int N, int32_t* bounds, hipStream_t stream) {
  if (bounds == nullptr || !sizes_ok(B, Hm, N)) return FM_ERR_INVALID;
  if (!pair_ok(lts, lte) || !pair_ok(uts, ute)) return FM_ERR_INVALID;
  return from_hip(fm::launch_tile_bounds(lts, lte, uts, ute, B * Hm, N, bounds, stream));
}

size_t fm_schedule_elems(int B, int Hm, int Nq, int Nk) {
  if (!rows_ok(B, Hm, Nq, Nk, 0)) return 0;
  const size_t units = (size_t)(Nq + fm::SCHED_UNIT - 1) / fm::SCHED_UNIT + (Nk + fm::SCHED_UNIT - 1) / fm::SCHED_UNIT;
  return (size_t)B * Hm * 2 * units;
}

fm_status fm_tile_schedule(const int32_t* bounds, int B, int Hm, int Nq, int Nk, int q_off, int causal,
                           int32_t* sched, hipStream_t stream) {
  if (sched == nullptr || !rows_ok(B, Hm, Nq, Nk, q_off)) return FM_ERR_INVALID;
  return from_hip(fm::launch_tile_schedule(bounds, B * Hm, Nq, Nk, q_off, causal != 0, sched, stream));
}

namespace {
fm_status fwd_impl(const void* q, const void* k, const void* v, fm_dtype dtype, int B, int H, int Nq, int Nk,
                   int q_off, int d, const int32_t* lts, const int32_t* lte, const int32_t* uts, const int32_t* ute,
                   int Hm, const int32_t* bounds, const int32_t* sched, int causal, float scale, const int32_t* omap,
                   void* out, float* lse, hipStream_t stream) {
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr || lse == nullptr) return FM_ERR_INVALID;
  if (!rows_ok(B, H, Nq, Nk, q_off) || !std::isfinite(scale) || !(scale > 0.f)) return FM_ERR_INVALID;
  fm_status st = mask_args_ok(lts, lte, uts, ute, Hm, H, bounds);
  if (st != FM_OK) return st;
  st = dtype_d_ok(dtype, d);
  if (st != FM_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return FM_ERR_INVALID;
  return from_hip(fm::launch_fwd(dtype == FM_BF16, d, q, k, v, out, lse, lts, lte, uts, ute, bounds, B, H, Nq, Nk,
                                 q_off, Hm, sched, causal != 0, scale, stream, omap));
}
}  // namespace

fm_status fm_fwd_rows(const void* q, const void* k, const void* v, fm_dtype dtype, int B, int H, int Nq, int Nk,
                      int q_off, int d, const int32_t* lts, const int32_t* lte, const int32_t* uts,
                      const int32_t* ute, int Hm, const int32_t* bounds, const int32_t* sched, int causal,
                      float scale, void* out, float* lse, hipStream_t stream) {
  return fwd_impl(q, k, v, dtype, B, H, Nq, Nk, q_off, d, lts, lte, uts, ute, Hm, bounds, sched, causal, scale,
                  nullptr, out, lse, stream);
}

fm_status fm_fwd_mapped(const void* q, const void* k, const void* v, fm_dtype dtype, int B, int H, int N, int d,
                        const int32_t* lts, const int32_t* lte, const int32_t* uts, const int32_t* ute, int Hm,
                        const int32_t* bounds, const int32_t* sched, int causal, float scale, const int32_t* omap,
                        void* out, float* lse, hipStream_t stream) {
  if (omap == nullptr) return FM_ERR_INVALID;
  return fwd_impl(q, k, v, dtype, B, H, N, N, 0, d, lts, lte, uts, ute, Hm, bounds, sched, causal, scale, omap, out,
                  lse, stream);
}

fm_status fm_fwd(const void* q, const void* k, const void* v, fm_dtype dtype, int B, int H, int N, int d,
                 const int32_t* lts, const int32_t* lte, const int32_t* uts, const int32_t* ute, int Hm,
                 const int32_t* bounds, const int32_t* sched, int causal, float scale, void* out, float* lse,
                 hipStream_t stream) {
  return fm_fwd_rows(q, k, v, dtype, B, H, N, N, 0, d, lts, lte, uts, ute, Hm, bounds, sched, causal, scale, out,
                     lse, stream);
}

size_t fm_bwd_workspace_bytes(fm_dtype dtype, int B, int H, int N, int d) {
  if (dtype_d_ok(dtype, d) != FM_OK || !sizes_ok(B, H, N)) return 0;
  const size_t rows = (size_t)B * H * N;
  return round_up(rows * sizeof(float));
}

namespace {
fm_status bwd_impl(const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
                   fm_dtype dtype, int B, int H, int Nq, int Nk, int q_off, int d, const int32_t* lts,
                   const int32_t* lte, const int32_t* uts, const int32_t* ute, int Hm, const int32_t* bounds,
                   const int32_t* sched, int causal, float scale, const int32_t* qmap, const int32_t* kmap,
                   void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, hipStream_t stream,
                   const void* plan = nullptr) {
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr || dout == nullptr || lse == nullptr ||
      dq == nullptr || dk == nullptr || dv == nullptr)
    return FM_ERR_INVALID;
  if (!rows_ok(B, H, Nq, Nk, q_off) || !std::isfinite(scale) || !(scale > 0.f)) return FM_ERR_INVALID;
  fm_status st = mask_args_ok(lts, lte, uts, ute, Hm, H, bounds);
  if (st != FM_OK) return st;
  st = dtype_d_ok(dtype, d);
  if (st != FM_OK) return st;
  const void* ptrs[] = {q, k, v, out, dout, dq, dk, dv};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FM_ERR_INVALID;
  const size_t need = fm_bwd_workspace_bytes(dtype, B, H, Nq, d);
  if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)) return FM_ERR_WORKSPACE;
  float* dd = static_cast<float*>(workspace);
  // Stored-dS mode: the workspace past D (a multiple of 256 bytes) holds whole dS tiles.
  void* cache = nullptr;
  long long cap = 0;
  fm::DsPlan view{};
  if (plan != nullptr) {
    cache = static_cast<char*>(workspace) + need;
    cap = (long long)((workspace_bytes - need) / (size_t)fm::DS_TILE_BYTES);
    view = fm::ds_plan_view(plan, B, H, Hm, Nk);
  }
  return from_hip(fm::launch_bwd(dtype == FM_BF16, d, q, k, v, out, dout, lse, dq, dk, dv, dd, lts, lte, uts, ute,
                                 bounds, B, H, Nq, Nk, q_off, Hm, sched, causal != 0, scale, stream, qmap, kmap,
                                 cache, cap, plan != nullptr ? &view : nullptr));
}
}  // namespace

fm_status fm_bwd_rows(const void* q, const void* k, const void* v, const void* out, const void* dout,
                      const float* lse, fm_dtype dtype, int B, int H, int Nq, int Nk, int q_off, int d,
                      const int32_t* lts, const int32_t* lte, const int32_t* uts, const int32_t* ute, int Hm,
                      const int32_t* bounds, const int32_t* sched, int causal, float scale, void* dq, void* dk,
                      void* dv, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return bwd_impl(q, k, v, out, dout, lse, dtype, B, H, Nq, Nk, q_off, d, lts, lte, uts, ute, Hm, bounds, sched,
                  causal, scale, nullptr, nullptr, dq, dk, dv, workspace, workspace_bytes, stream);
}

fm_status fm_bwd_mapped(const void* q, const void* k, const void* v, const void* out, const void* dout,
                        const float* lse, fm_dtype dtype, int B, int H, int N, int d, const int32_t* lts,
                        const int32_t* lte, const int32_t* uts, const int32_t* ute, int Hm, const int32_t* bounds,
                        const int32_t* sched, int causal, float scale, const int32_t* qmap, const int32_t* kmap,
                        void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (qmap == nullptr || kmap == nullptr) return FM_ERR_INVALID;
  return bwd_impl(q, k, v, out, dout, lse, dtype, B, H, N, N, 0, d, lts, lte, uts, ute, Hm, bounds, sched, causal,
                  scale, qmap, kmap, dq, dk, dv, workspace, workspace_bytes, stream);
}

fm_status fm_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
                 fm_dtype dtype, int B, int H, int N, int d, const int32_t* lts, const int32_t* lte,
                 const int32_t* uts, const int32_t* ute, int Hm, const int32_t* bounds, const int32_t* sched,
                 int causal, float scale, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                 hipStream_t stream) {
  return fm_bwd_rows(q, k, v, out, dout, lse, dtype, B, H, N, N, 0, d, lts, lte, uts, ute, Hm, bounds, sched,
                     causal, scale, dq, dk, dv, workspace, workspace_bytes, stream);
}

size_t fm_bwd_plan_bytes(int B, int H, int Hm, int N) {
  if (!sizes_ok(B, H, N) || (Hm != 1 && Hm != H)) return 0;
  return fm::ds_plan_bytes(B, H, Hm, N);
}

fm_status fm_bwd_plan(const int32_t* bounds, int B, int H, int Hm, int N, int causal, void* plan,
                      hipStream_t stream) {
  if (plan == nullptr || (reinterpret_cast<uintptr_t>(plan) & 7u) != 0) return FM_ERR_INVALID;
  if (!sizes_ok(B, H, N) || (Hm != 1 && Hm != H)) return FM_ERR_INVALID;
  return from_hip(fm::launch_ds_plan(bounds, B, H, Hm, N, causal != 0, plan, stream));
}

size_t fm_bwd_ds_workspace_bytes(fm_dtype dtype, int B, int H, int N, int d, int64_t tiles) {
  const size_t base = fm_bwd_workspace_bytes(dtype, B, H, N, d);
  const size_t tb = (size_t)fm::DS_TILE_BYTES;
  if (base == 0 || tiles < 0 || (uint64_t)tiles > (SIZE_MAX - base) / tb) return 0;
  return base + (size_t)tiles * tb;
}

fm_status fm_bwd_ds(const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
                    fm_dtype dtype, int B, int H, int N, int d, const int32_t* lts, const int32_t* lte,
                    const int32_t* uts, const int32_t* ute, int Hm, const int32_t* bounds, const int32_t* sched,
                    const void* plan, int causal, float scale, void* dq, void* dk, void* dv, void* workspace,
                    size_t workspace_bytes, hipStream_t stream) {
  if (plan == nullptr || (reinterpret_cast<uintptr_t>(plan) & 7u) != 0) return FM_ERR_INVALID;
  return bwd_impl(q, k, v, out, dout, lse, dtype, B, H, N, N, 0, d, lts, lte, uts, ute, Hm, bounds, sched, causal,
                  scale, nullptr, nullptr, dq, dk, dv, workspace, workspace_bytes, stream, plan);
}

fm_status fm_compact_keys(const int32_t* lts, const int32_t* lte, const int32_t* uts, const int32_t* ute, int B,
                          int Hm, int N, int causal, int32_t* kidx, int32_t* kpos, int32_t* counts, int32_t* lts2,
                          int32_t* lte2, int32_t* uts2, int32_t* ute2, hipStream_t stream) {
  if (kidx == nullptr || kpos == nullptr || counts == nullptr || lts2 == nullptr || lte2 == nullptr ||
      uts2 == nullptr || ute2 == nullptr)
    return FM_ERR_INVALID;
  if (!sizes_ok(B, Hm, N) || !pair_ok(lts, lte) || !pair_ok(uts, ute)) return FM_ERR_INVALID;
  return from_hip(fm::launch_compact_keys(lts, lte, uts, ute, B * Hm, N, causal != 0, kidx, kpos, counts, lts2,
                                          lte2, uts2, ute2, stream));
}

fm_status fm_gather_rows(const void* x, fm_dtype dtype, int B, int H, int N, int d, const int32_t* idx, int Hm,
                         void* y, hipStream_t stream) {
  if (x == nullptr || idx == nullptr || y == nullptr || x == y) return FM_ERR_INVALID;
  const fm_status st = dtype_d_ok(dtype, d);
  if (st != FM_OK) return st;
  if (!sizes_ok(B, H, N) || (Hm != 1 && Hm != H)) return FM_ERR_INVALID;
  if (!aligned16(x) || !aligned16(y)) return FM_ERR_INVALID;
  const int row_bytes = d * (dtype == FM_BF16 ? 2 : 4);
  return from_hip(fm::launch_gather_rows(x, idx, B, H, Hm, N, row_bytes, y, stream));
}

fm_status fm_lsh_buckets(const void* x, fm_dtype dtype, int B, int H, int N, int d, const float* rot, int Hr,
                         int nb, int32_t* buckets, hipStream_t stream) {
  if (x == nullptr || rot == nullptr || buckets == nullptr) return FM_ERR_INVALID;
  const fm_status st = dtype_d_ok(dtype, d);
  if (st != FM_OK) return st;
  if (!sizes_ok(B, H, N) || (Hr != 1 && Hr != H)) return FM_ERR_INVALID;
  if (nb < 2 || nb > fm::lsh_max_nb() || (nb & 1) != 0 || !aligned16(x)) return FM_ERR_INVALID;
  return from_hip(fm::launch_lsh_buckets(dtype == FM_BF16, d, x, rot, B, H, N, Hr, nb, buckets, stream));
}

fm_status fm_bucket_sort(const int32_t* qbucket, const int32_t* kbucket, int B, int H, int N, int nb, int32_t* qidx,
                         int32_t* qpos, int32_t* kidx, int32_t* kpos, int32_t* lts, int32_t* lte, int32_t* uts,
                         int32_t* ute, hipStream_t stream) {
  if (qbucket == nullptr || kbucket == nullptr || qidx == nullptr || qpos == nullptr || kidx == nullptr ||
      kpos == nullptr || lts == nullptr || lte == nullptr || uts == nullptr || ute == nullptr)
    return FM_ERR_INVALID;
  if (!sizes_ok(B, H, N) || nb < 1 || nb > fm::sort_max_nb()) return FM_ERR_INVALID;
  return from_hip(fm::launch_bucket_sort(qbucket, kbucket, B * H, N, nb, qidx, qpos, kidx, kpos, lts, lte, uts, ute,
                                         stream));
}

fm_status fm_tile_classes(const int32_t* bounds, int B, int Hm, int N, int causal, int qblock, uint8_t* classes,
                          hipStream_t stream) {
  if (classes == nullptr || qblock <= 0 || !sizes_ok(B, Hm, N)) return FM_ERR_INVALID;
  return from_hip(fm::launch_tile_classes(bounds, B * Hm, N, causal != 0, qblock, classes, stream));
}

const char* fm_status_str(fm_status s) {
  switch (s) {
    case FM_OK: return "ok";
    case FM_ERR_INVALID: return "invalid argument";
    case FM_ERR_UNSUPPORTED: return "unsupported head dim or dtype";
    case FM_ERR_WORKSPACE: return "workspace missing or too small";
    case FM_ERR_LAUNCH: return "kernel launch failed";
    default: break;  // the enum's range sentinels and any other value
  }
  return "unknown status";
}

}  // extern "C"
