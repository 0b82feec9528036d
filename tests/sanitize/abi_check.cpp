// Walks the whole C ABI of libfm against the host-only stand-in launchers (stub_launch.cpp): every entry
// point with valid arguments (one launch, FM_OK) and with each kind of bad argument (the documented error,
// no launch), including sizes at and past FM_MAX_N and workspace sizes that overflow. Built with
// AddressSanitizer and UndefinedBehaviorSanitizer, it checks the argument validation for memory errors
// and undefined behaviour. Exit status 0 when every expectation holds.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <limits>

#include "fm.h"

extern long g_launches;
extern int g_stub_failures;

static int g_fail = 0;

#define EXPECT(call, st, nl)                                                                              \
  do {                                                                                                    \
    const long before_ = g_launches;                                                                      \
    const fm_status got_ = (call);                                                                        \
    if (got_ != (st) || g_launches - before_ != (nl)) {                                                   \
      std::fprintf(stderr, "line %d: %s -> %d (want %d), launches %ld (want %d)\n", __LINE__, #call,      \
                   (int)got_, (int)(st), g_launches - before_, (int)(nl));                                \
      ++g_fail;                                                                                           \
    }                                                                                                     \
  } while (0)

#define CHECK(cond)                                              \
  do {                                                           \
    if (!(cond)) {                                               \
      std::fprintf(stderr, "line %d: %s\n", __LINE__, #cond);    \
      ++g_fail;                                                  \
    }                                                            \
  } while (0)

alignas(256) static char g_buf[1 << 16];  // stand-in for device memory: never dereferenced
static void* P = g_buf;
static void* Q = g_buf + 4096;
static int32_t* I = reinterpret_cast<int32_t*>(g_buf + 8192);
static float* F = reinterpret_cast<float*>(g_buf + 12288);
static uint8_t* U8 = reinterpret_cast<uint8_t*>(g_buf + 16384);

static const int kMaxN = FM_MAX_N;
static const float kInf = std::numeric_limits<float>::infinity();
static const float kNaN = std::numeric_limits<float>::quiet_NaN();

static void sizes() {
  CHECK(fm_kblock() == 64);
  CHECK(fm_fwd_qblock(64) == 128 && fm_fwd_qblock(128) == 128 && fm_fwd_qblock(96) == 0);
  CHECK(fm_bounds_elems(1, 1, 1) == 8 && fm_bounds_elems(0, 1, 1) == 0 && fm_bounds_elems(1, 1, kMaxN + 1) == 0);
  CHECK(fm_bounds_elems(1, 1, kMaxN) == (size_t)kMaxN / 64 * 8);
  CHECK(fm_schedule_elems(1, 1, 0, 1) == 0 && fm_schedule_elems(1, 1, 256, 256) == 8);
  CHECK(fm_bwd_workspace_bytes(FM_BF16, 1, 2, 100, 64) == 1024 && fm_bwd_workspace_bytes(FM_BF16, 1, 2, 100, 96) == 0);
  CHECK(fm_bwd_workspace_bytes((fm_dtype)7, 1, 1, 1, 64) == 0);
  CHECK(fm_bwd_plan_bytes(1, 2, 3, 100) == 0 && fm_bwd_plan_bytes(1, 2, 2, 100) > 0);
  CHECK(fm_bwd_plan_bytes(1 << 20, 1, 1, kMaxN) == 0);  // B * H * row tiles past the limits
  CHECK(fm_bwd_ds_workspace_bytes(FM_BF16, 1, 1, 64, 64, 2) == 256 + 2 * 16384);
  CHECK(fm_bwd_ds_workspace_bytes(FM_BF16, 1, 1, 64, 64, -1) == 0);
  CHECK(fm_bwd_ds_workspace_bytes(FM_BF16, 1, 1, 64, 64, std::numeric_limits<int64_t>::max()) == 0);
  for (int s = -1; s < 7; ++s) CHECK(fm_status_str((fm_status)s) != nullptr);
}

static void bounds_and_schedule() {
  EXPECT(fm_tile_bounds(I, I, I, I, 1, 1, 100, I, 0), FM_OK, 1);
  EXPECT(fm_tile_bounds(nullptr, nullptr, nullptr, nullptr, 2, 3, kMaxN, I, 0), FM_OK, 1);
  EXPECT(fm_tile_bounds(I, nullptr, I, I, 1, 1, 100, I, 0), FM_ERR_INVALID, 0);
  EXPECT(fm_tile_bounds(I, I, I, I, 1, 1, 100, nullptr, 0), FM_ERR_INVALID, 0);
  EXPECT(fm_tile_bounds(I, I, I, I, 0, 1, 100, I, 0), FM_ERR_INVALID, 0);
  EXPECT(fm_tile_bounds(I, I, I, I, 1, 1, kMaxN + 1, I, 0), FM_ERR_INVALID, 0);
  EXPECT(fm_tile_bounds(I, I, I, I, 1 << 20, 1 << 11, 100, I, 0), FM_ERR_INVALID, 0);
  EXPECT(fm_tile_schedule(I, 1, 1, 300, 500, 200, 1, I, 0), FM_OK, 1);
  EXPECT(fm_tile_schedule(I, 1, 1, 300, 500, -1, 1, I, 0), FM_ERR_INVALID, 0);
  EXPECT(fm_tile_schedule(I, 1, 1, 300, 500, kMaxN - 299, 1, I, 0), FM_ERR_INVALID, 0);
  EXPECT(fm_tile_schedule(I, 1, 1, 300, 500, 0, 1, nullptr, 0), FM_ERR_INVALID, 0);
  EXPECT(fm_tile_classes(I, 1, 1, 100, 1, 128, U8, 0), FM_OK, 1);
  EXPECT(fm_tile_classes(I, 1, 1, 100, 1, 0, U8, 0), FM_ERR_INVALID, 0);
  EXPECT(fm_tile_classes(I, 1, 1, 100, 1, 64, nullptr, 0), FM_ERR_INVALID, 0);
}

static fm_status fwd(const void* q, fm_dtype dt, int B, int H, int N, int d, const int32_t* lts, const int32_t* lte,
                     const int32_t* uts, const int32_t* ute, int Hm, const int32_t* bounds, float scale, void* out,
                     float* lse) {
  return fm_fwd(q, P, P, dt, B, H, N, d, lts, lte, uts, ute, Hm, bounds, nullptr, 1, scale, out, lse, 0);
}

static void forward() {
  EXPECT(fwd(P, FM_BF16, 1, 2, 100, 64, nullptr, nullptr, nullptr, nullptr, 1, nullptr, 0.125f, Q, F), FM_OK, 1);
  EXPECT(fwd(P, FM_F32, 2, 3, 100, 128, I, I, I, I, 3, I, 0.125f, Q, F), FM_OK, 1);
  EXPECT(fwd(nullptr, FM_BF16, 1, 2, 100, 64, nullptr, nullptr, nullptr, nullptr, 1, nullptr, 0.125f, Q, F),
         FM_ERR_INVALID, 0);
  EXPECT(fwd(P, FM_BF16, 1, 2, 100, 64, nullptr, nullptr, nullptr, nullptr, 1, nullptr, 0.125f, nullptr, F),
         FM_ERR_INVALID, 0);
  EXPECT(fwd(P, FM_BF16, 1, 2, 100, 64, nullptr, nullptr, nullptr, nullptr, 1, nullptr, 0.125f, Q, nullptr),
         FM_ERR_INVALID, 0);
  for (float bad : {0.f, -1.f, kInf, kNaN})
    EXPECT(fwd(P, FM_BF16, 1, 2, 100, 64, nullptr, nullptr, nullptr, nullptr, 1, nullptr, bad, Q, F),
           FM_ERR_INVALID, 0);
  EXPECT(fwd(P, FM_BF16, 1, 2, 100, 96, nullptr, nullptr, nullptr, nullptr, 1, nullptr, 0.125f, Q, F),
         FM_ERR_UNSUPPORTED, 0);
  EXPECT(fwd(P, (fm_dtype)5, 1, 2, 100, 64, nullptr, nullptr, nullptr, nullptr, 1, nullptr, 0.125f, Q, F),
         FM_ERR_UNSUPPORTED, 0);
  EXPECT(fwd(P, FM_BF16, 1, 2, 100, 64, I, nullptr, nullptr, nullptr, 1, I, 0.125f, Q, F), FM_ERR_INVALID, 0);
  EXPECT(fwd(P, FM_BF16, 1, 2, 100, 64, I, I, nullptr, nullptr, 1, nullptr, 0.125f, Q, F), FM_ERR_INVALID, 0);
  EXPECT(fwd(P, FM_BF16, 1, 4, 100, 64, I, I, nullptr, nullptr, 2, I, 0.125f, Q, F), FM_ERR_INVALID, 0);
  EXPECT(fwd(static_cast<char*>(P) + 8, FM_BF16, 1, 2, 100, 64, nullptr, nullptr, nullptr, nullptr, 1, nullptr,
             0.125f, Q, F),
         FM_ERR_INVALID, 0);
  EXPECT(fwd(P, FM_BF16, 0, 2, 100, 64, nullptr, nullptr, nullptr, nullptr, 1, nullptr, 0.125f, Q, F),
         FM_ERR_INVALID, 0);
  EXPECT(fwd(P, FM_BF16, 1, 2, kMaxN + 1, 64, nullptr, nullptr, nullptr, nullptr, 1, nullptr, 0.125f, Q, F),
         FM_ERR_INVALID, 0);
  EXPECT(fwd(P, FM_BF16, std::numeric_limits<int>::max(), std::numeric_limits<int>::max(), 100, 64, nullptr,
             nullptr, nullptr, nullptr, 1, nullptr, 0.125f, Q, F),
         FM_ERR_INVALID, 0);
  // row blocks and mapped outputs
  EXPECT(fm_fwd_rows(P, P, P, FM_BF16, 1, 2, 100, 300, 200, 64, nullptr, nullptr, nullptr, nullptr, 1, nullptr,
                     nullptr, 1, 0.125f, Q, F, 0),
         FM_OK, 1);
  EXPECT(fm_fwd_rows(P, P, P, FM_BF16, 1, 2, 100, 300, -1, 64, nullptr, nullptr, nullptr, nullptr, 1, nullptr,
                     nullptr, 1, 0.125f, Q, F, 0),
         FM_ERR_INVALID, 0);
  EXPECT(fm_fwd_rows(P, P, P, FM_BF16, 1, 2, 100, 300, kMaxN - 50, 64, nullptr, nullptr, nullptr, nullptr, 1,
                     nullptr, nullptr, 1, 0.125f, Q, F, 0),
         FM_ERR_INVALID, 0);
  EXPECT(fm_fwd_mapped(P, P, P, FM_BF16, 1, 2, 100, 64, nullptr, nullptr, nullptr, nullptr, 1, nullptr, nullptr, 0,
                       0.125f, I, Q, F, 0),
         FM_OK, 1);
  EXPECT(fm_fwd_mapped(P, P, P, FM_BF16, 1, 2, 100, 64, nullptr, nullptr, nullptr, nullptr, 1, nullptr, nullptr, 0,
                       0.125f, nullptr, Q, F, 0),
         FM_ERR_INVALID, 0);
}

static void backward() {
  const size_t ws = fm_bwd_workspace_bytes(FM_BF16, 1, 2, 100, 64);
  auto bwd = [&](void* w, size_t wb, int d, float scale) {
    return fm_bwd(P, P, P, P, P, F, FM_BF16, 1, 2, 100, d, nullptr, nullptr, nullptr, nullptr, 1, nullptr, nullptr, 1,
                  scale, Q, Q, Q, w, wb, 0);
  };
  EXPECT(bwd(Q, ws, 64, 0.125f), FM_OK, 1);
  EXPECT(bwd(Q, ws - 1, 64, 0.125f), FM_ERR_WORKSPACE, 0);
  EXPECT(bwd(nullptr, ws, 64, 0.125f), FM_ERR_WORKSPACE, 0);
  EXPECT(bwd(static_cast<char*>(Q) + 4, ws, 64, 0.125f), FM_ERR_WORKSPACE, 0);
  EXPECT(bwd(Q, ws, 80, 0.125f), FM_ERR_UNSUPPORTED, 0);
  EXPECT(bwd(Q, ws, 64, kNaN), FM_ERR_INVALID, 0);
  EXPECT(fm_bwd(P, P, P, P, nullptr, F, FM_BF16, 1, 2, 100, 64, nullptr, nullptr, nullptr, nullptr, 1, nullptr, nullptr,
                1, 0.125f, Q, Q, Q, Q, ws, 0),
         FM_ERR_INVALID, 0);
  EXPECT(fm_bwd_rows(P, P, P, P, P, F, FM_F32, 1, 2, 100, 300, 100, 128, I, I, nullptr, nullptr, 1, I, nullptr, 1,
                     0.125f, Q, Q, Q, Q, ws, 0),
         FM_OK, 1);
  EXPECT(fm_bwd_mapped(P, P, P, P, P, F, FM_BF16, 1, 2, 100, 64, nullptr, nullptr, nullptr, nullptr, 1, nullptr,
                       nullptr, 0, 0.125f, I, nullptr, Q, Q, Q, Q, ws, 0),
         FM_ERR_INVALID, 0);
  EXPECT(fm_bwd_mapped(P, P, P, P, P, F, FM_BF16, 1, 2, 100, 64, nullptr, nullptr, nullptr, nullptr, 1, nullptr,
                       nullptr, 0, 0.125f, I, I, Q, Q, Q, Q, ws, 0),
         FM_OK, 1);
  // stored-dS plan and backward
  alignas(256) static char plan[1 << 12];
  EXPECT(fm_bwd_plan(I, 1, 2, 2, 100, 1, plan, 0), FM_OK, 1);
  EXPECT(fm_bwd_plan(nullptr, 1, 2, 1, 100, 0, plan, 0), FM_OK, 1);
  EXPECT(fm_bwd_plan(I, 1, 2, 3, 100, 1, plan, 0), FM_ERR_INVALID, 0);
  EXPECT(fm_bwd_plan(I, 1, 2, 2, 100, 1, nullptr, 0), FM_ERR_INVALID, 0);
  EXPECT(fm_bwd_plan(I, 1, 2, 2, 100, 1, plan + 4, 0), FM_ERR_INVALID, 0);
  EXPECT(fm_bwd_plan(I, 1, 2, 2, 0, 1, plan, 0), FM_ERR_INVALID, 0);
  const size_t wsd = fm_bwd_ds_workspace_bytes(FM_BF16, 1, 2, 100, 64, 3);
  auto bwd_ds = [&](const void* pl, void* w, size_t wb, fm_dtype dt) {
    return fm_bwd_ds(P, P, P, P, P, F, dt, 1, 2, 100, 64, nullptr, nullptr, nullptr, nullptr, 1, nullptr, nullptr, pl,
                     1, 0.125f, Q, Q, Q, w, wb, 0);
  };
  EXPECT(bwd_ds(plan, Q, wsd, FM_BF16), FM_OK, 1);
  EXPECT(bwd_ds(plan, Q, ws, FM_BF16), FM_OK, 1);         // no room for a tile: every head recomputes
  EXPECT(bwd_ds(plan, Q, wsd, FM_F32), FM_OK, 1);         // float32 keeps the recomputing pass
  EXPECT(bwd_ds(nullptr, Q, wsd, FM_BF16), FM_ERR_INVALID, 0);
  EXPECT(bwd_ds(plan + 8, Q, wsd, FM_BF16), FM_OK, 1);    // 8-byte alignment is enough
  EXPECT(bwd_ds(plan + 2, Q, wsd, FM_BF16), FM_ERR_INVALID, 0);
  EXPECT(bwd_ds(plan, Q, ws - 1, FM_BF16), FM_ERR_WORKSPACE, 0);
}

static void compaction_and_hashing() {
  EXPECT(fm_compact_keys(I, I, nullptr, nullptr, 1, 1, 100, 1, I, I, I, I, I, I, I, 0), FM_OK, 1);
  EXPECT(fm_compact_keys(I, I, nullptr, nullptr, 1, 1, 100, 1, I, nullptr, I, I, I, I, I, 0), FM_ERR_INVALID, 0);
  EXPECT(fm_compact_keys(I, nullptr, nullptr, nullptr, 1, 1, 100, 1, I, I, I, I, I, I, I, 0), FM_ERR_INVALID, 0);
  EXPECT(fm_gather_rows(P, FM_BF16, 1, 2, 100, 64, I, 2, Q, 0), FM_OK, 1);
  EXPECT(fm_gather_rows(P, FM_BF16, 1, 2, 100, 64, I, 3, Q, 0), FM_ERR_INVALID, 0);
  EXPECT(fm_gather_rows(P, FM_BF16, 1, 2, 100, 64, I, 1, P, 0), FM_ERR_INVALID, 0);
  EXPECT(fm_gather_rows(P, FM_BF16, 1, 2, 100, 48, I, 1, Q, 0), FM_ERR_UNSUPPORTED, 0);
  EXPECT(fm_lsh_buckets(P, FM_BF16, 1, 2, 100, 128, F, 2, 16, I, 0), FM_OK, 1);
  for (int nb : {0, 1, 3, 66, 1 << 30})
    EXPECT(fm_lsh_buckets(P, FM_BF16, 1, 2, 100, 128, F, 2, nb, I, 0), FM_ERR_INVALID, 0);
  EXPECT(fm_lsh_buckets(P, FM_BF16, 1, 2, 100, 128, F, 3, 16, I, 0), FM_ERR_INVALID, 0);
  EXPECT(fm_bucket_sort(I, I, 1, 2, 100, 512, I, I, I, I, I, I, I, I, 0), FM_OK, 1);
  EXPECT(fm_bucket_sort(I, I, 1, 2, 100, 513, I, I, I, I, I, I, I, I, 0), FM_ERR_INVALID, 0);
  EXPECT(fm_bucket_sort(I, I, 1, 2, 100, 0, I, I, I, I, I, I, I, I, 0), FM_ERR_INVALID, 0);
  EXPECT(fm_bucket_sort(I, I, 1, 2, 100, 8, I, I, I, I, I, nullptr, I, I, 0), FM_ERR_INVALID, 0);
}

int main() {
  std::memset(g_buf, 0, sizeof(g_buf));
  sizes();
  bounds_and_schedule();
  forward();
  backward();
  compaction_and_hashing();
  if (g_fail || g_stub_failures) {
    std::fprintf(stderr, "abi_check: %d expectation(s) failed, %d stub check(s) failed\n", g_fail, g_stub_failures);
    return 1;
  }
  std::printf("abi_check: all expectations hold (%ld launches)\n", g_launches);
  return 0;
}
