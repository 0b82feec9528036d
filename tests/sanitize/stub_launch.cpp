// Host-only stand-ins for the kernel launchers of libfm, for building the C-ABI argument checks
// (fm_api.hip) without a GPU under AddressSanitizer and UndefinedBehaviorSanitizer. Each stand-in counts
// its calls and checks what a launch relies on (the arguments fm_api.hip promises to have validated);
// nothing is launched and no pointer is dereferenced except the host-side plan view.
#include <cstdio>
#include <cstdlib>

#include "fm_launch.h"

long g_launches = 0;
int g_stub_failures = 0;

namespace {
void need(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "stub: launch reached with %s\n", what);
    ++g_stub_failures;
  }
}
hipError_t launched() {
  ++g_launches;
  return hipSuccess;
}
}  // namespace

namespace fm {

int fwd_qblock() { return 128; }
int lsh_max_nb() { return LSH_NB_LIMIT; }
int sort_max_nb() { return SORT_NB_LIMIT; }

hipError_t launch_tile_bounds(const int* lts, const int* lte, const int* uts, const int* ute, int rows, int N,
                              int* bounds, hipStream_t) {
  need(bounds != nullptr && rows > 0 && N > 0, "tile bounds: bad output or sizes");
  need((lts == nullptr) == (lte == nullptr) && (uts == nullptr) == (ute == nullptr), "tile bounds: half pair");
  return launched();
}

hipError_t launch_tile_classes(const int*, int rows, int N, int, int qblock, uint8_t* classes, hipStream_t) {
  need(classes != nullptr && rows > 0 && N > 0 && qblock > 0, "tile classes: bad arguments");
  return launched();
}

hipError_t launch_fwd(bool, int d, const void* q, const void* k, const void* v, void* out, float* lse,
                      const int* lts, const int* lte, const int* uts, const int* ute, const int* bounds, int B, int H,
                      int Nq, int Nk, int q_off, int Hm, const int*, int, float scale, hipStream_t, const int*) {
  need(q && k && v && out && lse, "fwd: null tensor");
  need(d == 64 || d == 128, "fwd: head dim");
  need(B > 0 && H > 0 && Nq > 0 && Nk > 0 && q_off >= 0 && (Hm == 1 || Hm == H), "fwd: sizes");
  need(((lts == nullptr && uts == nullptr) || bounds != nullptr) && (lts == nullptr) == (lte == nullptr) &&
           (uts == nullptr) == (ute == nullptr), "fwd: mask arguments");
  need(scale > 0.f, "fwd: scale");
  return launched();
}

hipError_t launch_bwd(bool, int d, const void* q, const void* k, const void* v, const void* out, const void* dout,
                      const float* lse, void* dq, void* dk, void* dv, float* dd, const int* lts, const int* lte,
                      const int* uts, const int* ute, const int* bounds, int B, int H, int Nq, int Nk, int q_off,
                      int Hm, const int*, int, float scale, hipStream_t, const int*, const int*, void* ds_cache,
                      long long ds_cap, const DsPlan* ds_plan) {
  need(q && k && v && out && dout && lse && dq && dk && dv && dd, "bwd: null tensor or workspace");
  need(d == 64 || d == 128, "bwd: head dim");
  need(B > 0 && H > 0 && Nq > 0 && Nk > 0 && q_off >= 0 && (Hm == 1 || Hm == H), "bwd: sizes");
  need(((lts == nullptr && uts == nullptr) || bounds != nullptr) && (lts == nullptr) == (lte == nullptr) &&
           (uts == nullptr) == (ute == nullptr), "bwd: mask arguments");
  need(scale > 0.f, "bwd: scale");
  need((ds_cache == nullptr) == (ds_plan == nullptr) && ds_cap >= 0, "bwd: stored-dS arguments");
  if (ds_plan != nullptr) need(ds_plan->nkt == (Nk + DS_KEYS - 1) / DS_KEYS, "bwd: plan view");
  return launched();
}

hipError_t launch_ds_plan(const int*, int B, int H, int Hm, int N, int, void* plan, hipStream_t) {
  need(plan != nullptr && B > 0 && H > 0 && N > 0 && (Hm == 1 || Hm == H), "plan: bad arguments");
  return launched();
}

hipError_t launch_tile_schedule(const int*, int rows, int Nq, int Nk, int q_off, int, int* sched, hipStream_t) {
  need(sched != nullptr && rows > 0 && Nq > 0 && Nk > 0 && q_off >= 0, "schedule: bad arguments");
  return launched();
}

hipError_t launch_compact_keys(const int*, const int*, const int*, const int*, int rows, int N, int, int* kidx,
                               int* kpos, int* counts, int* lts2, int* lte2, int* uts2, int* ute2, hipStream_t) {
  need(rows > 0 && N > 0 && kidx && kpos && counts && lts2 && lte2 && uts2 && ute2, "compact: bad arguments");
  return launched();
}

hipError_t launch_gather_rows(const void* x, const int* idx, int B, int H, int Hm, int N, int row_bytes, void* y,
                              hipStream_t) {
  need(x && idx && y && x != y && B > 0 && H > 0 && N > 0 && (Hm == 1 || Hm == H) && row_bytes > 0,
       "gather: bad arguments");
  return launched();
}

hipError_t launch_lsh_buckets(bool, int d, const void* x, const float* rot, int B, int H, int N, int Hr, int nb,
                              int* out, hipStream_t) {
  need(x && rot && out && (d == 64 || d == 128) && B > 0 && H > 0 && N > 0 && (Hr == 1 || Hr == H) && nb >= 2 &&
           nb <= LSH_NB_LIMIT && nb % 2 == 0,
       "lsh: bad arguments");
  return launched();
}

hipError_t launch_bucket_sort(const int* qb, const int* kb, int rows, int N, int nb, int* qidx, int* qpos,
                              int* kidx, int* kpos, int* lts, int* lte, int* uts, int* ute, hipStream_t) {
  need(qb && kb && qidx && qpos && kidx && kpos && lts && lte && uts && ute && rows > 0 && N > 0 && nb >= 1 &&
           nb <= SORT_NB_LIMIT,
       "bucket sort: bad arguments");
  return launched();
}

}  // namespace fm
