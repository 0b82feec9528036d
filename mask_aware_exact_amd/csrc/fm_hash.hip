// Hash-bucket sparse causal attention on the column-wise mask path (gfx950).
//
// The SCFA review (nubint.ai, "proposed method" and Figure 3) computes attention restricted to hash
// buckets exactly, after reordering queries and keys by bucket; the reordering turns causal attention
// inside buckets into a non-triangular causal mask. Under the column-wise encoding that mask needs no new
// kernel: once queries and keys are sorted stably by bucket, the queries of bucket b sit in rows
// [qs_b, qe_b) in increasing position, and the rows attending the key at sorted column c (original
// position p, bucket b) are one contiguous range [lo_c, qe_b), lo_c = qs_b + (bucket-b queries before
// p). So the key's column is masked on UT = [0, lo_c) and LT = [qe_b, N), and the attention kernels run
// unchanged (causal flag off).
//   fm_lsh_buckets  bucket of each row: argmax of [x R, -x R] for a random R [d, nb/2] (Reformer-style
//                   geometric hashing), float32 dot products.
//   fm_bucket_sort  stable counting sort of queries and keys by bucket (out-of-range buckets form a
//                   trailing dropped group that attends and is attended by nothing), the permutations
//                   both ways, and the sorted problem's four vectors, in one sweep per head.
#include "fm_common.h"

namespace fm {

namespace {

constexpr int LSH_T = 256;     // rows per workgroup, one per thread
constexpr int LSH_CB = 8;      // rotation columns per pass
constexpr int SORT_T = 1024;   // threads of the sort kernel (16 waves)
constexpr int SORT_W = SORT_T / 64;
constexpr int LSH_NB_LIMIT = 64;    // largest bucket count of the hash (rotation staged in LDS)
constexpr int SORT_NB_LIMIT = 512;  // largest bucket count of the sort (per-wave group counts in LDS)

}  // namespace

int lsh_max_nb() { return LSH_NB_LIMIT; }
int sort_max_nb() { return SORT_NB_LIMIT; }

// One thread per row. The head's rotation (d x nh floats, nh = nb / 2) is staged in LDS and read by
// all lanes at the same address. Scores are accumulated over d in increasing order with fused
// multiply-adds; the bucket is the first index of the maximum over [p_0 .. p_nh-1, -p_0 .. -p_nh-1].
template <typename T, int D>
__global__ __launch_bounds__(LSH_T) void lsh_buckets_kernel(const T* __restrict__ x, const float* __restrict__ rot,
                                                            int H, int N, int Hr, int nh, int* __restrict__ out) {
  __shared__ float r_lds[D * LSH_NB_LIMIT / 2];
  const int nblk = (N + LSH_T - 1) / LSH_T;
  const int bh = (int)(blockIdx.x / nblk);
  const int row = (int)(blockIdx.x % nblk) * LSH_T + (int)threadIdx.x;
  const float* rh = rot + (size_t)(Hr > 1 ? bh % H : 0) * D * nh;
  for (int i = threadIdx.x; i < D * nh; i += LSH_T) r_lds[i] = rh[i];
  __syncthreads();
  if (row >= N) return;
  const T* xr = x + ((size_t)bh * N + row) * D;
  float best_p = -INFINITY, best_n = -INFINITY;
  int arg_p = 0, arg_n = 0;
  for (int c0 = 0; c0 < nh; c0 += LSH_CB) {
    float acc[LSH_CB];
#pragma unroll
    for (int c = 0; c < LSH_CB; ++c) acc[c] = 0.f;
    constexpr int EPV = 16 / (int)sizeof(T);  // elements per 16-byte load
#pragma unroll 4
    for (int k0 = 0; k0 < D; k0 += EPV) {
      float xv[EPV];
      if constexpr (sizeof(T) == 2) {
        const bf16x8 w = *reinterpret_cast<const bf16x8*>(xr + k0);
#pragma unroll
        for (int e = 0; e < EPV; ++e) xv[e] = (float)w[e];
      } else {
        const f32x4 w = *reinterpret_cast<const f32x4*>(xr + k0);
#pragma unroll
        for (int e = 0; e < EPV; ++e) xv[e] = w[e];
      }
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        const float* rr = r_lds + (k0 + e) * nh + c0;
#pragma unroll
        for (int c = 0; c < LSH_CB; ++c)
          if (c0 + c < nh) acc[c] = fmaf(xv[e], rr[c], acc[c]);
      }
    }
#pragma unroll
    for (int c = 0; c < LSH_CB; ++c) {
      if (c0 + c < nh) {
        if (acc[c] > best_p) { best_p = acc[c]; arg_p = c0 + c; }
        if (-acc[c] > best_n) { best_n = -acc[c]; arg_n = c0 + c; }
      }
    }
  }
  out[(size_t)bh * N + row] = best_n > best_p ? nh + arg_n : arg_p;
}

// One workgroup per (b, h) row. Pass 1 counts each group (bucket, or nb for dropped tokens) of queries
// and keys; the exclusive scans give the first sorted position of every group. Pass 2 sweeps the
// positions 1024 at a time in increasing order: inside a wave the tokens of one group are ranked by a
// ballot per distinct group, per-wave group counts in LDS give the offsets of earlier waves, and running
// bases carry the counts of earlier chunks. This keeps the sort stable, and it gives every key the number
// of same-group queries at earlier positions, which is its lo.
__global__ __launch_bounds__(SORT_T) void bucket_sort_kernel(const int* __restrict__ qb, const int* __restrict__ kb,
                                                             int N, int nb, int* __restrict__ qidx,
                                                             int* __restrict__ qpos, int* __restrict__ kidx,
                                                             int* __restrict__ kpos, int* __restrict__ lts,
                                                             int* __restrict__ lte, int* __restrict__ uts,
                                                             int* __restrict__ ute) {
  constexpr int G_MAX = SORT_NB_LIMIT + 1;
  __shared__ int qbase[G_MAX], kbase[G_MAX], qend[G_MAX];
  __shared__ int qcnt[SORT_W][G_MAX], kcnt[SORT_W][G_MAX];
  const int G = nb + 1;
  const size_t base = (size_t)blockIdx.x * N;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  auto group = [&](int v) { return (v >= 0 && v < nb) ? v : nb; };

  for (int g = tid; g < G; g += SORT_T) { qbase[g] = 0; kbase[g] = 0; }
  __syncthreads();
  for (int j = tid; j < N; j += SORT_T) {
    atomicAdd(&qbase[group(qb[base + j])], 1);
    atomicAdd(&kbase[group(kb[base + j])], 1);
  }
  __syncthreads();
  // exclusive scans: wave 0 for queries, wave 1 for keys (each lane owns a run of groups)
  if (wave < 2) {
    int* h = wave == 0 ? qbase : kbase;
    const int per = (G + 63) / 64;
    const int g0 = min(G, lane * per), g1 = min(G, g0 + per);
    int run = 0;
    for (int g = g0; g < g1; ++g) run += h[g];
    int incl = run;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o, 64);
      if (lane >= o) incl += t;
    }
    int acc = incl - run;
    for (int g = g0; g < g1; ++g) {
      const int c = h[g];
      h[g] = acc;
      if (wave == 0) qend[g] = acc + c;
      acc += c;
    }
  }

  for (int c0 = 0; c0 < N; c0 += SORT_T) {
    __syncthreads();  // bases of the previous chunk updated, its counts consumed
    for (int g = lane; g < G; g += 64) {
      qcnt[wave][g] = 0;
      kcnt[wave][g] = 0;
    }
    const int j = c0 + tid;
    const bool valid = j < N;
    const int gq = valid ? group(qb[base + j]) : -1;
    const int gk = valid ? group(kb[base + j]) : -1;
    // queries: rank among same-group lanes of this wave, and the wave's count per group
    int rank_q = 0;
    uint64_t active = __ballot(valid);
    while (active != 0ull) {
      const int lead = __builtin_ctzll(active);
      const int v = __shfl(gq, lead, 64);
      const uint64_t m = __ballot(gq == v);
      if (gq == v) rank_q = __builtin_popcountll(m & lt_mask);
      if (lane == lead) qcnt[wave][v] = __builtin_popcountll(m);
      active &= ~m;
    }
    // keys: the same, plus the same-group queries at earlier lanes (earlier positions) of this wave
    int rank_k = 0, q_before = 0;
    active = __ballot(valid);
    while (active != 0ull) {
      const int lead = __builtin_ctzll(active);
      const int v = __shfl(gk, lead, 64);
      const uint64_t m = __ballot(gk == v);
      const uint64_t mq = __ballot(gq == v);
      if (gk == v) {
        rank_k = __builtin_popcountll(m & lt_mask);
        q_before = __builtin_popcountll(mq & lt_mask);
      }
      if (lane == lead) kcnt[wave][v] = __builtin_popcountll(m);
      active &= ~m;
    }
    __syncthreads();
    if (valid) {
      int off_q = 0, off_k = 0, off_kq = 0;
      for (int w = 0; w < wave; ++w) {
        off_q += qcnt[w][gq];
        off_k += kcnt[w][gk];
        off_kq += qcnt[w][gk];
      }
      const int pq = qbase[gq] + off_q + rank_q;
      qidx[base + pq] = j;
      qpos[base + j] = pq;
      const int pk = kbase[gk] + off_k + rank_k;
      kidx[base + pk] = j;
      kpos[base + j] = pk;
      if (gk == nb) {  // dropped key: every row masked
        uts[base + pk] = 0;
        ute[base + pk] = N;
        lts[base + pk] = N;
        lte[base + pk] = N;
      } else {
        uts[base + pk] = 0;
        ute[base + pk] = qbase[gk] + off_kq + q_before;  // lo: first row of the group at or after j
        lts[base + pk] = qend[gk];                       // N when the group ends last: canonical empty
        lte[base + pk] = N;
      }
    }
    __syncthreads();
    for (int g = tid; g < G; g += SORT_T) {
      int sq = 0, sk = 0;
#pragma unroll
      for (int w = 0; w < SORT_W; ++w) {
        sq += qcnt[w][g];
        sk += kcnt[w][g];
      }
      qbase[g] += sq;
      kbase[g] += sk;
    }
  }
}

hipError_t launch_lsh_buckets(bool bf16_in, int d, const void* x, const float* rot, int B, int H, int N, int Hr,
                              int nb, int* out, hipStream_t stream) {
  const long grid = (long)B * H * ((N + LSH_T - 1) / LSH_T);
  const int nh = nb / 2;
  if (bf16_in) {
    if (d == 64)
      hipLaunchKernelGGL((lsh_buckets_kernel<bf16, 64>), dim3((unsigned)grid), dim3(LSH_T), 0, stream,
                         static_cast<const bf16*>(x), rot, H, N, Hr, nh, out);
    else
      hipLaunchKernelGGL((lsh_buckets_kernel<bf16, 128>), dim3((unsigned)grid), dim3(LSH_T), 0, stream,
                         static_cast<const bf16*>(x), rot, H, N, Hr, nh, out);
  } else {
    if (d == 64)
      hipLaunchKernelGGL((lsh_buckets_kernel<float, 64>), dim3((unsigned)grid), dim3(LSH_T), 0, stream,
                         static_cast<const float*>(x), rot, H, N, Hr, nh, out);
    else
      hipLaunchKernelGGL((lsh_buckets_kernel<float, 128>), dim3((unsigned)grid), dim3(LSH_T), 0, stream,
                         static_cast<const float*>(x), rot, H, N, Hr, nh, out);
  }
  return hipGetLastError();
}

hipError_t launch_bucket_sort(const int* qb, const int* kb, int rows, int N, int nb, int* qidx, int* qpos,
                              int* kidx, int* kpos, int* lts, int* lte, int* uts, int* ute, hipStream_t stream) {
  hipLaunchKernelGGL(bucket_sort_kernel, dim3((unsigned)rows), dim3(SORT_T), 0, stream, qb, kb, N, nb, qidx, qpos,
                     kidx, kpos, lts, lte, uts, ute);
  return hipGetLastError();
}

}  // namespace fm
