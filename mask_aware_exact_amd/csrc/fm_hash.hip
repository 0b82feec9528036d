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
//                   geometric hashing), float32 dot products (matrix-core products for bf16 rows);
//                   HBM-bound (2 d bytes read per bf16 row).
//   fm_bucket_sort  stable counting sort of queries and keys by bucket (out-of-range buckets form a
//                   trailing dropped group that attends and is attended by nothing), the permutations
//                   both ways, and the sorted problem's four vectors, in one sweep per head.
#include "fm_common.h"

namespace fm {

namespace {

constexpr int LSH_T = 256;     // threads and rows per workgroup (64 rows per wave)
constexpr int LSH_CB = 8;      // rotation columns per pass
constexpr int LSH_BATCH = 4;   // row steps whose loads a wave issues together
constexpr int SORT_T = 1024;   // threads of the sort kernel (16 waves)
constexpr int SORT_W = SORT_T / 64;
constexpr int SORT_STAGE = 16;  // chunks of bucket groups staged in LDS at a time
constexpr int SORT_SEG = 2048;  // least tokens per segment when a head's sort is split over workgroups

template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of L lanes (L = 8, 16 or 32), the result in every lane of the group: quad
// swaps, then the mirror within 8 lanes and within 16 lanes (data-parallel moves on the vector ALU), then
// a cross-row exchange for 32.
template <int L>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp_move<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v += dpp_move<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v += dpp_move<0x141>(v);  // row_half_mirror
  if constexpr (L >= 16) v += dpp_move<0x140>(v);  // row_mirror
  if constexpr (L >= 32) v += __shfl_xor(v, 16, 64);
  return v;
}

}  // namespace

int lsh_max_nb() { return LSH_NB_LIMIT; }
int sort_max_nb() { return SORT_NB_LIMIT; }

// float32 rows: a row is read by a group of L = 16-byte chunks per row lanes (16 lanes at d = 64), so one
// load instruction of a wave covers 64 / L whole rows, contiguous in memory; a wave issues the loads of
// LSH_BATCH such steps before using them. The head's rotation (d x nh floats, nh = nb / 2) is staged in
// LDS grouped by chunk, each chunk's block padded by 4 floats so that the L lanes of a group, which read
// different chunks' blocks at the same time, fall into different banks. Each lane forms partial dot
// products over its chunk (the rotation slice kept in registers when nh <= 8), the group sums them with
// data-parallel lane moves (float32, a fixed order), and the group's first lane writes the first index of
// the maximum over [p_0 .. p_nh-1, -p_0 .. -p_nh-1].
template <typename T, int D>
__global__ __launch_bounds__(LSH_T) void lsh_buckets_kernel(const T* __restrict__ x, const float* __restrict__ rot,
                                                            int H, int N, int Hr, int nh, int* __restrict__ out) {
  constexpr int EPV = 16 / (int)sizeof(T);  // elements per 16-byte chunk
  constexpr int L = D / EPV;                 // lanes per row
  constexpr int RPI = 64 / L;                // rows per wave per step
  __shared__ __attribute__((aligned(16))) float r_lds[D * LSH_NB_LIMIT / 2 + 4 * L];
  const int nblk = (N + LSH_T - 1) / LSH_T;
  const int bh = (int)(blockIdx.x / nblk);
  const int row0 = (int)(blockIdx.x % nblk) * LSH_T;
  const float* rh = rot + (size_t)(Hr > 1 ? bh % H : 0) * D * nh;
  const int SP = EPV * nh + 4;  // floats per chunk block in LDS
  for (int i = threadIdx.x; i < D * nh; i += LSH_T) {
    const int k = i / nh, c = i - k * nh;
    r_lds[(k / EPV) * SP + (k % EPV) * nh + c] = rh[i];
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane % L;  // this lane's chunk of the row
  const float* rl = r_lds + sub * SP;
  static_assert(L == 8 || L == 16 || L == 32, "lane groups the reduction supports");
  const bool small = nh <= LSH_CB;  // the whole rotation slice of this lane fits in registers
  float rreg[EPV][LSH_CB];
#pragma unroll
  for (int e = 0; e < EPV; ++e)
#pragma unroll
    for (int c = 0; c < LSH_CB; ++c) rreg[e][c] = (small && c < nh) ? rl[e * nh + c] : 0.f;
  static_assert((64 / RPI) % LSH_BATCH == 0, "row steps per wave split into whole batches");
  for (int it0 = 0; it0 < 64 / RPI; it0 += LSH_BATCH) {
    i32x4 raw[LSH_BATCH];
#pragma unroll
    for (int u = 0; u < LSH_BATCH; ++u) {  // the batch's loads, all in flight together
      const int r = row0 + wave * 64 + (it0 + u) * RPI + lane / L;
      raw[u] = r < N ? *reinterpret_cast<const i32x4*>(x + ((size_t)bh * N + r) * D + sub * EPV)
                     : i32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < LSH_BATCH; ++u) {
      const int row = row0 + wave * 64 + (it0 + u) * RPI + lane / L;
      float xv[EPV];
      if constexpr (sizeof(T) == 2) {
        const bf16x8 v = __builtin_bit_cast(bf16x8, raw[u]);
#pragma unroll
        for (int e = 0; e < EPV; ++e) xv[e] = (float)v[e];
      } else {
        const f32x4 v = __builtin_bit_cast(f32x4, raw[u]);
#pragma unroll
        for (int e = 0; e < EPV; ++e) xv[e] = v[e];
      }
      float best_p = -INFINITY, best_n = -INFINITY;
      int arg_p = 0, arg_n = 0;
      for (int c0 = 0; c0 < nh; c0 += LSH_CB) {
        float acc[LSH_CB];
#pragma unroll
        for (int c = 0; c < LSH_CB; ++c) acc[c] = 0.f;
        if (small) {
#pragma unroll
          for (int e = 0; e < EPV; ++e)
#pragma unroll
            for (int c = 0; c < LSH_CB; ++c) acc[c] = fmaf(xv[e], rreg[e][c], acc[c]);
        } else {
#pragma unroll
          for (int e = 0; e < EPV; ++e) {
            const float* rr = rl + e * nh + c0;
#pragma unroll
            for (int c = 0; c < LSH_CB; ++c)
              if (c0 + c < nh) acc[c] = fmaf(xv[e], rr[c], acc[c]);
          }
        }
#pragma unroll
        for (int c = 0; c < LSH_CB; ++c) acc[c] = group_sum<L>(acc[c]);
#pragma unroll
        for (int c = 0; c < LSH_CB; ++c) {
          if (c0 + c < nh) {
            if (acc[c] > best_p) { best_p = acc[c]; arg_p = c0 + c; }
            if (-acc[c] > best_n) { best_n = -acc[c]; arg_n = c0 + c; }
          }
        }
      }
      if (row < N && sub == 0) out[(size_t)bh * N + row] = best_n > best_p ? nh + arg_n : arg_p;
    }
  }
}

// Segment s of nseg equal parts of [0, N).
__device__ __forceinline__ int seg_begin(int s, int N, int nseg) { return (int)((long)s * N / nseg); }

// Split sort, pass 1: the group counts of one segment (queries, then keys) into the first 2 G entries of the
// segment's own qpos range (a segment holds at least SORT_SEG >= 3 G positions).
__global__ __launch_bounds__(256) void bucket_count_kernel(const int* __restrict__ qb, const int* __restrict__ kb, int N,
                                                           int nb, int nseg, int* __restrict__ qpos) {
  constexpr int G_MAX = SORT_NB_LIMIT + 1;
  __shared__ int hq[G_MAX], hk[G_MAX];
  const int G = nb + 1;
  const int row = (int)(blockIdx.x / nseg), seg = (int)(blockIdx.x % nseg);
  const size_t base = (size_t)row * N;
  const int s0 = seg_begin(seg, N, nseg), s1 = seg_begin(seg + 1, N, nseg);
  for (int g = threadIdx.x; g < G; g += 256) { hq[g] = 0; hk[g] = 0; }
  __syncthreads();
  for (int j = s0 + (int)threadIdx.x; j < s1; j += 256) {
    const int vq = qb[base + j], vk = kb[base + j];
    atomicAdd(&hq[(vq >= 0 && vq < nb) ? vq : nb], 1);
    atomicAdd(&hk[(vk >= 0 && vk < nb) ? vk : nb], 1);
  }
  __syncthreads();
  for (int g = threadIdx.x; g < G; g += 256) {
    qpos[base + s0 + g] = hq[g];
    qpos[base + s0 + G + g] = hk[g];
  }
}

// Split sort, pass 2 (one workgroup per row): group totals, their exclusive scans (the first sorted position
// of each group), and for every segment the position its first token of each group takes, replacing the
// counts in place; the query group ends go to entries [2 G, 3 G) of every segment. Column j < 2 G of the
// counts (queries at j < G, keys at j >= G) is the work of S lanes of a wave, S the segment count rounded
// up to a power of two and at most 64, with the lanes over S segments at a time: a prefix sum over the S
// lanes turns the counts into the positions before the segment within the group, written in place, and
// the last lane's running sum is the group total. After the scans over groups, the same lanes add each
// group's first position. Every entry is read and written by one lane.
template <int W>
__device__ __forceinline__ int group_incl_sum(int v, int sl, int S) {  // over aligned groups of S lanes
#pragma unroll
  for (int o = 1; o < W; o <<= 1) {
    const int t = __shfl_up(v, o, S);
    if (o < S && sl >= o) v += t;
  }
  return v;
}

__global__ __launch_bounds__(1024) void bucket_scan_kernel(int N, int nb, int nseg, int* __restrict__ qpos) {
  constexpr int G_MAX = SORT_NB_LIMIT + 1;
  __shared__ int tot[2 * G_MAX], qe[G_MAX];
  const int G = nb + 1;
  const size_t base = (size_t)blockIdx.x * N;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = nseg >= 64 ? 64 : 1 << (32 - __builtin_clz((unsigned)(nseg - 1) | 1u));  // lanes per column
  const int cpw = 64 / S;  // columns per wave at a time
  const int sub = lane / S, sl = lane % S;
  for (int j0 = wave * cpw; j0 < 2 * G; j0 += 16 * cpw) {
    const int j = j0 + sub;
    int carry = 0;
    for (int s0 = 0; s0 < nseg; s0 += S) {
      const int sg = s0 + sl;
      const bool live = j < 2 * G && sg < nseg;
      const size_t o = base + seg_begin(min(sg, nseg - 1), N, nseg) + min(j, 2 * G - 1);
      const int c = live ? qpos[o] : 0;
      const int incl = group_incl_sum<64>(c, sl, S);
      if (live) qpos[o] = carry + incl - c;
      carry += __shfl(incl, S - 1, S);
    }
    if (j < 2 * G && sl == 0) tot[j] = carry;
  }
  __syncthreads();
  if (wave < 2) {  // exclusive scans over groups: wave 0 queries, wave 1 keys
    int* h = tot + wave * G;
    const int per = (G + 63) / 64;
    const int g0 = min(G, lane * per), g1 = min(G, g0 + per);
    int run = 0;
    for (int g = g0; g < g1; ++g) run += h[g];
    int acc = group_incl_sum<64>(run, lane, 64) - run;
    for (int g = g0; g < g1; ++g) {
      const int c = h[g];
      h[g] = acc;
      if (wave == 0) qe[g] = acc + c;
      acc += c;
    }
  }
  __syncthreads();
  for (int j0 = wave * cpw; j0 < 2 * G; j0 += 16 * cpw) {
    const int j = j0 + sub;
    if (j >= 2 * G) continue;
    const int start = tot[j];
    for (int s0 = 0; s0 < nseg; s0 += S) {
      const int sg = s0 + sl;
      if (sg < nseg) {
        const size_t o = base + seg_begin(sg, N, nseg);
        qpos[o + j] += start;
        if (j < G) qpos[o + 2 * G + j] = qe[j];
      }
    }
  }
}

// One workgroup per (b, h) row. Pass 1 counts each group (bucket, or nb for dropped tokens) of queries
// and keys; the exclusive scans give the first sorted position of every group. Pass 2 sweeps the
// positions 1024 at a time in increasing order: inside a wave the tokens of one group are ranked with one
// ballot per bit of the group id, per-wave group counts in LDS give the offsets of earlier waves, and running
// bases carry the counts of earlier chunks. This keeps the sort stable, and it gives every key the number
// of same-group queries at earlier positions, which is its lo. The bucket groups of SORT_STAGE chunks are
// loaded into LDS (16 bits each) at once: the vector memory counter covers loads and stores alike, so
// waiting for loads also waits for the scattered output stores, and staging makes that one wait per
// SORT_STAGE chunks. The bases are double-buffered and the per-wave counts carry their chunk number
// (count | chunk << 16), so two barriers per chunk suffice and nothing is cleared.
__global__ __launch_bounds__(SORT_T) void bucket_sort_kernel(const int* __restrict__ qb, const int* __restrict__ kb,
                                                             int N, int nb, int nseg, int* __restrict__ qidx,
                                                             int* __restrict__ qpos, int* __restrict__ kidx,
                                                             int* __restrict__ kpos, int* __restrict__ lts,
                                                             int* __restrict__ lte, int* __restrict__ uts,
                                                             int* __restrict__ ute) {
  constexpr int G_MAX = SORT_NB_LIMIT + 1;
  __shared__ int qbase[2][G_MAX], kbase[2][G_MAX], qend[G_MAX];
  __shared__ unsigned qcnt[SORT_W][G_MAX], kcnt[SORT_W][G_MAX];
  __shared__ uint16_t qg_lds[SORT_STAGE * SORT_T], kg_lds[SORT_STAGE * SORT_T];
  const int G = nb + 1;
  const int nbits = 32 - __builtin_clz((unsigned)nb);  // bits of the largest group id, nb (>= 1)
  const int row = (int)(blockIdx.x / nseg), seg = (int)(blockIdx.x % nseg);
  const size_t base = (size_t)row * N;
  const int s0 = seg_begin(seg, N, nseg), s1 = seg_begin(seg + 1, N, nseg);  // this workgroup's positions
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  auto group = [&](int v) { return (v >= 0 && v < nb) ? v : nb; };

  for (int i = tid; i < SORT_W * G_MAX; i += SORT_T) {
    (&qcnt[0][0])[i] = 0xFFFFFFFFu;  // chunk tag 0xFFFF: no chunk
    (&kcnt[0][0])[i] = 0xFFFFFFFFu;
  }
  if (nseg > 1) {
    // bases of this segment and the group ends, left in the segment's own qpos range by the scan
    for (int g = tid; g < G; g += SORT_T) {
      qbase[0][g] = qpos[base + s0 + g];
      kbase[0][g] = qpos[base + s0 + G + g];
      qend[g] = qpos[base + s0 + 2 * G + g];
    }
  } else {  // one workgroup for the whole row: count and scan here
    for (int g = tid; g < G; g += SORT_T) { qbase[0][g] = 0; kbase[0][g] = 0; }
    __syncthreads();
    for (int j0 = tid; j0 < N; j0 += 4 * SORT_T) {
      int vq[4], vk[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = j0 + u * SORT_T;
        vq[u] = j < N ? qb[base + j] : 0;
        vk[u] = j < N ? kb[base + j] : 0;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (j0 + u * SORT_T < N) {
          atomicAdd(&qbase[0][group(vq[u])], 1);
          atomicAdd(&kbase[0][group(vk[u])], 1);
        }
      }
    }
    __syncthreads();
    // exclusive scans: wave 0 for queries, wave 1 for keys (each lane owns a run of groups)
    if (wave < 2) {
      int* h = wave == 0 ? qbase[0] : kbase[0];
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
  }

  auto count_of = [](unsigned c, unsigned chunk) { return (c >> 16) == chunk ? (int)(c & 0xFFFFu) : 0; };
  int par = 0;
  unsigned chunk = 0;
  __syncthreads();  // bases and group ends are in LDS before any position is written (qpos held them)
  for (int c0 = s0; c0 < s1; c0 += SORT_T, ++chunk, par ^= 1) {
    const int j = c0 + tid;
    const bool valid = j < s1;
    const int slot = (int)(chunk % SORT_STAGE);
    if (slot == 0) {  // stage the groups of the next SORT_STAGE chunks
      __syncthreads();  // the previous stage is consumed
      int vq[SORT_STAGE], vk[SORT_STAGE];
#pragma unroll
      for (int u = 0; u < SORT_STAGE; ++u) {
        const int jj = j + u * SORT_T;
        vq[u] = jj < s1 ? qb[base + jj] : 0;
        vk[u] = jj < s1 ? kb[base + jj] : 0;
      }
#pragma unroll
      for (int u = 0; u < SORT_STAGE; ++u) {
        qg_lds[u * SORT_T + tid] = (uint16_t)group(vq[u]);
        kg_lds[u * SORT_T + tid] = (uint16_t)group(vk[u]);
      }
    }
    __syncthreads();  // the previous chunk's counts and bases are consumed; the new bases are visible
    const int gq = valid ? (int)qg_lds[slot * SORT_T + tid] : -1;
    const int gk = valid ? (int)kg_lds[slot * SORT_T + tid] : -1;
    // Same-group lane masks by one ballot per bit of the group id: a lane's mask is the AND over the
    // bits of the ballot (bit set) or its complement (bit clear). The query-bit ballots also give, for
    // each key, the queries of the key's group in this wave.
    const uint64_t vmask = __ballot(valid);
    uint64_t same_q = vmask, same_k = vmask, q_of_k = vmask;
    for (int bit = 0; bit < nbits; ++bit) {
      const uint64_t bq = __ballot(valid && ((gq >> bit) & 1));
      const uint64_t bk = __ballot(valid && ((gk >> bit) & 1));
      same_q &= ((gq >> bit) & 1) ? bq : ~bq;
      same_k &= ((gk >> bit) & 1) ? bk : ~bk;
      q_of_k &= ((gk >> bit) & 1) ? bq : ~bq;
    }
    const int rank_q = __builtin_popcountll(same_q & lt_mask);
    const int rank_k = __builtin_popcountll(same_k & lt_mask);
    const int q_before = __builtin_popcountll(q_of_k & lt_mask);
    // the first lane of each group in this wave records the wave's count for it
    if (valid && rank_q == 0) qcnt[wave][gq] = (chunk << 16) | (unsigned)__builtin_popcountll(same_q);
    if (valid && rank_k == 0) kcnt[wave][gk] = (chunk << 16) | (unsigned)__builtin_popcountll(same_k);
    __syncthreads();
    if (valid) {
      int off_q = 0, off_k = 0, off_kq = 0;
#pragma unroll
      for (int w = 0; w < SORT_W; ++w) {  // all reads issued together; earlier waves counted
        const int a = count_of(qcnt[w][gq], chunk), b = count_of(kcnt[w][gk], chunk);
        const int c = count_of(qcnt[w][gk], chunk);
        off_q += w < wave ? a : 0;
        off_k += w < wave ? b : 0;
        off_kq += w < wave ? c : 0;
      }
      const int pq = qbase[par][gq] + off_q + rank_q;
      qidx[base + pq] = j;
      qpos[base + j] = pq;
      const int pk = kbase[par][gk] + off_k + rank_k;
      kidx[base + pk] = j;
      kpos[base + j] = pk;
      if (gk == nb) {  // dropped key: every row masked
        uts[base + pk] = 0;
        ute[base + pk] = N;
        lts[base + pk] = N;
        lte[base + pk] = N;
      } else {
        uts[base + pk] = 0;
        ute[base + pk] = qbase[par][gk] + off_kq + q_before;  // lo: first row of the group at or after j
        lts[base + pk] = qend[gk];                            // N when the group ends last: canonical empty
        lte[base + pk] = N;
      }
    }
    for (int g = tid; g < G; g += SORT_T) {
      int sq = 0, sk = 0;
#pragma unroll
      for (int w = 0; w < SORT_W; ++w) {
        sq += count_of(qcnt[w][g], chunk);
        sk += count_of(kcnt[w][g], chunk);
      }
      qbase[par ^ 1][g] = qbase[par][g] + sq;
      kbase[par ^ 1][g] = kbase[par][g] + sk;
    }
  }
}

// bf16 rows: the projections x R of 32 rows at a time as one matrix product. The rotation is the A operand
// (rows = rotation columns c, zero past nh; k = d) and the row block the B operand (k = d, columns = rows).
// R is split into three bf16 parts, hi = bf16(R), mid = bf16(R - hi), lo = bf16(R - hi - mid), which
// leave less than 2^-24 |R| out; their products with the bf16 row are exact in float32 and accumulate in
// float32 (hi in one accumulator, mid and lo in another). Lane (l32, g) then holds the 16 projections
// c = 8 (r / 4) + 4 g + r % 4 of row l32, so the first index of the maximum takes 16 compares in the lane
// and one exchange with lane ^ 32. The parts are staged once per workgroup in LDS in operand order
// (lane-linear 16-byte reads), read one k step at a time, so that four waves per SIMD fit in the
// registers to keep enough row loads in flight. Each wave takes one 32-row block.
constexpr int LSHM_ROWS = 128;  // rows per workgroup: four waves of 32

template <int D>
__global__ __launch_bounds__(LSH_T) __attribute__((amdgpu_waves_per_eu(4))) void lsh_buckets_mfma_kernel(const bf16* __restrict__ x,
                                                                 const float* __restrict__ rot, int H, int N, int Hr,
                                                                 int nh, int* __restrict__ out) {
  constexpr int NK = D / 16;  // k steps of one product
  static_assert(NK % 4 == 0 || 4 % NK == 0, "the waves split the rotation's k steps evenly");
  __shared__ __attribute__((aligned(16))) bf16x8 a_lds[3][NK][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int nblk = (N + LSHM_ROWS - 1) / LSHM_ROWS;
  const int bh = (int)(blockIdx.x / nblk);
  const int row = (int)(blockIdx.x % nblk) * LSHM_ROWS + wave * 32 + l32;  // this lane's row
  const float* rh = rot + (size_t)(Hr > 1 ? bh % H : 0) * D * nh;
  const bf16* xh = x + (size_t)bh * N * D;

  // the row's fragments (rows past N read row N - 1; their buckets are not written)
  bf16x8 xf[NK];
  {
    const int r = min(row, N - 1);
#pragma unroll
    for (int k = 0; k < NK; ++k) xf[k] = load_kcontig_frag<bf16>(xh + (size_t)r * D + k * 16 + 8 * g);
  }
  for (int k = wave; k < NK; k += 4) {
    bf16x8 hi, mid, lo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = l32 < nh ? rh[(size_t)(k * 16 + 8 * g + e) * nh + l32] : 0.f;
      hi[e] = (bf16)v;
      const float v1 = v - (float)hi[e];
      mid[e] = (bf16)v1;
      lo[e] = (bf16)(v1 - (float)mid[e]);
    }
    a_lds[0][k][lane] = hi;
    a_lds[1][k][lane] = mid;
    a_lds[2][k][lane] = lo;
  }
  __syncthreads();

  {
    f32x16 acc = zero16(), acc2 = zero16();
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      acc = MM<bf16>::mma(a_lds[0][k][lane], xf[k], acc);
      acc2 = MM<bf16>::mma(a_lds[1][k][lane], xf[k], acc2);
      acc2 = MM<bf16>::mma(a_lds[2][k][lane], xf[k], acc2);
      __builtin_amdgcn_sched_barrier(0);  // keep the next step's operand reads after these products
    }
    float best_p = -INFINITY, best_n = -INFINITY;
    int arg_p = 0, arg_n = 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) {  // c increases with r: strict compares keep the first index
      const int c = 8 * (r >> 2) + 4 * g + (r & 3);
      const float v = acc[r] + acc2[r];
      if (c < nh) {
        if (v > best_p) { best_p = v; arg_p = c; }
        if (-v > best_n) { best_n = -v; arg_n = c; }
      }
    }
    const float op = __shfl_xor(best_p, 32, 64), on = __shfl_xor(best_n, 32, 64);
    const int oap = __shfl_xor(arg_p, 32, 64), oan = __shfl_xor(arg_n, 32, 64);
    if (op > best_p || (op == best_p && oap < arg_p)) { best_p = op; arg_p = oap; }
    if (on > best_n || (on == best_n && oan < arg_n)) { best_n = on; arg_n = oan; }
    if (g == 0 && row < N) out[(size_t)bh * N + row] = best_n > best_p ? nh + arg_n : arg_p;
  }
}

hipError_t launch_lsh_buckets(bool bf16_in, int d, const void* x, const float* rot, int B, int H, int N, int Hr,
                              int nb, int* out, hipStream_t stream) {
  const long grid = (long)B * H * ((N + LSH_T - 1) / LSH_T);
  const long grid_m = (long)B * H * ((N + LSHM_ROWS - 1) / LSHM_ROWS);
  const int nh = nb / 2;
  if (bf16_in) {
    if (d == 64)
      hipLaunchKernelGGL((lsh_buckets_mfma_kernel<64>), dim3((unsigned)grid_m), dim3(LSH_T), 0, stream,
                         static_cast<const bf16*>(x), rot, H, N, Hr, nh, out);
    else
      hipLaunchKernelGGL((lsh_buckets_mfma_kernel<128>), dim3((unsigned)grid_m), dim3(LSH_T), 0, stream,
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
  // Long rows are split into segments of at least SORT_SEG positions, one workgroup each, after a count
  // and a scan pass; short rows take one workgroup that counts and scans for itself.
  const int nseg = N >= 2 * SORT_SEG ? N / SORT_SEG : 1;
  static_assert(SORT_SEG >= 3 * (SORT_NB_LIMIT + 1), "a segment holds its counts, bases and the group ends");
  if (nseg > 1) {
    hipLaunchKernelGGL(bucket_count_kernel, dim3((unsigned)((long)rows * nseg)), dim3(256), 0, stream, qb, kb, N, nb,
                       nseg, qpos);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bucket_scan_kernel, dim3((unsigned)rows), dim3(1024), 0, stream, N, nb, nseg, qpos);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(bucket_sort_kernel, dim3((unsigned)((long)rows * nseg)), dim3(SORT_T), 0, stream, qb, kb, N, nb,
                     nseg, qidx, qpos, kidx, kpos, lts, lte, uts, ute);
  return hipGetLastError();
}

}  // namespace fm
