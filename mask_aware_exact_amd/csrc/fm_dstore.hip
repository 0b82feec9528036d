// Backward with stored dS tiles (gfx950): the key-tile-parallel dK/dV pass writes every dS tile it forms,
// and dQ = scale * dS K becomes a streaming, block-sparse product over the stored tiles instead of a second
// pass that recomputes S, dP, P and dS (4 d FLOP per unmasked pair less matrix work, paid for with
// 2 bytes of HBM writes and reads per stored (query, key) pair). The pages do not describe the backward's
// work split; tiles that the mask covers completely are skipped on both sides as in the forward
// (FlashMask abstract, papers.pytorch.kr 2410.01359).
//
// Storage unit: one dS tile = 64 query rows x 128 keys (the dK/dV pass's query tile against its key
// tile), bf16, 16 KB. A (key tile, query tile) pair gets a tile when the dK/dV pass visits it (class not
// FULL). Per (b, hm, key tile) the visited query tiles lie between the first and last live one; the plan
// gives each key tile that whole span (a FULL tile inside it keeps an unused slot), so the slot of a pair
// is base[key tile] + (query tile - first[key tile]) inside the region of its (b, h).
//
// Tile layout (written by role 1 of the dK/dV pass with 16-byte stores, each wave instruction covering
// 1 KB contiguous): key group kg (32 keys), store s = 2 ib + p and position w hold 8 bf16 at byte
//     ((kg * 4 + s) * 64 + w) * 16,   w = g * 32 + (kl ^ (8 g + 4 p)),
// for key 32 kg + kl: query rows 32 ib + 16 p + 4 g + (0..3), then 32 ib + 16 p + 8 + 4 g + (0..3). The
// XOR spreads the reads of the dQ pass (transposing 8-byte reads, below) over all 32 bank pairs of a half
// wave.
#include "fm_common.h"

namespace fm {

// ------------------------------------------------------------------ plan

struct PlanArgs {
  const int* bounds;
  int B, H, Hm, N;
  int causal;
  int nkb;  // bounds entries per (b, hm) row
  int nkt;  // 128-key tiles per row
  int nq;   // 64-row query tiles per head
  long long* total;     // [1]
  long long* region;    // [B * H]
  long long* base;      // [B * Hm * nkt]: span, then (after the scan) the exclusive prefix of the spans
  long long* rowtotal;  // [B * Hm]
  int* first;           // [B * Hm * nkt]
};

// One wave per (b, hm, key tile): the first and last live 64-row query tile, 64 tiles per ballot from
// each end. The classification is exactly the dK/dV pass's.
__global__ __launch_bounds__(256) void ds_span_kernel(PlanArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long long gw = (long long)blockIdx.x * 4 + wave;
  if (gw >= (long long)a.B * a.Hm * a.nkt) return;
  const long long row = gw / a.nkt;
  const int kt = (int)(gw % a.nkt);
  const int N = a.N;
  const int* brow = a.bounds == nullptr ? nullptr : a.bounds + row * a.nkb * 8;
  const TileBounds bnd = merged_bounds(brow, 2 * kt, min(a.nkb, 2 * kt + 2), N);
  const int c0 = kt * DS_KEYS, c1 = min(N, c0 + DS_KEYS);
  const bool causal = a.causal != 0;
  auto live = [&](int qt) {
    return classify_tile(qt * DS_QROWS, min(N, qt * DS_QROWS + DS_QROWS), c0, c1, bnd, causal) != CLS_FULL;
  };
  const int begin = causal ? c0 / DS_QROWS : 0;
  int first = -1;
  for (int s = begin; s < a.nq; s += 64) {
    const int qt = s + lane;
    const uint64_t m = __ballot(qt < a.nq && live(qt));
    if (m != 0) {
      first = s + __builtin_ctzll(m);
      break;
    }
  }
  int last = -1;
  if (first >= 0) {
    for (int top = a.nq; top > first; top -= 64) {
      const int qt = top - 64 + lane;
      const uint64_t m = __ballot(qt >= first && live(qt));
      if (m != 0) {
        last = top - 64 + 63 - __builtin_clzll(m);
        break;
      }
    }
  }
  if (lane == 0) {
    a.first[gw] = first < 0 ? 0 : first;
    a.base[gw] = first < 0 ? 0 : (long long)(last - first + 1);
  }
}

// Exclusive prefix sum over n int64 values in place, by one workgroup of 256 threads; returns the total
// (valid in every thread).
__device__ long long block_exclusive_scan(long long* v, long long n, long long* lds) {
  const int tid = threadIdx.x;
  const long long per = (n + 255) / 256;
  const long long s0 = min(n, tid * per), s1 = min(n, s0 + per);
  long long sum = 0;
  for (long long i = s0; i < s1; ++i) sum += v[i];
  lds[tid] = sum;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const long long add = tid >= off ? lds[tid - off] : 0;
    __syncthreads();
    lds[tid] += add;
    __syncthreads();
  }
  long long run = lds[tid] - sum;  // exclusive prefix of this thread's chunk
  const long long total = lds[255];
  for (long long i = s0; i < s1; ++i) {
    const long long x = v[i];
    v[i] = run;
    run += x;
  }
  __syncthreads();
  return total;
}

// One workgroup per (b, hm): spans -> exclusive prefix, and the row's total.
__global__ __launch_bounds__(256) void ds_row_scan_kernel(PlanArgs a) {
  __shared__ long long lds[256];
  const long long row = blockIdx.x;
  const long long t = block_exclusive_scan(a.base + row * a.nkt, a.nkt, lds);
  if (threadIdx.x == 0) a.rowtotal[row] = t;
}

// One workgroup: the region of each (b, h), heads in order, and the grand total.
__global__ __launch_bounds__(256) void ds_region_kernel(PlanArgs a) {
  __shared__ long long lds[256];
  const long long n = (long long)a.B * a.H;
  for (long long i = threadIdx.x; i < n; i += 256) {
    const long long b = i / a.H, h = i % a.H;
    a.region[i] = a.rowtotal[b * a.Hm + (a.Hm > 1 ? h : 0)];
  }
  __syncthreads();
  const long long t = block_exclusive_scan(a.region, n, lds);
  if (threadIdx.x == 0) *a.total = t;
}

hipError_t launch_ds_plan(const int* bounds, int B, int H, int Hm, int N, int causal, void* plan,
                          hipStream_t stream) {
  const DsPlan v = ds_plan_view(plan, B, H, Hm, N);
  PlanArgs a;
  a.bounds = bounds;
  a.B = B; a.H = H; a.Hm = Hm; a.N = N;
  a.causal = causal;
  a.nkb = (N + KBLOCK - 1) / KBLOCK;
  a.nkt = v.nkt;
  a.nq = (N + DS_QROWS - 1) / DS_QROWS;
  a.total = v.total; a.region = v.region; a.base = v.base; a.rowtotal = v.rowtotal; a.first = v.first;
  const long long waves = (long long)B * Hm * a.nkt;
  hipLaunchKernelGGL(ds_span_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ds_row_scan_kernel, dim3((unsigned)(B * Hm)), dim3(256), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ds_region_kernel, dim3(1), dim3(256), 0, stream, a);
  return hipGetLastError();
}

// ------------------------------------------------------------------ dQ from the stored tiles

struct DqsArgs {
  const bf16* k;
  const char* ds;  // the stored tiles
  bf16* dq;
  const int* bounds;
  DsPlan plan;
  long long cap;  // stored tiles that fit in the cache
  int B, H, Hm, N;
  int nkb;
  int causal;
  float scale;
};

// Wait until at most n of this wave's vector memory operations are outstanding (they complete in issue
// order); n is wave-uniform and small.
__device__ __forceinline__ void wait_vm_at_most(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0); break;
    case 1: __builtin_amdgcn_s_waitcnt(1); break;
    case 2: __builtin_amdgcn_s_waitcnt(2); break;
    case 3: __builtin_amdgcn_s_waitcnt(3); break;
    case 4: __builtin_amdgcn_s_waitcnt(4); break;
    case 5: __builtin_amdgcn_s_waitcnt(5); break;
    default: __builtin_amdgcn_s_waitcnt(6); break;
  }
}

// One workgroup of 8 waves per (b, h, 256-row query tile) of a head whose tiles are stored: rows
// [256 qt + 64 x, + 64) form stored query tile 4 qt + x ("quarter x"). Wave w owns the 32 rows 32 (w & 1)
// of quarter w >> 1 and accumulates dQ^T += K^T dS^T over the live 64-key steps: K from a swizzled LDS
// tile shared by the 8 waves (transposing reads), dS^T from the stored tiles copied verbatim into LDS
// (transposing 8-byte reads whose per-lane addresses pick the layout apart). No masking is needed:
// masked pairs hold dS = 0. Steps are triple-buffered with two in flight, so that the HBM stream of
// stored tiles keeps enough bytes requested to cover the memory latency.
template <int D>
__global__ __launch_bounds__(512, 1) void dq_stream_kernel(DqsArgs a) {
  using M = MM<bf16>;
  constexpr int BC = 64;        // keys per step
  constexpr int QROWS = 256;    // query rows per workgroup
  constexpr int NQ = QROWS / DS_QROWS;  // stored query tiles per workgroup
  constexpr int NDB = D / 32;
  constexpr int HALF = BC * DS_QROWS * 2;  // bytes of one stored query tile's 64-key half (8 KB)
  constexpr int NBUF = 3;
  constexpr int KCOPY = TileCopy<D, BC, 8>::NK;  // K copy instructions per wave and step
  __shared__ __attribute__((aligned(16))) bf16 k_lds[NBUF][BC * D];
  __shared__ __attribute__((aligned(16))) char s_lds[NBUF][NQ][HALF];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int g = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(wave);

  const int BH = a.B * a.H;
  const int bh = blockIdx.x % BH;
  const int rank = (int)(blockIdx.x / BH);
  const int b = bh / a.H;
  const int h = bh % a.H;
  const int hm = a.Hm > 1 ? h : 0;
  const long long mrow = (long long)b * a.Hm + hm;
  if (!ds_head_stored(a.plan, a.cap, bh, mrow)) return;  // this head is handled by the recomputing pass
  const long long region = a.plan.region[bh];
  const int N = a.N;
  const int nq = (N + QROWS - 1) / QROWS;
  const int qt = nq - 1 - rank;  // heaviest (latest) query tiles first
  const int r0 = qt * QROWS;
  const int r1 = min(N, r0 + QROWS);
  const int quarter = wave >> 1, ib = wave & 1;

  const bf16* __restrict__ kg = a.k + (size_t)bh * N * D;
  const int* brow = a.bounds == nullptr ? nullptr : a.bounds + mrow * a.nkb * 8;
  const int* pfirst = a.plan.first + mrow * a.plan.nkt;
  const bool causal = a.causal != 0;

  // Live 64-key steps, 64 at a time: lane l of a window describes step t = wbase + l. Quarter x is live
  // against key tile t when its class is not FULL (then the 128-key stored tile that holds t is live too:
  // a FULL merged tile is FULL in each half) and its slot lies inside the plan's span for that tile (always,
  // for a plan that belongs to the problem). The lane keeps the slot of quarter 0 for its step in
  // registers; a step reads it with readlane, so that no memory load sits between the tile copies in flight
  // (the compiler's wait for such a load would also wait for the untracked copies).
  const int nkt = (N + BC - 1) / BC;
  const int kt_end = causal ? min(nkt, (r1 - 1) / BC + 1) : nkt;
  int wbase = -64;
  uint64_t wl[NQ] = {0, 0, 0, 0};
  long long wslot = 0;  // this lane's step: slot of quarter 0 (region + lo - first + NQ qt)
  auto next_live = [&](int from) {
    while (from < kt_end) {
      if (from >= wbase + 64) {
        wbase = from;
        const int t = from + lane;
        const bool in = t < kt_end;
        const TileBounds bt = merged_bounds(brow, in ? t : 0, in ? t + 1 : 1, N);
        const int c0 = t * BC, c1 = min(N, c0 + BC);
        long long lo = 0, span = 0;
        int first = 0;
        if (in) {
          span = ds_tile_span(a.plan, mrow, t >> 1, lo);
          first = pfirst[t >> 1];
        }
        wslot = region + lo - first + (long long)NQ * qt;
#pragma unroll
        for (int x = 0; x < NQ; ++x) {
          const int q0 = r0 + x * DS_QROWS, q1 = min(N, q0 + DS_QROWS);
          const long long r = (long long)NQ * qt + x - first;
          wl[x] = __ballot(in && q0 < q1 && r >= 0 && r < span &&
                           classify_tile(q0, q1, c0, c1, bt, causal) != CLS_FULL);
        }
        __builtin_amdgcn_s_waitcnt(0);  // the window's loads are done before any further copy is issued
      }
      const uint64_t rest = (wl[0] | wl[1] | wl[2] | wl[3]) >> (from - wbase);
      if (rest != 0) return from + __builtin_ctzll(rest);
      from = wbase + 64;
    }
    return kt_end;
  };

  // Per-lane LDS byte offsets of the transposing dS reads (the tile layout at the top of this file): lane
  // u = 4 i + j of its 16-lane group G addresses key 16 tk + 8 hi + 4 g + i and rows
  // 32 ib + 16 (G & 1) + 4 j .. + 3 of its stored query tile, i.e. store p = G & 1 of block ib, written by
  // lane (g' = j & 1, kl), the 8-byte half j >> 1.
  int soff[2][2];  // [tk & 1][hi]
  {
    const int G = lane >> 4, u = lane & 15, i = u >> 2, j = u & 3;
    const int p = G & 1, gp = j & 1;
    const int X = 8 * gp + 4 * p;
#pragma unroll
    for (int t1 = 0; t1 < 2; ++t1) {
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) {
        const int kl = 16 * t1 + 8 * hi + 4 * g + i;
        soff[t1][hi] = ((ib * 2 + p) * 64 + gp * 32 + (kl ^ X)) * 16 + (j >> 1) * 8;
      }
    }
  }
  auto ds_frag = [&](const char* tile, int tk) {
    typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
    const char* base = tile + (tk >> 1) * (8 * 64 * 8);
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base + soff[tk & 1][0]));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base + soff[tk & 1][1]));
    bf16x8 f;
    f[0] = lo[0]; f[1] = lo[1]; f[2] = lo[2]; f[3] = lo[3];
    f[4] = hi[0]; f[5] = hi[1]; f[6] = hi[2]; f[7] = hi[3];
    return f;
  };

  SwzColReads<D> kcd;
  kcd.init(lane);
  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = zero16();

  // Issue the copies of step t into buffer `buf`: the K tile (KCOPY instructions per wave) and, for each
  // stored quarter, one 1 KB instruction per wave. Returns the mask of the quarters copied (a quarter that
  // is not live, or outside the plan's span, which a plan belonging to the problem never gives, is skipped).
  const uint32_t s_lds0 = lds_addr(s_lds);
  auto fetch = [&](int t, int buf) {
    copy_tile_async<D, BC, 8>(k_lds[buf], kg, t * BC, N, wave, lane);
    const int idx = t - wbase;  // wave-uniform
    const uint64_t ws = (uint64_t)wslot;
    const long long slot0 = (long long)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(ws >> 32), idx) << 32) |
                                        (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)ws, idx));
    int m = 0;
#pragma unroll
    for (int x = 0; x < NQ; ++x) {
      if ((wl[x] >> idx) & 1) {
        const char* gsrc = a.ds + (slot0 + x) * DS_TILE_BYTES + (long long)(t & 1) * HALF;
        const uint32_t dst = s_lds0 + (uint32_t)((buf * NQ + x) * HALF) + (uint32_t)wv * 1024u;
        lds_copy16_nt(gsrc + wv * 1024, (uint32_t)lane * 16u, dst);
        m |= 1 << x;
      }
    }
    return m;
  };

  int t0 = next_live(0);
  int m0 = t0 < kt_end ? fetch(t0, 0) : 0;
  int t1 = t0 < kt_end ? next_live(t0 + 1) : kt_end;
  int m1 = t1 < kt_end ? fetch(t1, 1) : 0;
  int buf = 0;
  while (t0 < kt_end) {
    // step t0's copies have landed once at most step t1's are outstanding
    wait_vm_at_most(t1 < kt_end ? KCOPY + __builtin_popcount(m1) : 0);
    __syncthreads();  // every wave's copies of step t0 are in LDS; buffer (buf + 2) % 3 is free
    const int t2 = t1 < kt_end ? next_live(t1 + 1) : kt_end;
    const int nb = buf == 0 ? 2 : buf - 1;  // (buf + 2) % 3
    const int m2 = t2 < kt_end ? fetch(t2, nb) : 0;
    if ((m0 >> quarter) & 1) {
      const bf16* kt_lds = k_lds[buf];
      const char* st = s_lds[buf][quarter];
#pragma unroll
      for (int tk = 0; tk < 4; ++tk) {
        const bf16x8 sf = ds_frag(st, tk);
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[db] = M::mma(kcd.read(kt_lds, tk, db), sf, acc[db]);
      }
    }
    t0 = t1; m0 = m1;
    t1 = t2; m1 = m2;
    buf = buf == 2 ? 0 : buf + 1;
  }
  __builtin_amdgcn_s_waitcnt(0);

  // dq = scale * dQ^T, whole rows through LDS (the dS buffers, free once every wave is past its last step).
  static_assert(sizeof(s_lds) >= 8 * 32 * D * 2, "staging area of eight waves");
  __syncthreads();
  const int w0 = r0 + quarter * DS_QROWS + ib * 32;
  store_rows_staged<D>(&s_lds[0][0][0] + wave * (32 * D * 2), acc, a.scale, a.dq + (size_t)bh * N * D + (size_t)w0 * D,
                       N - w0, lane);
}

hipError_t launch_dq_stream(int d, const void* k, const void* ds, long long cap, const DsPlan& plan, void* dq,
                            const int* bounds, int B, int H, int Hm, int N, int causal, float scale,
                            hipStream_t stream) {
  DqsArgs a;
  a.k = static_cast<const bf16*>(k);
  a.ds = static_cast<const char*>(ds);
  a.dq = static_cast<bf16*>(dq);
  a.bounds = bounds;
  a.plan = plan;
  a.cap = cap;
  a.B = B; a.H = H; a.Hm = Hm; a.N = N;
  a.nkb = (N + KBLOCK - 1) / KBLOCK;
  a.causal = causal;
  a.scale = scale;
  const long grid = (long)((N + 255) / 256) * B * H;
  if (d == 64) {
    hipLaunchKernelGGL(dq_stream_kernel<64>, dim3((unsigned)grid), dim3(512), 0, stream, a);
  } else {
    hipLaunchKernelGGL(dq_stream_kernel<128>, dim3((unsigned)grid), dim3(512), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace fm
