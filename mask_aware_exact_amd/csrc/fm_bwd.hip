// Backward pass of exact attention under the column-wise mask (gfx950).
//
// The gradient of sum(out * dO) through softmax attention, recomputing P from q, k and the forward's
// lse, with tiles the mask covers completely skipped (FlashMask abstract, papers.pytorch.kr
// 2410.01359). Two kernels run in order on the caller's stream, and neither uses atomics:
//  1. bwd_dq: query-tile parallel, laid out like the forward (one query row per lane). Per live key
//     tile it forms S^T = K Q^T and dP^T = V dO^T, then P = exp(S - lse) (0 where masked) and
//     dS = P o (dP - D), and accumulates dQ^T += K^T dS^T with dS^T straight from registers. It also
//     forms D_i = sum_d dO_id out_id for its rows and stores it for kernel 2.
//  2. bwd_dkdv: key-tile parallel. Per live query tile it forms S, dP, P and dS with one key column
//     per lane and accumulates dV^T += dO^T P and dK^T += Q^T dS on chip for the whole query loop.
// Recomputing S and dP in kernel 1 costs 4 d FLOP per unmasked pair more than adding partial dQ tiles
// from kernel 2 with float atomics, whose traffic (one float32 dQ tile per live tile pair) was
// measured to cost more than that on MI355X.
#include "fm_common.h"

namespace fm {

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* out;
  const void* dout;
  const float* lse;
  float* dd;  // D_i, written by bwd_dq, read by bwd_dkdv
  void* dq;
  void* dk;
  void* dv;
  const int* lts;
  const int* lte;
  const int* uts;
  const int* ute;
  const int* bounds;
  int B, H, Hm;
  int Nq, Nk;  // query rows and keys per head
  int q_off;   // global index of query row 0: the mask and the causal rule see rows q_off + i
  int nkb;  // bounds entries per (b, hm) row
  const int* sched;  // longest-first unit order (query units at 0, key units at sched_nq) or null
  int sched_stride;  // int32 per (b, hm) row of sched
  int sched_nq;      // query units of 128 rows
  int causal;
  float scale;
  float scale_log2;
  // null, or [B, H, Nq] / [B, H, Nk]: row r of out (read) and dq (written) of (b, h) is row qmap[r]; key
  // row j of dk and dv (written) is row kmap[j]. Rows outside the range are not written and read as zero.
  const int* qmap;
  const int* kmap;
  // Stored-dS mode (ds_cache not null): heads whose region of the plan fits in ds_cap tiles get their dS
  // tiles written by the dK/dV pass and their dq formed from them afterwards; for those heads the dq pass
  // only forms D. Other heads run as without a cache.
  char* ds_cache;
  long long ds_cap;
  DsPlan ds;
};

// Whether head (b, h) with mask row mrow has its dS tiles stored.
__device__ __forceinline__ bool ds_stored(const BwdArgs& a, int bh, long long mrow) {
  return a.ds_cache != nullptr && ds_head_stored(a.ds, a.ds_cap, bh, mrow);
}

// ------------------------------------------------------------------ 1. dQ (and D), query-tile parallel

template <typename T, int D, int BC_ = 64>
struct DqTraits {
  static_assert(BC_ == 64 || (BC_ == 128 && sizeof(T) == 2 && D == 64), "128-key tiles: bf16 at d = 64 only");
  static constexpr int BR = 128;  // query rows per workgroup (4 waves x 32)
  static constexpr int BC = BC_;  // keys per tile (BC / 64 bounds entries)
  static constexpr int NKB = BC / 32;  // 32-key blocks per tile
  // workgroups per CU: three at d = 64 with 64-key tiles; two when the registers of the larger tiles need it
  static constexpr int OCC = (sizeof(T) == 2 && D == 64 && BC == 64) ? 3 : 2;
  static constexpr int NT = 256;
  static constexpr bool SWZ = sizeof(T) == 2;            // bf16 K and V tiles: swizzled, unpadded
  static constexpr int KP = SWZ ? D : D + 4;             // row pitch (elements)
  static constexpr int VP = KP;
  static constexpr int NQF = D / MM<T>::KW;
  static constexpr int NDB = D / 32;
  static constexpr int TPB = 16 / MM<T>::E;
  static constexpr int CPR = D * (int)sizeof(T) / 16;
  static constexpr int CH = BC * CPR / NT;
};

template <typename T, int D, int BC_>
__global__ __launch_bounds__(256, (DqTraits<T, D, BC_>::OCC)) void bwd_dq_kernel(BwdArgs a) {
  using Tr = DqTraits<T, D, BC_>;
  using M = MM<T>;
  constexpr int BR = Tr::BR, BC = Tr::BC, KP = Tr::KP, VP = Tr::VP, CPR = Tr::CPR, CH = Tr::CH;
  constexpr bool SWZ = Tr::SWZ;
  __shared__ __attribute__((aligned(16))) T k_lds[2][BC * KP];
  __shared__ __attribute__((aligned(16))) T v_lds[2][BC * VP];
  __shared__ __attribute__((aligned(16))) int vec_lds[2][4][BC];  // LTS, LTE, UTS, UTE of the tile's columns
  __shared__ __attribute__((aligned(16))) uint32_t cw_lds[4][BC];  // per wave: masked-row words of a tile

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int g = lane >> 5;
  const int l32 = lane & 31;

  const int BH = a.B * a.H;
  const int nq = (a.Nq + BR - 1) / BR;
  const int bh = blockIdx.x % BH;
  const int rank = (int)(blockIdx.x / BH);
  const int b = bh / a.H;
  const int h = bh % a.H;
  const int hm = a.Hm > 1 ? h : 0;
  // without a schedule the heaviest (latest) query tiles go first
  static_assert(BR == SCHED_UNIT, "query units of the schedule are dq tiles");
  const int qt = scheduled_unit(a.sched, a.sched_stride, (size_t)b * a.Hm + hm, 0, rank, nq, nq - 1 - rank);
  if (qt < 0) return;
  const int Nq = a.Nq, N = a.Nk;  // N: keys
  const int r0 = qt * BR;
  const int r1 = min(Nq, r0 + BR);
  const int row = r0 + wave * 32 + l32;  // this lane's query row
  const int g0 = a.q_off + r0, g1 = a.q_off + r1;  // the tile's rows in the mask's coordinates
  const int gend = a.q_off + Nq;

  const size_t qhead = (size_t)bh * Nq * D, khead = (size_t)bh * N * D;
  const T* __restrict__ qg = static_cast<const T*>(a.q) + qhead;
  const T* __restrict__ kg = static_cast<const T*>(a.k) + khead;
  const T* __restrict__ vg = static_cast<const T*>(a.v) + khead;
  const T* __restrict__ og = static_cast<const T*>(a.out) + qhead;
  const T* __restrict__ dog = static_cast<const T*>(a.dout) + qhead;
  const size_t vrow = ((size_t)b * a.Hm + hm) * N;
  const int* brow = a.bounds == nullptr ? nullptr : a.bounds + ((size_t)b * a.Hm + hm) * a.nkb * 8;
  const bool has_lt = a.lts != nullptr;
  const bool has_ut = a.uts != nullptr;
  const bool causal = a.causal != 0;
  const float sl2 = a.scale_log2;

  // A head whose dS tiles are stored gets its dq from them later: here it only needs D.
  const bool d_only = ds_stored(a, bh, (long long)b * a.Hm + hm);
  // Q^T and dO^T operands (k = d), O and lse for this lane's row (D_i is formed from them further down).
  typename M::frag qf[Tr::NQF], df[Tr::NQF], of[Tr::NQF];
  const int orow = (a.qmap != nullptr && row < Nq) ? a.qmap[(size_t)bh * Nq + row] : row;  // out / dq row
  const bool orow_ok = (unsigned)orow < (unsigned)Nq;
  const float lraw = (row < Nq && orow_ok) ? a.lse[(size_t)bh * Nq + row] : 0.f;
#pragma unroll
  for (int c = 0; c < Tr::NQF; ++c) {
    if (row < Nq) {
      const size_t e = (size_t)row * D + c * M::KW + g * M::E;
      qf[c] = d_only ? typename M::frag{} : load_kcontig_frag<T>(qg + e);
      df[c] = load_kcontig_frag<T>(dog + e);
      of[c] = orow_ok ? load_kcontig_frag<T>(og + (size_t)orow * D + c * M::KW + g * M::E) : typename M::frag{};
    } else {
      qf[c] = typename M::frag{};
      df[c] = typename M::frag{};
      of[c] = typename M::frag{};
    }
  }
  f32x16 acc[Tr::NDB];
#pragma unroll
  for (int db = 0; db < Tr::NDB; ++db) acc[db] = zero16();

  SwzRowReads<D> krd;
  SwzColReads<D> kcd;
  if constexpr (SWZ) {
    krd.init(lane);
    kcd.init(lane);
  }

  const int nkt = (N + BC - 1) / BC;
  const int kt_end = causal ? min(nkt, (g1 - 1) / BC + 1) : nkt;

  // Next tile: K / V and the tile's mask vectors. bf16: straight into LDS buffer `dst` by direct copies
  // (one vector per wave); float: into staging registers, stored by stash().
  constexpr int CHR = SWZ ? 1 : CH;
  i32x4 kr[CHR], vr[CHR];
  i32x4 mr = {0, 0, 0, 0};
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  auto fetch_vectors = [&](int kt, int dst) {
    copy_tile_vectors<BC>(vec_lds[dst], a.lts, a.lte, a.uts, a.ute, vrow, kt * BC, N, wv, lane);
  };
  auto fetch = [&](int kt, int dst) {
    const int c0 = kt * BC;
    if constexpr (SWZ) {
      copy_tile_async<D, BC, 4>(reinterpret_cast<bf16*>(k_lds[dst]), reinterpret_cast<const bf16*>(kg), c0, N, wave,
                                lane);
      copy_tile_async<D, BC, 4>(reinterpret_cast<bf16*>(v_lds[dst]), reinterpret_cast<const bf16*>(vg), c0, N, wave,
                                lane);
      fetch_vectors(kt, dst);
    } else {
#pragma unroll
      for (int it = 0; it < CH; ++it) {
        const int c = it * Tr::NT + tid;
        const int r = c / CPR, cc = c % CPR;
        const size_t rr = (size_t)min(c0 + r, N - 1);
        kr[it] = ld16(reinterpret_cast<const char*>(kg + rr * D) + cc * 16);
        vr[it] = ld16(reinterpret_cast<const char*>(vg + rr * D) + cc * 16);
      }
      if (tid < BC) {
        const int j = c0 + tid;
        mr = i32x4{0, 0, 0, 0};
        if (j < N) {
          if (has_lt) { mr[0] = a.lts[vrow + j]; mr[1] = a.lte[vrow + j]; }
          if (has_ut) { mr[2] = a.uts[vrow + j]; mr[3] = a.ute[vrow + j]; }
        }
      }
    }
  };
  auto stash = [&](int buf) {
    if constexpr (!SWZ) {
#pragma unroll
      for (int it = 0; it < CH; ++it) {
        const int c = it * Tr::NT + tid;
        const int r = c / CPR, cc = c % CPR;
        st16(reinterpret_cast<char*>(&k_lds[buf][r * KP]) + cc * 16, kr[it]);
        st16(reinterpret_cast<char*>(&v_lds[buf][r * VP]) + cc * 16, vr[it]);
      }
      if (tid < BC) {
#pragma unroll
        for (int e = 0; e < 4; ++e) vec_lds[buf][e][tid] = mr[e];
      }
    }
  };

  auto class_of = [&](int t) {
    constexpr int EPT = BC / KBLOCK;  // bounds entries per tile
    const TileBounds bt = merged_bounds(brow, t * EPT, min(a.nkb, t * EPT + EPT), N);
    return classify_tile(g0, g1, t * BC, min(N, t * BC + BC), bt, causal);
  };
  // The tile scan and the first tile's copies go out before D is formed, so that their round trips overlap
  // the Q / dO / O loads instead of following them (a D-only head has no tiles).
  TileWindow win = empty_window();
  int kt = kt_end;
  if (!d_only) {
    kt = next_live_tile(win, 0, kt_end, class_of, lane);
    if (kt < kt_end) fetch(kt, 0);
  }
  int buf = 0;

  float part = 0.f;
#pragma unroll
  for (int c = 0; c < Tr::NQF; ++c) {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int s = 0; s < 8; ++s) part += (float)df[c][s] * (float)of[c][s];
    } else {
      part += df[c] * of[c];
    }
  }
  const float Di = pair_sum(part);
  float lse2 = INFINITY;  // rows past N, without any unmasked key or dropped by qmap: exp(S - lse) = 0
  if (row < Nq) {
    if (orow_ok) lse2 = (lraw == -INFINITY) ? INFINITY : lraw * LOG2E;
    if (g == 0) a.dd[(size_t)bh * Nq + row] = Di;  // every row's D is written (0 for a dropped row)
  }
  // bf16 at d = 64: dP^T - D comes out of the products. One more product per 32-key block adds -D_i to
  // column i: the first operand is 1 at k = 0, 1, 2 for every key, the second holds -D_i split into three
  // bf16 parts at k = 0, 1, 2 (8 significant bits each: their sum is -D_i to float precision). Four
  // products per 128-key tile on constant registers in place of 64 subtractions per lane.
  constexpr bool FOLD_D = SWZ && D == 64;
  typename M::frag ones_f{}, negd_f{};
  if constexpr (FOLD_D) {
    if (g == 0) {
      const bf16 p0 = (bf16)(-Di);
      const float r1 = -Di - (float)p0;
      const bf16 p1 = (bf16)r1;
      const bf16 p2 = (bf16)(r1 - (float)p1);
      ones_f[0] = (bf16)1.f;
      ones_f[1] = (bf16)1.f;
      ones_f[2] = (bf16)1.f;
      negd_f[0] = p0;
      negd_f[1] = p1;
      negd_f[2] = p2;
    }
  }

  if (d_only) return;

  while (kt < kt_end) {
    const int c0 = kt * BC;
    const bool need_mask = window_partial(win, kt) || (c0 + BC > N);
    stash(buf);
    if constexpr (SWZ) __builtin_amdgcn_s_waitcnt(0);  // this tile's direct copies have landed
    __syncthreads();
    const int kt_next = next_live_tile(win, kt + 1, kt_end, class_of, lane);
    // bf16: the next tile's copies go out one at a time between the products below, so that they queue
    // while the matrix cores work instead of holding up the products. Without a next tile the current
    // one is copied into the other buffer, which is never read, so the sequence is the same.
    TileCopy<D, BC, 4> kcp, vcp;
    if constexpr (SWZ) {
      const int cn = (kt_next < kt_end ? kt_next : kt) * BC;
      kcp.prep(reinterpret_cast<bf16*>(k_lds[buf ^ 1]), reinterpret_cast<const bf16*>(kg), cn, N, wave, lane);
      vcp.prep(reinterpret_cast<bf16*>(v_lds[buf ^ 1]), reinterpret_cast<const bf16*>(vg), cn, N, wave, lane);
      if (kt_next < kt_end) fetch_vectors(kt_next, buf ^ 1);
    } else {
      if (kt_next < kt_end) fetch(kt_next, buf ^ 1);
    }

    const T* kt_lds = k_lds[buf];
    const T* vt_lds = v_lds[buf];
    // S^T = K Q^T and dP^T = V dO^T for the 32-key blocks of the tile (rows = keys, columns = queries).
    // Product blocks run at raised wave priority, so the two waves of a SIMD drift into opposite phases.
    __builtin_amdgcn_s_setprio(2);
    f32x16 s[Tr::NKB], dp[Tr::NKB];
#pragma unroll
    for (int jb = 0; jb < Tr::NKB; ++jb) {
      s[jb] = zero16();
      dp[jb] = zero16();
#pragma unroll
      for (int c = 0; c < Tr::NQF; ++c) {
        if constexpr (SWZ) {
          constexpr int NC = 2 * TileCopy<D, BC, 4>::NK;  // copies, one after every other product pair
          static_assert(NC == Tr::NKB * Tr::NQF / 2, "one copy per two product pairs");
          s[jb] = M::mma(krd.read(kt_lds, jb, c), qf[c], s[jb]);
          dp[jb] = M::mma(krd.read(vt_lds, jb, c), df[c], dp[jb]);
          if constexpr (FOLD_D) {
            if (c == Tr::NQF - 1) dp[jb] = M::mma(ones_f, negd_f, dp[jb]);
          }
          if (c & 1) {
            const int k = (jb * Tr::NQF + c) >> 1;
            if (k < NC / 2) kcp.issue(k); else vcp.issue(k - NC / 2);
          }
        } else {
          s[jb] = M::mma(load_kcontig_frag<T>(kt_lds + (jb * 32 + l32) * KP + g * M::E + c * M::KW), qf[c], s[jb]);
          dp[jb] = M::mma(load_kcontig_frag<T>(vt_lds + (jb * 32 + l32) * VP + g * M::E + c * M::KW), df[c], dp[jb]);
        }
      }
    }
    interleave_reads<2 * Tr::NKB * Tr::NQF + (FOLD_D ? Tr::NKB : 0), 2 * Tr::NKB * Tr::NQF, 2>();
    __builtin_amdgcn_s_setprio(0);
    // dS^T = P^T o (dP^T - D), P^T = exp(S^T - lse) with masked entries 0 (masked scores set to -inf).
    if (need_mask) {
      tile_column_words<BC>(cw_lds[wave], &vec_lds[buf][0][0], g0 + wave * 32, c0, gend, N, causal, has_lt, has_ut,
                            lane);
#pragma unroll
      for (int jb = 0; jb < Tr::NKB; ++jb) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const i32x4 w4 = column_words4(cw_lds[wave], jb, q4, g);
#pragma unroll
          for (int e = 0; e < 4; ++e) s[jb][4 * q4 + e] = select_neg_inf(row_mask_of(w4[e], l32), s[jb][4 * q4 + e]);
        }
      }
    }
#pragma unroll
    for (int jb = 0; jb < Tr::NKB; ++jb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(s[jb][r] * sl2 - lse2);
        dp[jb][r] = FOLD_D ? p * dp[jb][r] : p * (dp[jb][r] - Di);
      }
    }
    // dQ^T += K^T dS^T over the keys of the tile.
    __builtin_amdgcn_s_setprio(2);
#pragma unroll
    for (int t = 0; t < Tr::NKB * Tr::TPB; ++t) {
      const typename M::frag sf = acc_frag<T>(dp[t / Tr::TPB], t % Tr::TPB);
#pragma unroll
      for (int db = 0; db < Tr::NDB; ++db) {
        if constexpr (SWZ) {
          acc[db] = M::mma(kcd.read(kt_lds, t, db), sf, acc[db]);
        } else {
          acc[db] = M::mma(load_kmajor_frag<T>(kt_lds, KP, 0, db * 32, t, lane), sf, acc[db]);
        }
      }
    }
    interleave_reads<Tr::NKB * Tr::TPB * Tr::NDB, 2 * Tr::NKB * Tr::TPB * Tr::NDB, 4>();
    __builtin_amdgcn_s_setprio(0);
    kt = kt_next;
    buf ^= 1;
  }

  if constexpr (SWZ) __builtin_amdgcn_s_waitcnt(0);  // the last tile's copies (never read) have landed
  if constexpr (SWZ && (D == 128 || BC == 128)) {
    if (a.qmap == nullptr) {
      // Unmapped bf16 dq: whole rows through LDS (the K tile buffers, free once every wave is here). Not with
      // 64-key tiles at d = 64, where the staging code's registers make the kernel spill (three waves per SIMD).
      static_assert(sizeof(k_lds) >= 4 * 32 * D * 2, "staging area of four waves");
      __syncthreads();
      const int w0 = r0 + wave * 32;
      store_rows_staged<D>(reinterpret_cast<char*>(&k_lds[0][0]) + wave * (32 * D * 2), acc, a.scale,
                           static_cast<bf16*>(a.dq) + qhead + (size_t)w0 * D, Nq - w0, lane);
      return;
    }
  }
  // dq = scale * dQ^T for this lane's row.
  if (row < Nq && orow_ok) {
    T* dqg = static_cast<T*>(a.dq) + qhead + (size_t)orow * D;
#pragma unroll
    for (int db = 0; db < Tr::NDB; ++db) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = db * 32 + 8 * q4 + 4 * g;
        if constexpr (sizeof(T) == 2) {
          bf16x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = (bf16)(acc[db][4 * q4 + e] * a.scale);
          *reinterpret_cast<bf16x4*>(dqg + d0) = w;
        } else {
          f32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = acc[db][4 * q4 + e] * a.scale;
          *reinterpret_cast<f32x4*>(dqg + d0) = w;
        }
      }
    }
  }
}

// ------------------------------------------------------------------ 2a. dK / dV, bf16, wave pairs

// Eight waves per 128-key tile: waves w and w + 4 share the 32 keys of group w % 4 (one key column per
// lane) and split the work so that each stays under 256 registers (two waves per SIMD):
//   role 0 (w < 4) holds K, forms S = Q K^T and P, passes P to its partner through LDS and accumulates
//     all of dV += P^T dO;
//   role 1 (w >= 4) holds V, forms dP = dO V^T and dS = P o (dP - D) and accumulates all of dK += dS^T Q.
// Two barriers per query tile t. Phase 1: role 0 forms S_t and P_t (exponentials) while role 1 issues
// dP_t and the dK products of tile t - 1, whose dS it kept in registers. Phase 2: role 0 issues the dV
// products of tile t while role 1 forms dS_t. So one wave of a SIMD runs vector arithmetic while the
// other issues matrix products. Q is kept for three tiles (t - 1, t and the prefetched t + 1).
template <int D, int BR_>
struct PairTraits {
  static constexpr int BC = 128;          // keys per workgroup
  static constexpr int BR = BR_;          // query rows per iteration (a pair of barriers)
  static constexpr int NIB = BR / 32;     // 32-row blocks per query tile
  static constexpr int NT = 512;
  static constexpr int NKF = D / 16;      // K or V fragments per lane (k = d)
  static constexpr int NDB = D / 32;      // 32-wide d blocks
};

template <int D, int BR_>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_pair_kernel(BwdArgs a) {
  using Tr = PairTraits<D, BR_>;
  static_assert(BR_ == 64 || BR_ == 128, "query tiles of 64 or 128 rows");
  // At d = 64 role 1 forms dP - D in its products (accumulators started at -D, which the D staging
  // stores negated) instead of subtracting afterwards: the BERT-like backward 3-4% faster. Both d = 64
  // tile heights do it, so that fm_bwd and fm_bwd_ds keep identical dK and dV. At d = 128 the loads ahead
  // of the products cost more than the subtractions (+1 to +2%).
  constexpr bool FOLD_D = D == 64;
  using M = MM<bf16>;
  constexpr int BC = Tr::BC, BR = Tr::BR;
  constexpr int TILE = BR * D;
  // Swizzled, unpadded Q (ring of three) and dO (two) tiles, filled by direct global-to-LDS copies.
  __shared__ __attribute__((aligned(16))) bf16 q_lds[3 * TILE];
  __shared__ __attribute__((aligned(16))) bf16 do_lds[2 * TILE];
  // P passes from role 0 to role 1 in register order, lane-interleaved: chunk k (4 values) of lane l sits
  // at [group][k][l], so every 8-byte access of a wave is 512 contiguous bytes.
  __shared__ __attribute__((aligned(16))) bf16x4 p_xch[4][Tr::NIB * 4][64];
  __shared__ __attribute__((aligned(16))) float lse_lds[2][BR];
  __shared__ __attribute__((aligned(16))) float dd_lds[2][BR];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int g = lane >> 5;
  const int l32 = lane & 31;
  const int kgrp = wave & 3;
  const int role = wave >> 2;

  const int BH = a.B * a.H;
  const int bh = blockIdx.x % BH;
  const int rank = (int)(blockIdx.x / BH);
  const int b = bh / a.H;
  const int h = bh % a.H;
  const int hm = a.Hm > 1 ? h : 0;
  // without a schedule early key tiles, which carry the most causal work, go first
  static_assert(BC == SCHED_UNIT, "key units of the schedule are dk/dv tiles");
  const int kt = scheduled_unit(a.sched, a.sched_stride, (size_t)b * a.Hm + hm, a.sched_nq, rank,
                                (a.Nk + BC - 1) / BC, rank);
  if (kt < 0) return;
  const int N = a.Nk, Nq = a.Nq, qoff = a.q_off;  // N: keys
  const int c0 = kt * BC;
  const int c1 = min(N, c0 + BC);
  const int jl = kgrp * 32 + l32;  // this lane's key column inside the tile
  const int j = c0 + jl;

  const size_t qhead = (size_t)bh * Nq * D, khead = (size_t)bh * N * D;
  const bf16* __restrict__ qg = static_cast<const bf16*>(a.q) + qhead;
  const bf16* __restrict__ kg = static_cast<const bf16*>(a.k) + khead;
  const bf16* __restrict__ vg = static_cast<const bf16*>(a.v) + khead;
  const bf16* __restrict__ dog = static_cast<const bf16*>(a.dout) + qhead;
  const float* __restrict__ lseg = a.lse + (size_t)bh * Nq;
  const float* __restrict__ ddg = a.dd + (size_t)bh * Nq;
  const size_t vrow = ((size_t)b * a.Hm + hm) * N;
  const int* brow = a.bounds == nullptr ? nullptr : a.bounds + ((size_t)b * a.Hm + hm) * a.nkb * 8;
  const bool has_lt = a.lts != nullptr;
  const bool has_ut = a.uts != nullptr;
  const bool causal = a.causal != 0;
  const float sl2 = a.scale_log2;

  // This lane's key column: mask values (role 0) and K (role 0) or V (role 1) fragments with k = d.
  int m_lts = 0, m_lte = 0, m_uts = 0, m_ute = 0;
  bf16x8 xf[Tr::NKF];
  {
    const bf16* src = role == 0 ? kg : vg;
    if (j < N) {
      if (has_lt) { m_lts = a.lts[vrow + j]; m_lte = a.lte[vrow + j]; }
      if (has_ut) { m_uts = a.uts[vrow + j]; m_ute = a.ute[vrow + j]; }
#pragma unroll
      for (int c = 0; c < Tr::NKF; ++c) xf[c] = load_kcontig_frag<bf16>(src + (size_t)j * D + c * 16 + g * 8);
    } else {
#pragma unroll
      for (int c = 0; c < Tr::NKF; ++c) xf[c] = bf16x8{};
    }
  }
  SwzRowReads<D> rrd;
  SwzColReads<D> crd;
  rrd.init(lane);
  crd.init(lane);

  // Stored-dS mode: role 1 writes each dS tile it forms (64 query rows x the workgroup's 128 keys) to slot
  // ds_slot0 + (qt - ds_first) of the cache with four 16-byte stores per lane, each covering 1 KB
  // contiguous: store (ib, p) of lane (g, l32) holds rows 32 ib + 16 p + 4 g + (0..3) and then
  // 32 ib + 16 p + 8 + 4 g + (0..3) of its key, at position g * 32 + (l32 ^ (8 g + 4 p)).
  static_assert(BC == DS_KEYS, "stored dS tiles are the dK/dV pass's tiles");
  // (stored dS tiles are 64 query rows: a launch with 128-row query tiles never has a cache)
  const bool ds_on = BR == DS_QROWS && role == 1 && ds_stored(a, bh, (long long)b * a.Hm + hm);
  long long ds_slot0 = 0, ds_span = 0;  // tile qt goes to slot ds_slot0 + (qt - ds_first) when inside the span
  int ds_first = 0;
  int ds_off[2];
  if (ds_on) {
    const long long mrow = (long long)b * a.Hm + hm;
    long long lo;
    ds_span = ds_tile_span(a.ds, mrow, kt, lo);
    ds_first = a.ds.first[mrow * a.ds.nkt + kt];
    ds_slot0 = a.ds.region[bh] + lo;
  }
#pragma unroll
  for (int p = 0; p < 2; ++p) ds_off[p] = kgrp * 4096 + (g * 32 + (l32 ^ (8 * g + 4 * p))) * 16;

  // dV^T (role 0) or dK^T (role 1) for this lane's key column, all of d.
  f32x16 acc[Tr::NDB];
#pragma unroll
  for (int db = 0; db < Tr::NDB; ++db) acc[db] = zero16();

  const TileBounds bnd = merged_bounds(brow, kt * (BC / KBLOCK), min(a.nkb, (kt + 1) * (BC / KBLOCK)), N);
  const int nq = (Nq + BR - 1) / BR;
  const int qt_begin = causal ? max(0, c0 - qoff) / BR : 0;
  auto class_of = [&](int qt) {
    return classify_tile(qoff + qt * BR, qoff + min(Nq, qt * BR + BR), c0, c1, bnd, causal);
  };

  // Next query tile: Q and dO straight into their ring slots (direct global-to-LDS copies; rows past N
  // read row N - 1, which gets lse = +inf below and so contributes nothing), lse and D into registers.
  float lr = 0.f, ddr = 0.f;
  int l_row = 0;
  int lmap = 0;  // the row's qmap entry: a row whose entry is out of range is dropped (contributes nothing)
  auto fetch_rows = [&](int qt) {
    if (tid < BR) {
      l_row = qt * BR + tid;
      const int i = min(l_row, Nq - 1);
      lr = lseg[i];
      ddr = ddg[i];
      if (a.qmap != nullptr) lmap = a.qmap[(size_t)bh * Nq + i];
    }
  };
  auto fetch = [&](int qt, int qslot, int dslot) {
    const int q0 = qt * BR;
    fetch_rows(qt);
    copy_tile_async<D, BR, 8>(q_lds + qslot * TILE, qg, q0, Nq, wave, lane);
    copy_tile_async<D, BR, 8>(do_lds + dslot * TILE, dog, q0, Nq, wave, lane);
  };
  auto stash = [&](int ds) {
    if (tid < BR) {
      // rows past N, rows without any unmasked key (lse = -inf) and dropped rows get +inf: exp(S - lse) = 0
      const bool ldrop = a.qmap != nullptr && (unsigned)lmap >= (unsigned)Nq;
      const float l = (l_row >= Nq || lr == -INFINITY || ldrop) ? INFINITY : lr;
      lse_lds[ds][tid] = l * LOG2E;
      dd_lds[ds][tid] = FOLD_D ? -ddr : ddr;
    }
  };

  // dK^T += Q^T dS for one query tile, dS in register order (role 1). With STORE, the tile's dS also goes
  // to `st` (stored-dS mode), its 4 stores placed after products 1, 3, 5 and 7, so that they leave while
  // the matrix cores work instead of holding up the end of the tile.
  auto dk_products = [&](auto store_tag, const bf16x4 (&sv)[Tr::NIB][4], const bf16* qb, char* st) {
    constexpr bool STORE = decltype(store_tag)::value;
    constexpr int NM = 2 * Tr::NIB * Tr::NDB;  // products
    static_assert(NM >= 8, "a store after every other product");
#pragma unroll
    for (int t = 0; t < 2 * Tr::NIB; ++t) {
      bf16x8 sf;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sf[e] = sv[t >> 1][2 * (t & 1)][e];
        sf[4 + e] = sv[t >> 1][2 * (t & 1) + 1][e];
      }
#pragma unroll
      for (int db = 0; db < Tr::NDB; ++db) {
        acc[db] = M::mma(crd.read(qb, t, db), sf, acc[db]);
        if constexpr (STORE) {
          const int m = t * Tr::NDB + db;
          if ((m & 1) && m < 8) {
            const int ib = m >> 2, p = (m >> 1) & 1;  // store k = (m - 1) / 2 = 2 ib + p
            bf16x8 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              w[e] = sv[ib][2 * p][e];
              w[4 + e] = sv[ib][2 * p + 1][e];
            }
            // non-temporal: the tile is read back once, by the dq pass, and should not evict Q / dO tiles
            i32x4 wi;
            __builtin_memcpy(&wi, &w, 16);
            __builtin_nontemporal_store(wi, reinterpret_cast<i32x4*>(st + (2 * ib + p) * 1024 + ds_off[p]));
          }
        }
      }
    }
    if constexpr (STORE) {
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, (2 * NM - 4 + NM - 1) / NM, 0);
        if ((m & 1) && m < 8) __builtin_amdgcn_sched_group_barrier(0x040, 1, 0);
      }
    } else {
      interleave_reads<NM, 2 * NM, 4>();
    }
  };


  TileWindow win = empty_window();
  int qt = next_live_tile(win, qt_begin, nq, class_of, lane);
  if (qt < nq) fetch(qt, 0, 0);
  int qs = 0, ds = 0;     // ring slots of the current tile's Q and dO (and lse / D)
  int qs_prev = -1;       // role 1: slot of the previous tile's Q, whose dS is still pending
  bf16x4 sv[Tr::NIB][4];  // role 1: that dS, register order
  char* st_prev = nullptr;  // role 1: that dS's destination in the cache (stored-dS mode), or null
  // dK products of the previous tile, storing its dS on the way when it has a destination
  auto dk_pass = [&](const bf16* qb) {
    if (st_prev != nullptr) {
      dk_products(Flag<true>{}, sv, qb, st_prev);
    } else {
      dk_products(Flag<false>{}, sv, qb, nullptr);
    }
  };

  // Every load issued so far (K or V fragments, mask values, bounds, plan entries, the first tile) is
  // first used inside the loop. Left pending at the loop's entry, the compiler's wait-count analysis
  // carries them into every iteration as in-loop vmcnt waits, which also catch the untracked tile copies
  // issued between the products and stall each tile on their latency.
  __builtin_amdgcn_s_waitcnt(0);
  while (qt < nq) {
    const int q0 = qt * BR;
    const bool need_mask = window_partial(win, qt) || (q0 + BR > Nq) || (c0 + BC > N);
    stash(ds);
    __builtin_amdgcn_s_waitcnt(0);  // this tile's direct copies have landed
    __syncthreads();  // (A) the tile is in LDS; every wave is past the previous tile's work
    const int qt_next = next_live_tile(win, qt + 1, nq, class_of, lane);
    // The next tile's Q and dO copies go out one at a time between the score (role 0) or dP (role 1)
    // products below, so that they queue while the matrix cores work. Without a next tile the current
    // one is copied into the free slots, which are never read, so the sequence is the same.
    TileCopy<D, BR, 8> cp;
    const int qn = (qt_next < nq ? qt_next : qt) * BR;
    cp.prep(q_lds + (qs == 2 ? 0 : qs + 1) * TILE, qg, qn, Nq, wave, lane);
    const uint32_t dlds0 = lds_addr(do_lds + (ds ^ 1) * TILE) + (uint32_t)__builtin_amdgcn_readfirstlane(wave) * 1024u;
    const char* dgb = reinterpret_cast<const char*>(dog + (size_t)qn * D);
    constexpr int NCP = 2 * TileCopy<D, BR, 8>::NK;  // copies per wave
    constexpr int NMP = Tr::NIB * Tr::NKF;           // products in the block that carries them
    static_assert(NMP % NCP == 0, "copies must spread evenly over the products");
    auto copy_after = [&](int m) {  // after product m (compile-time after unrolling)
      if ((m + 1) % (NMP / NCP) == 0) {
        const int k = (m + 1) / (NMP / NCP) - 1;
        if (k < NCP / 2) cp.issue(k); else cp.issue_to(dgb, dlds0, k - NCP / 2);
      }
    };
    if (qt_next < nq) fetch_rows(qt_next);

    const bf16* qb = q_lds + qs * TILE;
    const bf16* dob = do_lds + ds * TILE;

    // Phase 1. Role 0: S (rows = query rows, columns = this lane's keys) and P, written to LDS.
    // Role 1: dP, then the dK products of the previous tile.
    bf16x4 pv[Tr::NIB][4];  // P, register order
    f32x16 x[Tr::NIB];
    if (role == 0) {
      __builtin_amdgcn_s_setprio(3);
#pragma unroll
      for (int ib = 0; ib < Tr::NIB; ++ib) {
        x[ib] = zero16();
#pragma unroll
        for (int c = 0; c < Tr::NKF; ++c) {
          x[ib] = M::mma(rrd.read(qb, ib, c), xf[c], x[ib]);
          copy_after(ib * Tr::NKF + c);
        }
      }
      interleave_reads<Tr::NIB * Tr::NKF, Tr::NIB * Tr::NKF, 2>();
      __builtin_amdgcn_s_setprio(0);
      if (need_mask) {
#pragma unroll
        for (int ib = 0; ib < Tr::NIB; ++ib) {
          // masked-row bits of this lane's key column for the 64 rows holding block ib (two blocks per call)
          const uint64_t mbits = masked_row_bits(qoff + q0 + 64 * (ib >> 1), j, qoff + Nq, N, causal, has_lt,
                                                 has_ut, m_lts, m_lte, m_uts, m_ute);
          const uint32_t mw = (uint32_t)(mbits >> (32 * (ib & 1) + 4 * g));
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4 lse4 = *reinterpret_cast<const f32x4*>(&lse_lds[ds][ib * 32 + 8 * q4 + 4 * g]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float xm = select_neg_inf(row_mask_of((int)mw, 8 * q4 + e), x[ib][4 * q4 + e]);
              pv[ib][q4][e] = (bf16)__builtin_amdgcn_exp2f(xm * sl2 - lse4[e]);
            }
            p_xch[kgrp][4 * ib + q4][lane] = pv[ib][q4];
          }
        }
      } else {
#pragma unroll
        for (int ib = 0; ib < Tr::NIB; ++ib) {
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4 lse4 = *reinterpret_cast<const f32x4*>(&lse_lds[ds][ib * 32 + 8 * q4 + 4 * g]);
#pragma unroll
            for (int e = 0; e < 4; ++e) pv[ib][q4][e] = (bf16)__builtin_amdgcn_exp2f(x[ib][4 * q4 + e] * sl2 - lse4[e]);
            p_xch[kgrp][4 * ib + q4][lane] = pv[ib][q4];
          }
        }
      }
    } else {
      // above the default priority of the other roles' arithmetic, below role 0's products
      __builtin_amdgcn_s_setprio(1);
      if (qs_prev >= 0) dk_pass(q_lds + qs_prev * TILE);
#pragma unroll
      for (int ib = 0; ib < Tr::NIB; ++ib) {
        if constexpr (FOLD_D) {
          // dP - D in one pass: the accumulators start at -D of their rows
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4 nd4 = *reinterpret_cast<const f32x4*>(&dd_lds[ds][ib * 32 + 8 * q4 + 4 * g]);
#pragma unroll
            for (int e = 0; e < 4; ++e) x[ib][4 * q4 + e] = nd4[e];
          }
        } else {
          x[ib] = zero16();
        }
#pragma unroll
        for (int c = 0; c < Tr::NKF; ++c) {
          x[ib] = M::mma(rrd.read(dob, ib, c), xf[c], x[ib]);
          copy_after(ib * Tr::NKF + c);
        }
      }
      interleave_reads<Tr::NIB * Tr::NKF, Tr::NIB * Tr::NKF, 2>();
      __builtin_amdgcn_s_setprio(0);
    }
    __syncthreads();  // (B) P is in LDS

    // Phase 2. Role 0: dV^T += dO^T P. Role 1: reads P back and forms dS, kept for the next tile.
    if (role == 0) {
      __builtin_amdgcn_s_setprio(3);
#pragma unroll
      for (int t = 0; t < 2 * Tr::NIB; ++t) {
        bf16x8 pf;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pf[e] = pv[t >> 1][2 * (t & 1)][e];
          pf[4 + e] = pv[t >> 1][2 * (t & 1) + 1][e];
        }
#pragma unroll
        for (int db = 0; db < Tr::NDB; ++db) acc[db] = M::mma(crd.read(dob, t, db), pf, acc[db]);
      }
      interleave_reads<2 * Tr::NIB * Tr::NDB, 4 * Tr::NIB * Tr::NDB, 4>();
      __builtin_amdgcn_s_setprio(0);
    } else {
#pragma unroll
      for (int ib = 0; ib < Tr::NIB; ++ib) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const bf16x4 p4 = p_xch[kgrp][4 * ib + q4][lane];
          if constexpr (FOLD_D) {
#pragma unroll
            for (int e = 0; e < 4; ++e) sv[ib][q4][e] = (bf16)((float)p4[e] * x[ib][4 * q4 + e]);
          } else {
            const f32x4 dd4 = *reinterpret_cast<const f32x4*>(&dd_lds[ds][ib * 32 + 8 * q4 + 4 * g]);
#pragma unroll
            for (int e = 0; e < 4; ++e) sv[ib][q4][e] = (bf16)((float)p4[e] * (x[ib][4 * q4 + e] - dd4[e]));
          }
        }
      }
      st_prev = (ds_on && qt >= ds_first && (long long)(qt - ds_first) < ds_span)
                    ? a.ds_cache + (ds_slot0 + (qt - ds_first)) * DS_TILE_BYTES
                    : nullptr;
      qs_prev = qs;
    }
    qt = qt_next;
    qs = qs == 2 ? 0 : qs + 1;
    ds ^= 1;
  }
  __builtin_amdgcn_s_waitcnt(0);  // the last tile's copies (never read) have landed
  // Role 1: the dK products of the last tile (its Q is still in LDS: nothing has been stored since).
  if (role == 1 && qs_prev >= 0) dk_pass(q_lds + qs_prev * TILE);

  // dV = dV^T (role 0) or dK = scale * dK^T (role 1) for this lane's key column, all of d.
  if (a.kmap == nullptr) {
    // Unmapped: whole rows through LDS, role 0 staging in the dO tiles and role 1 in the Q ring, both free
    // once role 1's last dK products are done and every wave's copies have landed.
    static_assert(sizeof(do_lds) >= 4 * 32 * D * 2 && sizeof(q_lds) >= 4 * 32 * D * 2, "staging areas");
    __syncthreads();
    char* stage = reinterpret_cast<char*>(role == 0 ? do_lds : q_lds) + kgrp * (32 * D * 2);
    const int k0 = c0 + kgrp * 32;
    store_rows_staged<D>(stage, acc, role == 0 ? 1.f : a.scale,
                         static_cast<bf16*>(role == 0 ? a.dv : a.dk) + khead + (size_t)k0 * D, N - k0, lane);
    return;
  }
  const int jo = (a.kmap != nullptr && j < N) ? a.kmap[(size_t)bh * N + j] : j;  // the row written
  if (j < N && (unsigned)jo < (unsigned)N) {
    bf16* dst = static_cast<bf16*>(role == 0 ? a.dv : a.dk) + khead + (size_t)jo * D;
    const float mul = role == 0 ? 1.f : a.scale;
#pragma unroll
    for (int db = 0; db < Tr::NDB; ++db) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (bf16)(acc[db][4 * q4 + e] * mul);
        *reinterpret_cast<bf16x4*>(dst + db * 32 + 8 * q4 + 4 * g) = w;
      }
    }
  }
}

// ------------------------------------------------------------------ 2b. dK / dV, float32

// float32 variant (used by the float32 workload): four waves, wave w owns keys 32 w .. 32 w + 31 and
// forms S, dP, P, dS and both dK and dV for them; padded row-major tiles, one query tile at a time.
template <int D>
struct F32Traits {
  static constexpr int BC = 128;
  static constexpr int BR = 32;
  static constexpr int NT = 256;
  static constexpr int PITCH = D + 4;
  static constexpr int NKF = D / 2;
  static constexpr int NDB = D / 32;
};

template <int D>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_f32_kernel(BwdArgs a) {
  using Tr = F32Traits<D>;
  using M = MM<float>;
  constexpr int BC = Tr::BC, BR = Tr::BR, PITCH = Tr::PITCH;
  __shared__ __attribute__((aligned(16))) float q_lds[BR * PITCH];
  __shared__ __attribute__((aligned(16))) float do_lds[BR * PITCH];
  __shared__ __attribute__((aligned(16))) float lse_lds[BR];
  __shared__ __attribute__((aligned(16))) float dd_lds[BR];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int g = lane >> 5;
  const int l32 = lane & 31;

  const int BH = a.B * a.H;
  const int bh = blockIdx.x % BH;
  const int rank = (int)(blockIdx.x / BH);
  const int b = bh / a.H;
  const int h = bh % a.H;
  const int hm = a.Hm > 1 ? h : 0;
  // without a schedule early key tiles, which carry the most causal work, go first
  static_assert(BC == SCHED_UNIT, "key units of the schedule are dk/dv tiles");
  const int kt = scheduled_unit(a.sched, a.sched_stride, (size_t)b * a.Hm + hm, a.sched_nq, rank,
                                (a.Nk + BC - 1) / BC, rank);
  if (kt < 0) return;
  const int N = a.Nk, Nq = a.Nq, qoff = a.q_off;  // N: keys
  const int c0 = kt * BC;
  const int c1 = min(N, c0 + BC);
  const int j = c0 + wave * 32 + l32;

  const size_t qhead = (size_t)bh * Nq * D, khead = (size_t)bh * N * D;
  const float* __restrict__ qg = static_cast<const float*>(a.q) + qhead;
  const float* __restrict__ kg = static_cast<const float*>(a.k) + khead;
  const float* __restrict__ vg = static_cast<const float*>(a.v) + khead;
  const float* __restrict__ dog = static_cast<const float*>(a.dout) + qhead;
  const size_t vrow = ((size_t)b * a.Hm + hm) * N;
  const int* brow = a.bounds == nullptr ? nullptr : a.bounds + ((size_t)b * a.Hm + hm) * a.nkb * 8;
  const bool has_lt = a.lts != nullptr;
  const bool has_ut = a.uts != nullptr;
  const bool causal = a.causal != 0;

  int m_lts = 0, m_lte = 0, m_uts = 0, m_ute = 0;
  float kf[Tr::NKF], vf[Tr::NKF];
#pragma unroll
  for (int c = 0; c < Tr::NKF; ++c) {
    kf[c] = j < N ? kg[(size_t)j * D + 2 * c + g] : 0.f;
    vf[c] = j < N ? vg[(size_t)j * D + 2 * c + g] : 0.f;
  }
  if (j < N) {
    if (has_lt) { m_lts = a.lts[vrow + j]; m_lte = a.lte[vrow + j]; }
    if (has_ut) { m_uts = a.uts[vrow + j]; m_ute = a.ute[vrow + j]; }
  }

  f32x16 dk[Tr::NDB], dv[Tr::NDB];
#pragma unroll
  for (int db = 0; db < Tr::NDB; ++db) {
    dk[db] = zero16();
    dv[db] = zero16();
  }
  const TileBounds bnd = merged_bounds(brow, kt * (BC / KBLOCK), min(a.nkb, (kt + 1) * (BC / KBLOCK)), N);
  const int nq = (Nq + BR - 1) / BR;
  for (int qt = causal ? max(0, c0 - qoff) / BR : 0; qt < nq; ++qt) {
    const int q0 = qt * BR;
    const int q1 = min(Nq, q0 + BR);
    const int cls = classify_tile(qoff + q0, qoff + q1, c0, c1, bnd, causal);
    if (cls == CLS_FULL) continue;
    const bool need_mask = (cls == CLS_PARTIAL) || (q1 - q0 < BR) || (c1 - c0 < BC);
    __syncthreads();
    load_tile<float, BR, D, PITCH, Tr::NT>(q_lds, qg, q0, Nq, tid);
    load_tile<float, BR, D, PITCH, Tr::NT>(do_lds, dog, q0, Nq, tid);
    if (tid < BR) {
      const int i = q0 + tid;
      const bool drop = i < Nq && a.qmap != nullptr && (unsigned)a.qmap[(size_t)bh * Nq + i] >= (unsigned)Nq;
      const float l = (i < Nq && !drop) ? a.lse[(size_t)bh * Nq + i] : INFINITY;
      lse_lds[tid] = ((l == -INFINITY) ? INFINITY : l) * LOG2E;
      dd_lds[tid] = i < Nq ? a.dd[(size_t)bh * Nq + i] : 0.f;
    }
    __syncthreads();
    f32x16 s = zero16(), dp = zero16();
#pragma unroll
    for (int c = 0; c < Tr::NKF; ++c) {
      s = M::mma(q_lds[l32 * PITCH + 2 * c + g], kf[c], s);
      dp = M::mma(do_lds[l32 * PITCH + 2 * c + g], vf[c], dp);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int il = 8 * (r >> 2) + 4 * g + (r & 3);
      const int i = q0 + il;
      float p = __builtin_amdgcn_exp2f(s[r] * a.scale_log2 - lse_lds[il]);
      const bool msk = need_mask & ((i >= Nq) | (j >= N) |
                                    masked_elem(qoff + i, j, causal, has_lt, has_ut, m_lts, m_lte, m_uts, m_ute));
      p = msk ? 0.f : p;
      s[r] = p;
      dp[r] = p * (dp[r] - dd_lds[il]);
    }
#pragma unroll
    for (int t = 0; t < 16; ++t) {
#pragma unroll
      for (int db = 0; db < Tr::NDB; ++db) {
        dv[db] = M::mma(load_kmajor_frag<float>(do_lds, PITCH, 0, db * 32, t, lane), s[t], dv[db]);
        dk[db] = M::mma(load_kmajor_frag<float>(q_lds, PITCH, 0, db * 32, t, lane), dp[t], dk[db]);
      }
    }
  }
  const int jo = (a.kmap != nullptr && j < N) ? a.kmap[(size_t)bh * N + j] : j;  // the row written
  if (j < N && (unsigned)jo < (unsigned)N) {
    float* dkg = static_cast<float*>(a.dk) + khead + (size_t)jo * D;
    float* dvg = static_cast<float*>(a.dv) + khead + (size_t)jo * D;
#pragma unroll
    for (int db = 0; db < Tr::NDB; ++db) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = db * 32 + 8 * q4 + 4 * g;
        f32x4 wk, wv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          wk[e] = dk[db][4 * q4 + e] * a.scale;
          wv[e] = dv[db][4 * q4 + e];
        }
        *reinterpret_cast<f32x4*>(dkg + d0) = wk;
        *reinterpret_cast<f32x4*>(dvg + d0) = wv;
      }
    }
  }
}

// ------------------------------------------------------------------ host launch

hipError_t launch_dq_stream(int d, const void* k, const void* ds, long long cap, const DsPlan& plan, void* dq,
                            const int* bounds, int B, int H, int Hm, int N, int causal, float scale,
                            hipStream_t stream);

template <typename T, int D>
static hipError_t launch_bwd_t(BwdArgs a, hipStream_t stream) {
  // bf16 at d = 64: 128-key tiles (half the barriers per key, as the dK/dV kernel's 128-row tiles there)
  constexpr int BCQ = (sizeof(T) == 2 && D == 64) ? 128 : 64;
  const long nq = (a.Nq + DqTraits<T, D, BCQ>::BR - 1) / DqTraits<T, D, BCQ>::BR;
  hipLaunchKernelGGL((bwd_dq_kernel<T, D, BCQ>), dim3((unsigned)(nq * a.B * a.H)), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long nkt = (a.Nk + 127) / 128;
  if constexpr (sizeof(T) == 2) {
    // 128-row query tiles at d = 64 (half the barriers and tile bookkeeping per row; the registers allow
    // it there), 64-row tiles at d = 128 and whenever dS tiles are stored (their unit is 64 rows).
    bool tall = false;
    if constexpr (D == 64) tall = a.ds_cache == nullptr;
    if (tall) {
      hipLaunchKernelGGL((bwd_dkdv_pair_kernel<64, 128>), dim3((unsigned)(nkt * a.B * a.H)), dim3(512), 0, stream, a);
    } else {
      hipLaunchKernelGGL((bwd_dkdv_pair_kernel<D, 64>), dim3((unsigned)(nkt * a.B * a.H)), dim3(512), 0, stream, a);
    }
    if (a.ds_cache != nullptr) {
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      return launch_dq_stream(D, a.k, a.ds_cache, a.ds_cap, a.ds, a.dq, a.bounds, a.B, a.H, a.Hm, a.Nk, a.causal,
                              a.scale, stream);
    }
  } else {
    hipLaunchKernelGGL((bwd_dkdv_f32_kernel<D>), dim3((unsigned)(nkt * a.B * a.H)), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_bwd(bool bf16_in, int d, const void* q, const void* k, const void* v, const void* out,
                      const void* dout, const float* lse, void* dq, void* dk, void* dv, float* dd, const int* lts,
                      const int* lte, const int* uts, const int* ute, const int* bounds, int B, int H, int Nq,
                      int Nk, int q_off, int Hm, const int* sched, int causal, float scale,
                      hipStream_t stream, const int* qmap, const int* kmap, void* ds_cache, long long ds_cap,
                      const DsPlan* ds_plan) {
  BwdArgs a;
  a.q = q; a.k = k; a.v = v; a.out = out; a.dout = dout; a.lse = lse; a.dd = dd;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.lts = lts; a.lte = lte; a.uts = uts; a.ute = ute; a.bounds = bounds;
  a.B = B; a.H = H; a.Hm = Hm;
  a.Nq = Nq; a.Nk = Nk; a.q_off = q_off;
  a.nkb = (Nk + KBLOCK - 1) / KBLOCK;
  a.sched = sched;
  a.sched_nq = (Nq + SCHED_UNIT - 1) / SCHED_UNIT;
  a.sched_stride = 2 * (a.sched_nq + (Nk + SCHED_UNIT - 1) / SCHED_UNIT);
  a.causal = causal;
  a.scale = scale;
  a.scale_log2 = scale * LOG2E;
  a.qmap = qmap;
  a.kmap = kmap;
  a.ds_cache = bf16_in ? static_cast<char*>(ds_cache) : nullptr;  // float32 keeps the recomputing dq pass
  a.ds_cap = ds_cap;
  a.ds = ds_plan != nullptr ? *ds_plan : DsPlan{};
  if (bf16_in) return d == 64 ? launch_bwd_t<bf16, 64>(a, stream) : launch_bwd_t<bf16, 128>(a, stream);
  return d == 64 ? launch_bwd_t<float, 64>(a, stream) : launch_bwd_t<float, 128>(a, stream);
}

}  // namespace fm
