// Forward pass of exact attention under the column-wise mask (gfx950).
//
// Tiled online softmax as in FlashAttention (FlashAttention-3 abstract, fugumt.com 2407.08608; the
// FlashAttention README on wenyanet.com), with tiles that the mask covers completely skipped and
// tiles it does not touch run without the elementwise mask (FlashMask abstract,
// papers.pytorch.kr 2410.01359).
//
// Work decomposition (a design for 64-wide waves and 32x32 matrix cores, not taken from the pages):
//  * one workgroup = 4 waves = BR = 128 query rows of one (b, h); wave w owns rows 32 w .. 32 w + 31;
//    two workgroups share a compute unit (one wave per SIMD each) so that one wave's softmax overlaps
//    the other's matrix products.
//  * key tiles of BC = 64 columns (one bounds entry). The live (not fully masked) tiles are found 64 at
//    a time with one wave-wide ballot; the next live tile is fetched from HBM into registers while the
//    current one is computed, and K / V are double-buffered in LDS. For bf16 the tiles are unpadded with
//    an XOR chunk swizzle (conflict-free for the row reads of K and the transposing reads of V) and are
//    filled by direct global-to-LDS copies, so no registers stage them.
//  * each wave computes S^T = K Q^T (keys as the M axis, its 32 queries as the N axis), so every lane
//    holds one query row and the row max needs one exchange with lane ^ 32; the row sum stays split
//    across the two lanes until the epilogue.
//  * exponentials use a per-row reference max that is only raised when a tile's max exceeds it by more
//    than 2^8 (log2 units); O and the row sum always share that reference, so the result is exact and
//    the accumulator rescale runs only when the reference moves.
//  * P^T stays in registers and is the k-operand of O^T += V^T P^T; V^T fragments come from the
//    row-major V tile through transposing LDS reads.
//  * grid order: heaviest query tiles first (causal / document masks load late tiles most).
#include "fm_common.h"

namespace fm {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  const int* lts;
  const int* lte;
  const int* uts;
  const int* ute;
  const int* bounds;
  int B, H, Hm;
  int Nq, Nk;  // query rows and keys per head
  int q_off;   // global index of query row 0: the mask and the causal rule see rows q_off + i
  int nq;   // query tiles per head
  int nkb;  // bounds entries per (b, hm) row
  const int* sched;  // longest-first unit order (query units at offset 0) or null
  int sched_stride;  // int32 per (b, hm) row of sched
  int causal;
  float scale_log2;  // scale * log2(e)
  const int* omap;   // null, or [B, H, Nq]: out row r of (b, h) is stored at row omap[r] (rows outside
                     // [0, Nq) are not stored); lse stays at row r
};

template <typename T, int D>
struct FwdTraits {
  static constexpr int BR = 128;
  static constexpr int BC = 64;
  static constexpr int NT = 256;
  static constexpr int PITCH = D + 16 / (int)sizeof(T);  // K rows: 16-byte padding (row-wise reads)
  // V rows (bf16): 64-byte padding, so that the four rows of one transposing read start 16 banks apart
  static constexpr int VPITCH = sizeof(T) == 2 ? D + 32 : PITCH;
  static constexpr int NQF = D / MM<T>::KW;              // Q fragments per lane
  static constexpr int NDB = D / 32;                     // 32-wide output column blocks
  static constexpr int TPB = 16 / MM<T>::E;              // products per 32-key block in P V
  static constexpr int CPR = D * (int)sizeof(T) / 16;    // 16-byte chunks per K / V row
  static constexpr int CH = BC * CPR / NT;               // chunks per thread per K / V tile
};

constexpr float RESCALE_THRESHOLD = 8.0f;  // log2 units: unnormalised probabilities stay below 256

template <typename T, int D>
__global__ __launch_bounds__(256, (sizeof(T) == 2 && D == 64) ? 4 : 2) void fwd_kernel(FwdArgs a) {
  using Tr = FwdTraits<T, D>;
  using M = MM<T>;
  constexpr int BR = Tr::BR, BC = Tr::BC, PITCH = Tr::PITCH, CPR = Tr::CPR, CH = Tr::CH;
  constexpr int VPITCH = Tr::VPITCH;
  // bf16: K and V tiles are swizzled and unpadded, filled by direct global-to-LDS copies (no staging
  // registers). float: padded row-major tiles staged through registers.
  constexpr bool SWZ = sizeof(T) == 2;
  constexpr int KLP = SWZ ? D : PITCH;
  constexpr int VLP = SWZ ? D : VPITCH;
  __shared__ __attribute__((aligned(16))) T k_lds[2][BC * KLP];
  __shared__ __attribute__((aligned(16))) T v_lds[2][BC * VLP];
  __shared__ __attribute__((aligned(16))) int vec_lds[2][4][BC];  // LTS, LTE, UTS, UTE of the tile's columns
  __shared__ __attribute__((aligned(16))) uint32_t cw_lds[4][BC];  // per wave: masked-row words of a tile

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
  static_assert(BR == SCHED_UNIT, "query units of the schedule are forward tiles");
  const int qt = scheduled_unit(a.sched, a.sched_stride, (size_t)b * a.Hm + hm, 0, rank, a.nq, a.nq - 1 - rank);
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
  const size_t vrow = ((size_t)b * a.Hm + hm) * N;
  const int* brow = a.bounds == nullptr ? nullptr : a.bounds + ((size_t)b * a.Hm + hm) * a.nkb * 8;
  const bool has_lt = a.lts != nullptr;
  const bool has_ut = a.uts != nullptr;
  const bool causal = a.causal != 0;
  const float sl2 = a.scale_log2;

  f32x16 o[Tr::NDB];
#pragma unroll
  for (int db = 0; db < Tr::NDB; ++db) o[db] = zero16();
  float m_ref = -INFINITY;  // reference max (log2 units) of this row's exponentials
  float l_run = 0.f;        // this lane's share of the denominator, relative to m_ref

  const int nkt = (N + BC - 1) / BC;
  const int kt_end = causal ? min(nkt, (g1 - 1) / BC + 1) : nkt;

  // Next tile: K / V and the tile's mask vectors. bf16: straight into LDS buffer `dst` by direct copies
  // (one vector per wave); float: into staging registers, stored by stash().
  constexpr int CHR = SWZ ? 1 : CH;
  i32x4 kr[CHR], vr[CHR];
  i32x4 mr = {0, 0, 0, 0};
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  auto fetch_vectors = [&](int kt, int dst) {
    copy_tile_vectors(vec_lds[dst], a.lts, a.lte, a.uts, a.ute, vrow, kt * BC, N, wv, lane);
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
        st16(reinterpret_cast<char*>(&k_lds[buf][r * PITCH]) + cc * 16, kr[it]);
        st16(reinterpret_cast<char*>(&v_lds[buf][r * VPITCH]) + cc * 16, vr[it]);
      }
      if (tid < BC) {
#pragma unroll
        for (int e = 0; e < 4; ++e) vec_lds[buf][e][tid] = mr[e];
      }
    }
  };
  SwzRowReads<D> krd;
  SwzColReads<D> vcd;
  if constexpr (SWZ) {
    krd.init(lane);
    vcd.init(lane);
  }

  auto class_of = [&](int t) {
    const TileBounds bt = merged_bounds(brow, t, t + 1, N);
    return classify_tile(g0, g1, t * BC, min(N, t * BC + BC), bt, causal);
  };
  TileWindow win = empty_window();
  int kt = next_live_tile(win, 0, kt_end, class_of, lane);
  if (kt < kt_end) fetch(kt, 0);
  // Q^T operand: lane holds row `row`, k = d in chunks of KW. Loaded after the tile scan and the first
  // tile's copies, so that the scan waits only for the tile bounds (loads complete in issue order) and the
  // Q loads travel with the copies.
  typename M::frag qf[Tr::NQF];
#pragma unroll
  for (int c = 0; c < Tr::NQF; ++c) {
    if (row < Nq) {
      qf[c] = load_kcontig_frag<T>(qg + (size_t)row * D + c * M::KW + g * M::E);
    } else {
      qf[c] = typename M::frag{};
    }
  }
  int buf = 0;
  // Loop-invariant parts of the next tile's copies: LDS bases of the tile buffers, and this wave's mask
  // vector (wave w of the first four copies LTS, LTE, UTS, UTE when present).
  const uint32_t k_lds0 = lds_addr(k_lds), v_lds0 = lds_addr(v_lds), vec_lds0 = lds_addr(vec_lds);
  const int* vsrc = wv == 0 ? a.lts : wv == 1 ? a.lte : wv == 2 ? a.uts : a.ute;
  const bool vcopy = vsrc != nullptr;
  if (vcopy) vsrc += vrow;

  while (kt < kt_end) {
    const int c0 = kt * BC;
    const bool need_mask = window_partial(win, kt) || (c0 + BC > N);
    stash(buf);
    if constexpr (SWZ) __builtin_amdgcn_s_waitcnt(0);  // this tile's direct copies have landed
    __syncthreads();
    // the first two K fragments, read before the tile scan so that their latency overlaps it
    bf16x8 kpre[2];
    if constexpr (SWZ) {
      kpre[0] = krd.read(reinterpret_cast<const bf16*>(k_lds[buf]), 0, 0);
      kpre[1] = krd.read(reinterpret_cast<const bf16*>(k_lds[buf]), 0, 1);
    }
    const int kt_next = next_live_tile(win, kt + 1, kt_end, class_of, lane);
    // bf16: the next tile's copies go out one at a time between the score products below, so that they
    // queue while the matrix cores work instead of holding up the products. Without a next tile the
    // current one is copied into the other buffer, which is never read, so the sequence is the same.
    TileCopy<D, BC, 4> kcp, vcp;
    if constexpr (SWZ) {
      const int cn = (kt_next < kt_end ? kt_next : kt) * BC;
      const uint32_t boff = (uint32_t)(buf ^ 1) * (BC * D * 2);
      kcp.prep_at(k_lds0 + boff, reinterpret_cast<const bf16*>(kg), cn, N, wave, lane);
      vcp.prep_at(v_lds0 + boff, reinterpret_cast<const bf16*>(vg), cn, N, wave, lane);
      if (vcopy && kt_next < kt_end)
        lds_copy4(vsrc, (uint32_t)min(kt_next * BC + lane, N - 1) * 4u,
                  vec_lds0 + (uint32_t)(buf ^ 1) * (4 * BC * 4) + (uint32_t)wv * (BC * 4));
    } else {
      if (kt_next < kt_end) fetch(kt_next, buf ^ 1);
    }

    const T* kt_lds = k_lds[buf];
    const T* vt_lds = v_lds[buf];
    // S^T for the two 32-key blocks: rows = keys, columns = this wave's queries. Matrix-product blocks
    // run at raised wave priority so that the two waves of a SIMD drift into opposite phases (one in
    // products, one in softmax arithmetic).
    __builtin_amdgcn_s_setprio(2);
    f32x16 s[2];
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
      s[jb] = zero16();
      if constexpr (SWZ) {
        constexpr int NC = 2 * TileCopy<D, BC, 4>::NK;  // copies, one after every other product
        static_assert(NC == Tr::NQF, "one copy per two score products");
#pragma unroll
        for (int c = 0; c < Tr::NQF; ++c) {
          s[jb] = M::mma(jb == 0 && c < 2 ? kpre[c] : krd.read(kt_lds, jb, c), qf[c], s[jb]);
          if (c & 1) {
            const int k = (jb * Tr::NQF + c) >> 1;
            if (k < NC / 2) kcp.issue(k); else vcp.issue(k - NC / 2);
          }
        }
      } else {
        const T* krow = kt_lds + (jb * 32 + l32) * PITCH + g * M::E;
#pragma unroll
        for (int c = 0; c < Tr::NQF; ++c) s[jb] = M::mma(load_kcontig_frag<T>(krow + c * M::KW), qf[c], s[jb]);
      }
    }
    interleave_reads<2 * Tr::NQF, 2 * Tr::NQF - 2, 2>();

    __builtin_amdgcn_s_setprio(0);
    // Scores stay unscaled until the exponent (scale * log2(e) > 0 keeps the max); masked ones are -inf.
    if (need_mask) {
      tile_column_words(cw_lds[wave], &vec_lds[buf][0][0], g0 + wave * 32, c0, gend, N, causal, has_lt, has_ut, lane);
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const i32x4 w4 = column_words4(cw_lds[wave], jb, q4, g);
#pragma unroll
          for (int e = 0; e < 4; ++e) s[jb][4 * q4 + e] = select_neg_inf(row_mask_of(w4[e], l32), s[jb][4 * q4 + e]);
        }
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[jb][r]);
    }
    mx = pair_max(mx) * sl2;
    // Raise the reference only when some row of the wave would exceed it by more than the threshold.
    const bool grow = mx > m_ref + RESCALE_THRESHOLD;
    if (__ballot(grow) != 0) {
      const float m_new = fmaxf(m_ref, mx);
      const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < Tr::NDB; ++db) {
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      }
    }
    const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
    float psum = 0.f;
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[jb][r], sl2, -m_use));
        s[jb][r] = p;
        psum += p;
      }
    }
    l_run += psum;

    // O^T += V^T P^T over the 64 keys of the tile.
    __builtin_amdgcn_s_setprio(2);
#pragma unroll
    for (int t = 0; t < 2 * Tr::TPB; ++t) {
      const typename M::frag pf = acc_frag<T>(s[t / Tr::TPB], t % Tr::TPB);
#pragma unroll
      for (int db = 0; db < Tr::NDB; ++db) {
        if constexpr (SWZ) {
          o[db] = M::mma(vcd.read(vt_lds, t, db), pf, o[db]);
        } else {
          o[db] = M::mma(load_kmajor_frag<T>(vt_lds, VPITCH, 0, db * 32, t, lane), pf, o[db]);
        }
      }
    }
    interleave_reads<2 * Tr::TPB * Tr::NDB, 4 * Tr::TPB * Tr::NDB, 4>();
    __builtin_amdgcn_s_setprio(0);
    kt = kt_next;
    buf ^= 1;
  }

  if constexpr (SWZ) __builtin_amdgcn_s_waitcnt(0);  // the last tile's copies (never read) have landed
  // Epilogue: out = O / l, lse = m_ref * ln2 + ln(l); rows with no unmasked key give 0 and -inf.
  const float l_tot = pair_sum(l_run);
  const float inv = !(l_tot > 0.f) ? 0.f : 1.f / l_tot;
  if constexpr (SWZ) {
    if (a.omap == nullptr) {
      // Unmapped bf16 output: whole rows through LDS (the K tile buffers, free once every wave is here).
      static_assert(sizeof(k_lds) >= 4 * 32 * D * 2, "staging area of four waves");
      __syncthreads();
      const int w0 = r0 + wave * 32;
      store_rows_staged<D>(reinterpret_cast<char*>(&k_lds[0][0]) + wave * (32 * D * 2), o, inv,
                           static_cast<bf16*>(a.out) + qhead + (size_t)w0 * D, Nq - w0, lane);
      if (row < Nq && g == 0) a.lse[(size_t)bh * Nq + row] = !(l_tot > 0.f) ? -INFINITY : m_ref * LN2 + logf(l_tot);
      return;
    }
  }
  const int orow = (a.omap != nullptr && row < Nq) ? a.omap[(size_t)bh * Nq + row] : row;
  if (row < Nq && (unsigned)orow < (unsigned)Nq) {
    T* og = static_cast<T*>(a.out) + qhead + (size_t)orow * D;
#pragma unroll
    for (int db = 0; db < Tr::NDB; ++db) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = db * 32 + 8 * q4 + 4 * g;
        if constexpr (sizeof(T) == 2) {
          bf16x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = (bf16)(o[db][4 * q4 + e] * inv);
          *reinterpret_cast<bf16x4*>(og + d0) = w;
        } else {
          f32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = o[db][4 * q4 + e] * inv;
          *reinterpret_cast<f32x4*>(og + d0) = w;
        }
      }
    }
  }
  if (row < Nq && g == 0) a.lse[(size_t)bh * Nq + row] = !(l_tot > 0.f) ? -INFINITY : m_ref * LN2 + logf(l_tot);
}

template <typename T, int D>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  const long grid = (long)a.nq * a.B * a.H;
  hipLaunchKernelGGL((fwd_kernel<T, D>), dim3((unsigned)grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

int fwd_qblock() { return 128; }

hipError_t launch_fwd(bool bf16_in, int d, const void* q, const void* k, const void* v, void* out, float* lse,
                      const int* lts, const int* lte, const int* uts, const int* ute, const int* bounds, int B, int H,
                      int Nq, int Nk, int q_off, int Hm, const int* sched, int causal, float scale,
                      hipStream_t stream, const int* omap) {
  FwdArgs a;
  a.q = q; a.k = k; a.v = v; a.out = out; a.lse = lse;
  a.lts = lts; a.lte = lte; a.uts = uts; a.ute = ute; a.bounds = bounds;
  a.B = B; a.H = H; a.Hm = Hm;
  a.Nq = Nq; a.Nk = Nk; a.q_off = q_off;
  a.nq = (Nq + 127) / 128;
  a.nkb = (Nk + KBLOCK - 1) / KBLOCK;
  a.sched = sched;
  a.sched_stride = 2 * (a.nq + (Nk + SCHED_UNIT - 1) / SCHED_UNIT);
  a.causal = causal;
  a.scale_log2 = scale * LOG2E;
  a.omap = omap;
  if (bf16_in) return d == 64 ? launch_fwd_t<bf16, 64>(a, stream) : launch_fwd_t<bf16, 128>(a, stream);
  return d == 64 ? launch_fwd_t<float, 64>(a, stream) : launch_fwd_t<float, 128>(a, stream);
}

}  // namespace fm
