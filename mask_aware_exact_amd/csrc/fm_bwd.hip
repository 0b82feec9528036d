// Backward pass of exact attention under the column-wise mask (gfx950).
//
// The gradient of sum(out * dO) through softmax attention, recomputing P from q, k and the forward's
// lse, with tiles the mask covers completely skipped (FlashMask abstract, papers.pytorch.kr
// 2410.01359). Three kernels run in order on the caller's stream:
//  1. bwd_pre:  D_i = sum_d dO_id out_id (float32) per row, and the float32 dq accumulator cleared.
//  2. bwd_main: one workgroup per (b, h, key tile of BC = 128 columns); wave w owns keys 32 w .. 32 w+31
//     (one key column per lane). The live query tiles (not fully masked for this key tile) are found
//     64 at a time with a wave ballot; the next one is loaded into registers while the current one is
//     computed, and Q / dO are double-buffered row-major in LDS. Per live query tile of BR rows:
//       S = Q K^T and dP = dO V^T with K, V held in registers (keys as the N axis, so every lane keeps
//       one key column and its four mask values in registers);
//       P = exp(S - lse) (0 where masked), dS = P o (dP - D);
//       dV^T += dO^T P and dK^T += Q^T dS, the k axis (query rows) read from the row-major Q / dO
//       tiles through transposing LDS reads, accumulated on chip for the whole query loop;
//       dS goes to LDS, and each wave forms dQ = dS K for one 32-wide d block over the workgroup's
//       128 keys, with that block of K held in registers (loaded once), and adds it into the float32
//       accumulator with hardware float atomics (one 128-byte row segment per instruction).
//  3. bwd_dq:   dq = accumulator rounded to the input type.
#include "fm_common.h"

namespace fm {

// ------------------------------------------------------------------ 1. D and accumulator clear

template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const T* __restrict__ out, const T* __restrict__ dout,
                                                      float* __restrict__ dd, float* __restrict__ dq_acc,
                                                      long rows) {
  constexpr int CPR = D * (int)sizeof(T) / 16;  // 16-byte chunks per row
  constexpr int EPC = 16 / (int)sizeof(T);      // elements per chunk
  constexpr int RPB = 256 / CPR;                // rows per block
  constexpr int ACC_CHUNKS = D * 4 / 16 / CPR;  // 16-byte accumulator chunks per lane
  const int tid = threadIdx.x;
  const long row = (long)blockIdx.x * RPB + tid / CPR;
  const int c = tid % CPR;
  float part = 0.f;
  if (row < rows) {
    const T* po = out + row * D + c * EPC;
    const T* pd = dout + row * D + c * EPC;
#pragma unroll
    for (int e = 0; e < EPC; ++e) part += (float)po[e] * (float)pd[e];
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < ACC_CHUNKS; ++k)
      *reinterpret_cast<f32x4*>(dq_acc + row * D + (c * ACC_CHUNKS + k) * 4) = z;
  }
#pragma unroll
  for (int m = CPR / 2; m >= 1; m >>= 1) part += __shfl_xor(part, m, 64);
  if (row < rows && c == 0) dd[row] = part;
}

// ------------------------------------------------------------------ 2. main key-tile-parallel kernel

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const float* lse;
  const float* dd;
  float* dq_acc;
  void* dk;
  void* dv;
  const int* lts;
  const int* lte;
  const int* uts;
  const int* ute;
  const int* bounds;
  int B, H, N, Hm;
  int nkt;  // key tiles of BC per head
  int nkb;  // bounds entries per (b, hm) row
  int causal;
  float scale;
  float scale_log2;
};

template <typename T, int D>
struct BwdTraits {
  static constexpr int BC = 128;                         // keys per workgroup
  static constexpr int BR = sizeof(T) == 2 ? 64 : 32;    // query rows per iteration
  static constexpr int NT = 256;
  static constexpr int PITCH = D + 16 / (int)sizeof(T);  // row-major Q / dO / K tiles
  static constexpr int PS = BR + 16 / (int)sizeof(T);    // dS tile [key][row]
  static constexpr int NKF = D / MM<T>::KW;              // K / V fragments per lane (k = d)
  static constexpr int NIB = BR / 32;                    // 32-row blocks per query tile
  static constexpr int NDB = D / 32;                     // 32-wide d blocks
  static constexpr int TPB = 16 / MM<T>::E;              // products per 32 k values
  static constexpr int NKQ = BC / 32 * TPB;              // products over the workgroup's keys (dQ)
  static constexpr int WPD = 4 / NDB;                    // waves sharing one d block in dQ
  static constexpr int CPR = D * (int)sizeof(T) / 16;    // 16-byte chunks per row
  static constexpr int CH = BR * CPR / NT;               // chunks per thread per Q / dO tile
  static_assert(BC * CPR % NT == 0 && CH >= 1, "tile copies must divide evenly");
};

template <typename T, int D>
__global__ __launch_bounds__(256, 1) void bwd_main_kernel(BwdArgs a) {
  using Tr = BwdTraits<T, D>;
  using M = MM<T>;
  constexpr int BC = Tr::BC, BR = Tr::BR, PITCH = Tr::PITCH, PS = Tr::PS, CPR = Tr::CPR, CH = Tr::CH;
  // q_lds / do_lds hold two query tiles each (double buffer); at start-up the same memory holds the K tile.
  static_assert(4 * BR >= BC, "the K tile is staged through the query-tile buffers");
  __shared__ __attribute__((aligned(16))) T qdo_lds[4 * BR * PITCH];
  T* const q_lds = qdo_lds;
  T* const do_lds = qdo_lds + 2 * BR * PITCH;
  __shared__ __attribute__((aligned(16))) T ds_lds[BC * PS];
  __shared__ __attribute__((aligned(16))) float lse_lds[2][BR];
  __shared__ __attribute__((aligned(16))) float dd_lds[2][BR];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int g = lane >> 5;
  const int l32 = lane & 31;

  const int BH = a.B * a.H;
  const int bh = blockIdx.x % BH;
  const int kt = (int)(blockIdx.x / BH);  // early key tiles carry the most causal work: dispatch them first
  const int b = bh / a.H;
  const int h = bh % a.H;
  const int hm = a.Hm > 1 ? h : 0;
  const int N = a.N;
  const int c0 = kt * BC;
  const int c1 = min(N, c0 + BC);
  const int jl = wave * 32 + l32;  // this lane's key column inside the tile
  const int j = c0 + jl;

  const size_t head = (size_t)bh * N * D;
  const T* __restrict__ qg = static_cast<const T*>(a.q) + head;
  const T* __restrict__ kg = static_cast<const T*>(a.k) + head;
  const T* __restrict__ vg = static_cast<const T*>(a.v) + head;
  const T* __restrict__ dog = static_cast<const T*>(a.dout) + head;
  const float* __restrict__ lseg = a.lse + (size_t)bh * N;
  const float* __restrict__ ddg = a.dd + (size_t)bh * N;
  float* __restrict__ dqg = a.dq_acc + head;
  const size_t vrow = ((size_t)b * a.Hm + hm) * N;
  const int* brow = a.bounds == nullptr ? nullptr : a.bounds + ((size_t)b * a.Hm + hm) * a.nkb * 8;
  const bool has_lt = a.lts != nullptr;
  const bool has_ut = a.uts != nullptr;
  const bool causal = a.causal != 0;
  const float sl2 = a.scale_log2;

  // This lane's key column: mask values and K / V fragments with k = d (operand B of S and dP).
  int m_lts = 0, m_lte = 0, m_uts = 0, m_ute = 0;
  typename M::frag kf[Tr::NKF], vf[Tr::NKF];
  if (j < N) {
    if (has_lt) { m_lts = a.lts[vrow + j]; m_lte = a.lte[vrow + j]; }
    if (has_ut) { m_uts = a.uts[vrow + j]; m_ute = a.ute[vrow + j]; }
#pragma unroll
    for (int c = 0; c < Tr::NKF; ++c) {
      kf[c] = load_kcontig_frag<T>(kg + (size_t)j * D + c * M::KW + g * M::E);
      vf[c] = load_kcontig_frag<T>(vg + (size_t)j * D + c * M::KW + g * M::E);
    }
  } else {
#pragma unroll
    for (int c = 0; c < Tr::NKF; ++c) {
      kf[c] = typename M::frag{};
      vf[c] = typename M::frag{};
    }
  }

  // K fragments with k = key (operand B of dQ = dS K) for this wave's 32-wide d block, read once
  // through the LDS from the row-major K tile.
  const int wd = wave % Tr::NDB;
  load_tile<T, BC, D, PITCH, Tr::NT>(q_lds, kg, c0, N, tid);
  __syncthreads();
  typename M::frag kq[Tr::NKQ];
#pragma unroll
  for (int t = 0; t < Tr::NKQ; ++t) kq[t] = load_kmajor_frag<T>(q_lds, PITCH, 0, wd * 32, t, lane);
  __syncthreads();

  f32x16 dk[Tr::NDB], dv[Tr::NDB];
#pragma unroll
  for (int db = 0; db < Tr::NDB; ++db) {
    dk[db] = zero16();
    dv[db] = zero16();
  }

  int bnd[8];
  merged_bounds(brow, kt * (BC / KBLOCK), min(a.nkb, (kt + 1) * (BC / KBLOCK)), N, bnd);
  const int nq = (N + BR - 1) / BR;
  const int qt_begin = causal ? c0 / BR : 0;
  auto class_of = [&](int qt) { return classify_tile(qt * BR, min(N, qt * BR + BR), c0, c1, bnd, causal); };

  // Prefetch registers for one query tile.
  i32x4 qr[CH], dr[CH];
  float lr = 0.f, ddr = 0.f;
  auto fetch = [&](int qt) {
    const int q0 = qt * BR;
#pragma unroll
    for (int it = 0; it < CH; ++it) {
      const int c = it * Tr::NT + tid;
      const int r = c / CPR, cc = c % CPR;
      qr[it] = i32x4{0, 0, 0, 0};
      dr[it] = i32x4{0, 0, 0, 0};
      if (q0 + r < N) {
        qr[it] = ld16(reinterpret_cast<const char*>(qg + (size_t)(q0 + r) * D) + cc * 16);
        dr[it] = ld16(reinterpret_cast<const char*>(dog + (size_t)(q0 + r) * D) + cc * 16);
      }
    }
    if (tid < BR) {
      const int i = q0 + tid;
      lr = i < N ? lseg[i] : INFINITY;
      ddr = i < N ? ddg[i] : 0.f;
    }
  };
  auto stash = [&](int buf) {
    T* qb = q_lds + buf * BR * PITCH;
    T* db_ = do_lds + buf * BR * PITCH;
#pragma unroll
    for (int it = 0; it < CH; ++it) {
      const int c = it * Tr::NT + tid;
      const int r = c / CPR, cc = c % CPR;
      st16(reinterpret_cast<char*>(qb + r * PITCH) + cc * 16, qr[it]);
      st16(reinterpret_cast<char*>(db_ + r * PITCH) + cc * 16, dr[it]);
    }
    if (tid < BR) {
      // a row without any unmasked key has lse = -inf; +inf makes exp(S - lse) = 0 for it
      const float l = (lr == -INFINITY) ? INFINITY : lr;
      lse_lds[buf][tid] = l * LOG2E;
      dd_lds[buf][tid] = ddr;
    }
  };

  TileWindow win = empty_window();
  int qt = next_live_tile(win, qt_begin, nq, class_of, lane);
  if (qt < nq) fetch(qt);
  int buf = 0;

  while (qt < nq) {
    const int q0 = qt * BR;
    const bool need_mask = window_partial(win, qt) || (q0 + BR > N) || (c0 + BC > N);
    stash(buf);
    __syncthreads();  // (A) this tile is in LDS; every wave is past the previous tile's dQ phase
    const int qt_next = next_live_tile(win, qt + 1, nq, class_of, lane);
    if (qt_next < nq) fetch(qt_next);

    const T* qb = q_lds + buf * BR * PITCH;
    const T* dob = do_lds + buf * BR * PITCH;
    // S = Q K^T and dP = dO V^T: rows = this tile's queries, columns = this wave's keys.
    f32x16 s[Tr::NIB], dp[Tr::NIB];
#pragma unroll
    for (int ib = 0; ib < Tr::NIB; ++ib) {
      s[ib] = zero16();
      dp[ib] = zero16();
      const T* qrow = qb + (ib * 32 + l32) * PITCH + g * M::E;
      const T* dorow = dob + (ib * 32 + l32) * PITCH + g * M::E;
#pragma unroll
      for (int c = 0; c < Tr::NKF; ++c) {
        s[ib] = M::mma(load_kcontig_frag<T>(qrow + c * M::KW), kf[c], s[ib]);
        dp[ib] = M::mma(load_kcontig_frag<T>(dorow + c * M::KW), vf[c], dp[ib]);
      }
    }

    // P and dS in place (s <- P, dp <- dS). Masked rows of this lane's key column come from a bitmap.
    const uint64_t mbits = need_mask ? masked_row_bits(q0, j, N, causal, has_lt, has_ut, m_lts, m_lte, m_uts, m_ute)
                                     : 0ull;
    const uint64_t mg = mbits >> (4 * g);
#pragma unroll
    for (int ib = 0; ib < Tr::NIB; ++ib) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int il0 = ib * 32 + 8 * q4 + 4 * g;
        const f32x4 lse4 = *reinterpret_cast<const f32x4*>(&lse_lds[buf][il0]);
        const f32x4 dd4 = *reinterpret_cast<const f32x4*>(&dd_lds[buf][il0]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * q4 + e;
          float p = __builtin_amdgcn_exp2f(s[ib][r] * sl2 - lse4[e]);
          p = ((mg >> (ib * 32 + 8 * q4 + e)) & 1) ? 0.f : p;
          s[ib][r] = p;
          dp[ib][r] = p * (dp[ib][r] - dd4[e]);
        }
      }
    }

    // dV^T += dO^T P and dK^T += Q^T dS (k = query rows of the tile).
#pragma unroll
    for (int t = 0; t < Tr::NIB * Tr::TPB; ++t) {
      const typename M::frag pf = acc_frag<T>(s[t / Tr::TPB], t % Tr::TPB);
      const typename M::frag sf = acc_frag<T>(dp[t / Tr::TPB], t % Tr::TPB);
#pragma unroll
      for (int db = 0; db < Tr::NDB; ++db) {
        dv[db] = M::mma(load_kmajor_frag<T>(dob, PITCH, 0, db * 32, t, lane), pf, dv[db]);
        dk[db] = M::mma(load_kmajor_frag<T>(qb, PITCH, 0, db * 32, t, lane), sf, dk[db]);
      }
    }

    // dS to LDS as [key][row], rounded to T.
#pragma unroll
    for (int ib = 0; ib < Tr::NIB; ++ib) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int il0 = ib * 32 + 8 * q4 + 4 * g;
        T* dst = ds_lds + jl * PS + il0;
        if constexpr (sizeof(T) == 2) {
          bf16x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = (bf16)dp[ib][4 * q4 + e];
          *reinterpret_cast<bf16x4*>(dst) = w;
        } else {
          f32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = dp[ib][4 * q4 + e];
          *reinterpret_cast<f32x4*>(dst) = w;
        }
      }
    }
    __syncthreads();  // (B) dS of all four waves is in LDS

    // dQ rows += scale * dS K over the workgroup's keys, for this wave's d block.
#pragma unroll
    for (int ib = wave / Tr::NDB; ib < Tr::NIB; ib += Tr::WPD) {
      f32x16 acc = zero16();
#pragma unroll
      for (int t = 0; t < Tr::NKQ; ++t) acc = M::mma(load_kmajor_frag<T>(ds_lds, PS, 0, ib * 32, t, lane), kq[t], acc);
      float* dst = dqg + (size_t)(q0 + ib * 32 + 4 * g) * D + wd * 32 + l32;
      if (q0 + BR <= N) {
#pragma unroll
        for (int r = 0; r < 16; ++r) unsafeAtomicAdd(dst + (8 * (r >> 2) + (r & 3)) * D, acc[r] * a.scale);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = q0 + ib * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          if (i < N) unsafeAtomicAdd(dst + (8 * (r >> 2) + (r & 3)) * D, acc[r] * a.scale);
        }
      }
    }
    qt = qt_next;
    buf ^= 1;
  }

  // dK = scale * dK^T, dV = dV^T for this lane's key column.
  if (j < N) {
    T* dkg = static_cast<T*>(a.dk) + head + (size_t)j * D;
    T* dvg = static_cast<T*>(a.dv) + head + (size_t)j * D;
#pragma unroll
    for (int db = 0; db < Tr::NDB; ++db) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = db * 32 + 8 * q4 + 4 * g;
        if constexpr (sizeof(T) == 2) {
          bf16x4 wk, wv;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            wk[e] = (bf16)(dk[db][4 * q4 + e] * a.scale);
            wv[e] = (bf16)dv[db][4 * q4 + e];
          }
          *reinterpret_cast<bf16x4*>(dkg + d0) = wk;
          *reinterpret_cast<bf16x4*>(dvg + d0) = wv;
        } else {
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
}

// ------------------------------------------------------------------ 2b. bf16 main kernel, wave pairs

// bf16 variant of the key-tile-parallel kernel with eight waves: waves w and w + 4 share the 32 keys of
// group w % 4 and split the work so that each keeps fewer than 256 registers (two waves per SIMD):
//   role 0 (w < 4) holds K, forms S = Q K^T and P, and writes P to LDS;
//   role 1 (w >= 4) holds V, forms dP = dO V^T, reads P back, forms dS and writes it to LDS;
//   each role accumulates dV and dK for one half of the d columns, and every wave then forms one
//   32 x 32 block of dQ = dS K over the workgroup's 128 keys.
// While one wave of a SIMD runs its exponentials or dS arithmetic the other issues matrix products.
template <int D>
struct PairTraits {
  static constexpr int BC = 128;          // keys per workgroup
  static constexpr int BR = 64;           // query rows per iteration
  static constexpr int NT = 512;
  static constexpr int PITCH = D + 8;     // row-major Q / dO / K tiles (16-byte row padding)
  static constexpr int PS = BR + 8;       // P and dS tiles [key][row]
  static constexpr int NKF = D / 16;      // K or V fragments per lane (k = d)
  static constexpr int NDB = D / 32;      // 32-wide d blocks
  static constexpr int HDB = NDB / 2;     // d blocks per role
  static constexpr int NQB = 2 * NDB;     // dQ blocks per query tile
  static constexpr int CPR = D * 2 / 16;  // 16-byte chunks per row
  static constexpr int CH = BR * CPR / NT;
  static_assert(BR * CPR % NT == 0 && BC * CPR % NT == 0, "tile copies must divide evenly");
};

template <int D>
__global__ __launch_bounds__(512, 1) void bwd_pair_kernel(BwdArgs a) {
  using Tr = PairTraits<D>;
  using M = MM<bf16>;
  constexpr int BC = Tr::BC, BR = Tr::BR, PITCH = Tr::PITCH, PS = Tr::PS, CPR = Tr::CPR, CH = Tr::CH;
  static_assert(4 * BR * D >= BC * PITCH, "the K tile is staged through the query-tile buffers");
  // Q and dO tiles are swizzled and unpadded (rows of D elements), two of each (double buffer).
  __shared__ __attribute__((aligned(16))) bf16 qdo_lds[4 * BR * D];
  __shared__ __attribute__((aligned(16))) bf16 p_lds[BC * PS];
  __shared__ __attribute__((aligned(16))) bf16 ds_lds[BC * PS];
  __shared__ __attribute__((aligned(16))) float lse_lds[2][BR];
  __shared__ __attribute__((aligned(16))) float dd_lds[2][BR];
  bf16* const q_lds = qdo_lds;
  bf16* const do_lds = qdo_lds + 2 * BR * D;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int g = lane >> 5;
  const int l32 = lane & 31;
  const int kgrp = wave & 3;
  const int role = wave >> 2;

  const int BH = a.B * a.H;
  const int bh = blockIdx.x % BH;
  const int kt = (int)(blockIdx.x / BH);  // early key tiles carry the most causal work: dispatch them first
  const int b = bh / a.H;
  const int h = bh % a.H;
  const int hm = a.Hm > 1 ? h : 0;
  const int N = a.N;
  const int c0 = kt * BC;
  const int c1 = min(N, c0 + BC);
  const int jl = kgrp * 32 + l32;  // this lane's key column inside the tile
  const int j = c0 + jl;

  const size_t head = (size_t)bh * N * D;
  const bf16* __restrict__ qg = static_cast<const bf16*>(a.q) + head;
  const bf16* __restrict__ kg = static_cast<const bf16*>(a.k) + head;
  const bf16* __restrict__ vg = static_cast<const bf16*>(a.v) + head;
  const bf16* __restrict__ dog = static_cast<const bf16*>(a.dout) + head;
  const float* __restrict__ lseg = a.lse + (size_t)bh * N;
  const float* __restrict__ ddg = a.dd + (size_t)bh * N;
  float* __restrict__ dqg = a.dq_acc + head;
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

  // dQ block of this wave (if any) and its K fragments with k = key, read once through the LDS.
  const int ob = wave;
  const bool has_dq = ob < Tr::NQB;
  const int dq_ib = ob / Tr::NDB;
  const int dq_db = ob % Tr::NDB;
  load_tile<bf16, BC, D, PITCH, Tr::NT>(qdo_lds, kg, c0, N, tid);
  __syncthreads();
  bf16x8 kq[BC / 16];
#pragma unroll
  for (int t = 0; t < BC / 16; ++t) kq[t] = load_kmajor_frag<bf16>(qdo_lds, PITCH, 0, dq_db * 32, t, lane);
  __syncthreads();

  f32x16 dk[Tr::HDB], dv[Tr::HDB];
#pragma unroll
  for (int hb = 0; hb < Tr::HDB; ++hb) {
    dk[hb] = zero16();
    dv[hb] = zero16();
  }
  const int db0 = role * Tr::HDB;  // first d block of this role

  int bnd[8];
  merged_bounds(brow, kt * (BC / KBLOCK), min(a.nkb, (kt + 1) * (BC / KBLOCK)), N, bnd);
  const int nq = (N + BR - 1) / BR;
  const int qt_begin = causal ? c0 / BR : 0;
  auto class_of = [&](int qt) { return classify_tile(qt * BR, min(N, qt * BR + BR), c0, c1, bnd, causal); };

  i32x4 qr[CH], dr[CH];
  float lr = 0.f, ddr = 0.f;
  auto fetch = [&](int qt) {
    const int q0 = qt * BR;
#pragma unroll
    for (int it = 0; it < CH; ++it) {
      const int c = it * Tr::NT + tid;
      const int r = c / CPR, cc = c % CPR;
      const bool ok = q0 + r < N;
      const int rr = ok ? q0 + r : 0;
      qr[it] = ld16(reinterpret_cast<const char*>(qg + (size_t)rr * D) + cc * 16);
      dr[it] = ld16(reinterpret_cast<const char*>(dog + (size_t)rr * D) + cc * 16);
      if (!ok) {
        qr[it] = i32x4{0, 0, 0, 0};
        dr[it] = i32x4{0, 0, 0, 0};
      }
    }
    if (tid < BR) {
      const int i = q0 + tid;
      lr = i < N ? lseg[i] : INFINITY;
      ddr = i < N ? ddg[i] : 0.f;
    }
  };
  auto stash = [&](int buf) {
    char* qb = reinterpret_cast<char*>(q_lds + buf * BR * D);
    char* db_ = reinterpret_cast<char*>(do_lds + buf * BR * D);
#pragma unroll
    for (int it = 0; it < CH; ++it) {
      const int c = it * Tr::NT + tid;
      const int r = c / CPR, cc = c % CPR;
      st16(qb + swz_off<D>(r, cc * 8), qr[it]);
      st16(db_ + swz_off<D>(r, cc * 8), dr[it]);
    }
    if (tid < BR) {
      // a row without any unmasked key has lse = -inf; +inf makes exp(S - lse) = 0 for it
      const float l = (lr == -INFINITY) ? INFINITY : lr;
      lse_lds[buf][tid] = l * LOG2E;
      dd_lds[buf][tid] = ddr;
    }
  };

  TileWindow win = empty_window();
  int qt = next_live_tile(win, qt_begin, nq, class_of, lane);
  if (qt < nq) fetch(qt);
  int buf = 0;

  while (qt < nq) {
    const int q0 = qt * BR;
    const bool need_mask = window_partial(win, qt) || (q0 + BR > N) || (c0 + BC > N);
    stash(buf);
    __syncthreads();  // (A) the tile is in LDS; every wave is past the previous tile's reads
    const int qt_next = next_live_tile(win, qt + 1, nq, class_of, lane);
    if (qt_next < nq) fetch(qt_next);

    const bf16* qb = q_lds + buf * BR * D;
    const bf16* dob = do_lds + buf * BR * D;
    const bf16* xb = role == 0 ? qb : dob;

    // Phase 1: role 0 forms S and P, role 1 forms dP (rows = query rows, columns = this lane's keys).
    f32x16 x[2];
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
      x[ib] = zero16();
#pragma unroll
      for (int c = 0; c < Tr::NKF; ++c)
        x[ib] = M::mma(swz_kcontig<D>(xb, ib * 32 + l32, c * 16 + g * 8), xf[c], x[ib]);
    }
    bf16x4 pv[2][4];  // P (role 0: computed, role 1: read back), register order
    if (role == 0) {
      const uint64_t mbits =
          need_mask ? masked_row_bits(q0, j, N, causal, has_lt, has_ut, m_lts, m_lte, m_uts, m_ute) : 0ull;
      const uint64_t mg = mbits >> (4 * g);
#pragma unroll
      for (int ib = 0; ib < 2; ++ib) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int il0 = ib * 32 + 8 * q4 + 4 * g;
          const f32x4 lse4 = *reinterpret_cast<const f32x4*>(&lse_lds[buf][il0]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float p = __builtin_amdgcn_exp2f(x[ib][4 * q4 + e] * sl2 - lse4[e]);
            p = ((mg >> (ib * 32 + 8 * q4 + e)) & 1) ? 0.f : p;
            pv[ib][q4][e] = (bf16)p;
          }
          *reinterpret_cast<bf16x4*>(p_lds + jl * PS + il0) = pv[ib][q4];
        }
      }
    }
    __syncthreads();  // (B) P is in LDS

    // Phase 2: role 1 reads P, forms dS and writes it; both roles accumulate their half of dV.
    bf16x4 sv[2][4];  // dS, register order
    if (role == 1) {
#pragma unroll
      for (int ib = 0; ib < 2; ++ib) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int il0 = ib * 32 + 8 * q4 + 4 * g;
          pv[ib][q4] = *reinterpret_cast<const bf16x4*>(p_lds + jl * PS + il0);
          const f32x4 dd4 = *reinterpret_cast<const f32x4*>(&dd_lds[buf][il0]);
#pragma unroll
          for (int e = 0; e < 4; ++e) sv[ib][q4][e] = (bf16)((float)pv[ib][q4][e] * (x[ib][4 * q4 + e] - dd4[e]));
          *reinterpret_cast<bf16x4*>(ds_lds + jl * PS + il0) = sv[ib][q4];
        }
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      bf16x8 pf;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pf[e] = pv[t >> 1][2 * (t & 1)][e];
        pf[4 + e] = pv[t >> 1][2 * (t & 1) + 1][e];
      }
#pragma unroll
      for (int hb = 0; hb < Tr::HDB; ++hb)
        dv[hb] = M::mma(swz_kmajor<D>(dob, 0, (db0 + hb) * 32, t, lane), pf, dv[hb]);
    }
    __syncthreads();  // (C) dS is in LDS

    // Phase 3: role 0 reads dS back; both roles accumulate their half of dK; every wave one block of dQ.
    if (role == 0) {
#pragma unroll
      for (int ib = 0; ib < 2; ++ib) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          sv[ib][q4] = *reinterpret_cast<const bf16x4*>(ds_lds + jl * PS + ib * 32 + 8 * q4 + 4 * g);
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      bf16x8 sf;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sf[e] = sv[t >> 1][2 * (t & 1)][e];
        sf[4 + e] = sv[t >> 1][2 * (t & 1) + 1][e];
      }
#pragma unroll
      for (int hb = 0; hb < Tr::HDB; ++hb)
        dk[hb] = M::mma(swz_kmajor<D>(qb, 0, (db0 + hb) * 32, t, lane), sf, dk[hb]);
    }
    if (has_dq) {
      f32x16 acc = zero16();
#pragma unroll
      for (int t = 0; t < BC / 16; ++t)
        acc = M::mma(load_kmajor_frag<bf16>(ds_lds, PS, 0, dq_ib * 32, t, lane), kq[t], acc);
      float* dst = dqg + (size_t)(q0 + dq_ib * 32 + 4 * g) * D + dq_db * 32 + l32;
      if (q0 + BR <= N) {
#pragma unroll
        for (int r = 0; r < 16; ++r) unsafeAtomicAdd(dst + (8 * (r >> 2) + (r & 3)) * D, acc[r] * a.scale);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = q0 + dq_ib * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          if (i < N) unsafeAtomicAdd(dst + (8 * (r >> 2) + (r & 3)) * D, acc[r] * a.scale);
        }
      }
    }
    qt = qt_next;
    buf ^= 1;
  }

  // dK = scale * dK^T, dV = dV^T for this lane's key column and this role's half of d.
  if (j < N) {
    bf16* dkg = static_cast<bf16*>(a.dk) + head + (size_t)j * D;
    bf16* dvg = static_cast<bf16*>(a.dv) + head + (size_t)j * D;
#pragma unroll
    for (int hb = 0; hb < Tr::HDB; ++hb) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = (db0 + hb) * 32 + 8 * q4 + 4 * g;
        bf16x4 wk, wv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          wk[e] = (bf16)(dk[hb][4 * q4 + e] * a.scale);
          wv[e] = (bf16)dv[hb][4 * q4 + e];
        }
        *reinterpret_cast<bf16x4*>(dkg + d0) = wk;
        *reinterpret_cast<bf16x4*>(dvg + d0) = wv;
      }
    }
  }
}

// ------------------------------------------------------------------ 3. dq = accumulator

template <typename T>
__global__ __launch_bounds__(256) void bwd_dq_kernel(const float* __restrict__ acc, T* __restrict__ dq, long n4) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n4) return;
  const f32x4 v = *reinterpret_cast<const f32x4*>(acc + 4 * i);
  if constexpr (sizeof(T) == 2) {
    bf16x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = (bf16)v[e];
    *reinterpret_cast<bf16x4*>(dq + 4 * i) = w;
  } else {
    *reinterpret_cast<f32x4*>(dq + 4 * i) = v;
  }
}

// ------------------------------------------------------------------ host launch

template <typename T, int D>
static hipError_t launch_bwd_t(const void* q, const void* k, const void* v, const void* out, const void* dout,
                               const float* lse, void* dq, void* dk, void* dv, float* dq_acc, float* dd,
                               const int* lts, const int* lte, const int* uts, const int* ute, const int* bounds,
                               int B, int H, int N, int Hm, int causal, float scale, hipStream_t stream) {
  const long rows = (long)B * H * N;
  constexpr int CPR = D * (int)sizeof(T) / 16;
  constexpr int RPB = 256 / CPR;
  hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, stream,
                     static_cast<const T*>(out), static_cast<const T*>(dout), dd, dq_acc, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  BwdArgs a;
  a.q = q; a.k = k; a.v = v; a.dout = dout; a.lse = lse; a.dd = dd; a.dq_acc = dq_acc; a.dk = dk; a.dv = dv;
  a.lts = lts; a.lte = lte; a.uts = uts; a.ute = ute; a.bounds = bounds;
  a.B = B; a.H = H; a.N = N; a.Hm = Hm;
  a.nkt = (N + BwdTraits<T, D>::BC - 1) / BwdTraits<T, D>::BC;
  a.nkb = (N + KBLOCK - 1) / KBLOCK;
  a.causal = causal;
  a.scale = scale;
  a.scale_log2 = scale * LOG2E;
  const long grid = (long)a.nkt * B * H;
  if constexpr (sizeof(T) == 2) {
    hipLaunchKernelGGL((bwd_pair_kernel<D>), dim3((unsigned)grid), dim3(512), 0, stream, a);
  } else {
    hipLaunchKernelGGL((bwd_main_kernel<T, D>), dim3((unsigned)grid), dim3(256), 0, stream, a);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  const long n4 = rows * D / 4;
  hipLaunchKernelGGL((bwd_dq_kernel<T>), dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, stream, dq_acc,
                     static_cast<T*>(dq), n4);
  return hipGetLastError();
}

hipError_t launch_bwd(bool bf16_in, int d, const void* q, const void* k, const void* v, const void* out,
                      const void* dout, const float* lse, void* dq, void* dk, void* dv, float* dq_acc, float* dd,
                      const int* lts, const int* lte, const int* uts, const int* ute, const int* bounds, int B,
                      int H, int N, int Hm, int causal, float scale, hipStream_t stream) {
  if (bf16_in) {
    if (d == 64)
      return launch_bwd_t<bf16, 64>(q, k, v, out, dout, lse, dq, dk, dv, dq_acc, dd, lts, lte, uts, ute, bounds, B, H,
                                    N, Hm, causal, scale, stream);
    return launch_bwd_t<bf16, 128>(q, k, v, out, dout, lse, dq, dk, dv, dq_acc, dd, lts, lte, uts, ute, bounds, B, H,
                                   N, Hm, causal, scale, stream);
  }
  if (d == 64)
    return launch_bwd_t<float, 64>(q, k, v, out, dout, lse, dq, dk, dv, dq_acc, dd, lts, lte, uts, ute, bounds, B, H,
                                   N, Hm, causal, scale, stream);
  return launch_bwd_t<float, 128>(q, k, v, out, dout, lse, dq, dk, dv, dq_acc, dd, lts, lte, uts, ute, bounds, B, H,
                                  N, Hm, causal, scale, stream);
}

}  // namespace fm
