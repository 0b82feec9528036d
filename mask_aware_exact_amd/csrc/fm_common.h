// Device helpers shared by the column-wise-mask attention kernels (gfx950 / CDNA4 only).
//
// Matrix-core conventions used throughout (measured on MI355X):
//  * v_mfma_f32_32x32x16_bf16: operand A row = lane % 32, operand B column = lane % 32; the 8 slots of
//    lanes 0-31 and of lanes 32-63 cover the 16 k values, identically for A and B.
//  * accumulator: lane l, register r holds C[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].
//  * v_mfma_f32_32x32x2_f32: A row / B column = lane % 32, k = lane / 32, same accumulator layout.
//  * ds_read_b64_tr_b16 over 16-lane groups: if lane s of a group addresses row k0 + s / 4, columns
//    4 (s % 4) .. +3 of a row-major 16-bit tile, lane t of the group receives column t, rows k0 .. k0+3.
//
// An accumulator used as the k operand of the next product keeps its register order: slot s of
// product t reads register r = t * E + s, i.e. k index 8 (r / 4) + 4 (l / 32) + r % 4. The other
// operand of such a product is read from LDS in the same k order (see load_kmajor_frag).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fm_launch.h"

namespace fm {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int KBLOCK = 64;  // key columns per bounds entry
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// A compile-time flag passed as an argument (selects a variant of a generic lambda).
template <bool V>
struct Flag {
  static constexpr bool value = V;
};

enum TileClass : int { CLS_NONE = 0, CLS_PARTIAL = 1, CLS_FULL = 2 };

// Per-key-tile bounds (min/max of each of LTS, LTE, UTS, UTE over the tile's columns). Named fields
// rather than an int[8]: a private array that is indexed in a loop may be placed in LDS by the compiler
// (one 32-byte slot per thread), and every read of it then hits the same few banks.
struct TileBounds {
  int lts_min, lts_max, lte_min, lte_max, uts_min, uts_max, ute_min, ute_max;
};

// Tile rule: rows [r0, r1), columns [c0, c1), both already clipped to N.
__device__ __host__ inline int classify_tile(int r0, int r1, int c0, int c1, const TileBounds& b, bool causal) {
  const bool causal_full = causal && (r1 - 1 < c0);
  const bool causal_none = !causal || (r0 >= c1 - 1);
  const bool lt_full = (r0 >= b.lts_max) && (r1 <= b.lte_min);
  const bool lt_none = (r1 <= b.lts_min) || (r0 >= b.lte_max);
  const bool ut_full = (r0 >= b.uts_max) && (r1 <= b.ute_min);
  const bool ut_none = (r1 <= b.uts_min) || (r0 >= b.ute_max);
  if (causal_full || lt_full || ut_full) return CLS_FULL;
  if (causal_none && lt_none && ut_none) return CLS_NONE;
  return CLS_PARTIAL;
}

// Bounds of key tiles [kt0, kt1) of one (b, hm) row merged by min/max; canonical empties when the
// bounds array is absent (all vectors absent).
__device__ inline TileBounds merged_bounds(const int* __restrict__ brow, int kt0, int kt1, int N) {
  TileBounds r;
  if (brow == nullptr) {
    r.lts_min = r.lts_max = r.lte_min = r.lte_max = N;
    r.uts_min = r.uts_max = r.ute_min = r.ute_max = 0;
    return r;
  }
  const int* p = brow + (size_t)kt0 * 8;
  r = TileBounds{p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]};
  for (int t = kt0 + 1; t < kt1; ++t) {
    const int* q = brow + (size_t)t * 8;
    r.lts_min = min(r.lts_min, q[0]);
    r.lts_max = max(r.lts_max, q[1]);
    r.lte_min = min(r.lte_min, q[2]);
    r.lte_max = max(r.lte_max, q[3]);
    r.uts_min = min(r.uts_min, q[4]);
    r.uts_max = max(r.uts_max, q[5]);
    r.ute_min = min(r.ute_min, q[6]);
    r.ute_max = max(r.ute_max, q[7]);
  }
  return r;
}

// Whether head (bh) with mask row mrow has its dS tiles stored: its region fits in the first `cap` slots.
__device__ __forceinline__ bool ds_head_stored(const DsPlan& p, long long cap, int bh, long long mrow) {
  const long long r = p.region[bh], t = p.rowtotal[mrow];
  return r >= 0 && t >= 0 && r <= cap - t;
}

// Slots of key tile kt inside its head's region: [lo, lo + span) with span returned. A plan whose entries
// are inconsistent gives span 0, so that a plan that does not belong to the problem can give wrong
// results but never an access outside the head's region.
__device__ __forceinline__ long long ds_tile_span(const DsPlan& p, long long mrow, int kt, long long& lo) {
  const long long e = mrow * p.nkt + kt;
  const long long t = p.rowtotal[mrow];
  const long long b0 = p.base[e];
  const long long b1 = kt + 1 < p.nkt ? p.base[e + 1] : t;
  lo = b0;
  return (b0 >= 0 && b1 >= b0 && b1 <= t) ? b1 - b0 : 0;
}

// Rows of a query work unit (forward, dq) and columns of a key work unit (dk, dv): the granule of the
// dispatch schedule.
constexpr int SCHED_UNIT = 128;

// Work unit of the workgroup at dispatch position `rank`: entry rank of the (b, hm) mask row `mrow` of a
// longest-first schedule (order at offset `off` of a row of `stride` int32), or `fallback` without a
// schedule. A scheduled value outside [0, n) gives -1: the workgroup does nothing, so a schedule that does
// not belong to the problem can give wrong results but never out-of-range accesses.
__device__ __forceinline__ int scheduled_unit(const int* __restrict__ sched, int stride, size_t mrow, int off,
                                              int rank, int n, int fallback) {
  if (sched == nullptr) return fallback;
  const int u = sched[mrow * stride + off + rank];
  return (u >= 0 && u < n) ? u : -1;
}

// Live-tile window over 64 consecutive tiles: bit t of `live` / `partial` describes tile base + t.
// One wave-wide ballot classifies 64 tiles at once; every wave of a workgroup computes the same window.
struct TileWindow {
  int base;
  uint64_t live;
  uint64_t partial;
};

template <typename ClassOf>
__device__ __forceinline__ TileWindow scan_window(int base, int end, ClassOf class_of, int lane) {
  TileWindow w;
  w.base = base;
  const int t = base + lane;
  const int cls = t < end ? class_of(t) : (int)CLS_FULL;
  w.live = __ballot(cls != CLS_FULL);
  w.partial = __ballot(cls == CLS_PARTIAL);
  return w;
}

// Next live tile at or after `from` (refilling the window as needed), or `end` when none is left.
template <typename ClassOf>
__device__ __forceinline__ int next_live_tile(TileWindow& w, int from, int end, ClassOf class_of, int lane) {
  while (from < end) {
    if (from >= w.base + 64) w = scan_window(from, end, class_of, lane);
    const uint64_t rest = w.live >> (from - w.base);
    if (rest != 0) return from + __builtin_ctzll(rest);
    from = w.base + 64;
  }
  return end;
}

__device__ __forceinline__ TileWindow empty_window() {
  TileWindow w;
  w.base = -64;
  w.live = 0;
  w.partial = 0;
  return w;
}

__device__ __forceinline__ bool window_partial(const TileWindow& w, int t) { return (w.partial >> (t - w.base)) & 1; }

// Whether query row i is masked for a key column with the given vector values. Bitwise operators
// only, so that the compiler emits selects rather than branches.
__device__ __forceinline__ bool masked_elem(int i, int j, bool causal, bool has_lt, bool has_ut, int lts,
                                            int lte, int uts, int ute) {
  return (causal & (i < j)) | (has_lt & (lts <= i) & (i < lte)) | (has_ut & (uts <= i) & (i < ute));
}

// Bits of the query rows [s, e) that fall in [q0, q0 + 64), bit k standing for row q0 + k.
__device__ __forceinline__ uint64_t row_span_bits(int s, int e, int q0) {
  // s and e are clamped into [q0, q0 + 64] before any difference, so no vector value can overflow it
  const int a = min(max(s, q0), q0 + 64) - q0;
  const int z = min(max(e, q0), q0 + 64) - q0;
  const uint64_t below_z = z >= 64 ? ~0ull : (1ull << z) - 1;
  const uint64_t below_a = a >= 64 ? ~0ull : (1ull << a) - 1;
  return below_z & ~below_a;
}

// Masked rows among q0 .. q0 + 63 for key column j. Rows are global query indices (the mask's own
// coordinates); rows at or past row_end and columns at or past nk count as masked.
__device__ __forceinline__ uint64_t masked_row_bits(int q0, int j, int row_end, int nk, bool causal, bool has_lt,
                                                    bool has_ut, int lts, int lte, int uts, int ute) {
  uint64_t m = row_span_bits(row_end, 0x7fffffff, q0);
  m |= causal ? row_span_bits(0, j, q0) : 0ull;
  m |= has_lt ? row_span_bits(lts, lte, q0) : 0ull;
  m |= has_ut ? row_span_bits(uts, ute, q0) : 0ull;
  return j >= nk ? ~0ull : m;
}

// The same for the 32 rows q0 .. q0 + 31.
__device__ __forceinline__ uint32_t row_span_bits32(int s, int e, int q0) {
  const int a = min(max(s, q0), q0 + 32) - q0;
  const int z = min(max(e, q0), q0 + 32) - q0;
  const uint32_t below_z = z >= 32 ? ~0u : (1u << z) - 1;
  const uint32_t below_a = a >= 32 ? ~0u : (1u << a) - 1;
  return below_z & ~below_a;
}

__device__ __forceinline__ uint32_t masked_row_bits32(int q0, int j, int row_end, int nk, bool causal, bool has_lt,
                                                      bool has_ut, int lts, int lte, int uts, int ute) {
  uint32_t m = row_span_bits32(row_end, 0x7fffffff, q0);
  m |= causal ? row_span_bits32(0, j, q0) : 0u;
  m |= has_lt ? row_span_bits32(lts, lte, q0) : 0u;
  m |= has_ut ? row_span_bits32(uts, ute, q0) : 0u;
  return j >= nk ? ~0u : m;
}

// Masks of a tile of BCOLS keys (64 or 128) in the S^T layout (rows = keys in 32-key blocks, columns =
// a wave's 32 query rows, one row per lane): lane c forms the masked-row word of key columns c0 + c
// (+ 64, ...) for the rows q0 .. q0 + 31 and stores it in the wave's own BCOLS-word LDS row; the wave then
// reads back the words of the columns its registers hold. LDS operations of one wave run in order, and
// the wave-scope fences keep the compiler from moving the read-back above the store. `vec` holds the
// tile's vectors as int [4][BCOLS]: LTS, LTE, UTS, UTE of its columns.
template <int BCOLS = 64>
__device__ __forceinline__ void tile_column_words(uint32_t* cw, const int* vec, int q0, int c0, int row_end, int nk,
                                                  bool causal, bool has_lt, bool has_ut, int lane) {
  // 64 columns written out as one pass: the loop form of the same arithmetic gives the forward kernel a
  // different instruction schedule
  if constexpr (BCOLS == 64) {
    const int lts = has_lt ? vec[lane] : 0, lte = has_lt ? vec[64 + lane] : 0;
    const int uts = has_ut ? vec[128 + lane] : 0, ute = has_ut ? vec[192 + lane] : 0;
    cw[lane] = masked_row_bits32(q0, c0 + lane, row_end, nk, causal, has_lt, has_ut, lts, lte, uts, ute);
  } else {
#pragma unroll
    for (int h = 0; h < BCOLS / 64; ++h) {
      const int c = 64 * h + lane;
      const int lts = has_lt ? vec[c] : 0, lte = has_lt ? vec[BCOLS + c] : 0;
      const int uts = has_ut ? vec[2 * BCOLS + c] : 0, ute = has_ut ? vec[3 * BCOLS + c] : 0;
      cw[c] = masked_row_bits32(q0, c0 + c, row_end, nk, causal, has_lt, has_ut, lts, lte, uts, ute);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Words of the four key columns 32 jb + 8 q4 + 4 g + e (e = 0..3) held by accumulator registers
// 4 q4 .. 4 q4 + 3 of block jb.
__device__ __forceinline__ i32x4 column_words4(const uint32_t* cw, int jb, int q4, int g) {
  return *reinterpret_cast<const i32x4*>(cw + jb * 32 + 8 * q4 + 4 * g);
}

// All ones when bit `row_bit` of the word is set (the lane's row is masked), else zero.
__device__ __forceinline__ int row_mask_of(int word, int row_bit) { return (int)((uint32_t)word << (31 - row_bit)) >> 31; }

// -inf where the given all-ones / all-zeros word is set, x elsewhere.
__device__ __forceinline__ float select_neg_inf(int all_ones_if_masked, float x) {
  const uint32_t m = (uint32_t)all_ones_if_masked;
  return __uint_as_float((__float_as_uint(x) & ~m) | (0xff800000u & m));
}

// Max / sum over the lane pair (l, l ^ 32), the same value on both lanes, without an LDS round trip:
// v_permlane32_swap with both operands x leaves lane (l & 31)'s x in the first result and lane
// (l & 31) + 32's in the second, on every lane (checked on the MI355X).
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ------------------------------------------------------------------ matrix-core traits

template <typename T>
struct MM;

template <>
struct MM<bf16> {
  static constexpr int E = 8;    // operand elements per lane
  static constexpr int KW = 16;  // k extent of one instruction
  using frag = bf16x8;
  static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <>
struct MM<float> {
  static constexpr int E = 1;
  static constexpr int KW = 2;
  using frag = float;
  static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int r = 0; r < 16; ++r) z[r] = 0.f;
  return z;
}

// E contiguous elements along k (the contiguous axis) at p: a k-contiguous operand fragment.
template <typename T>
__device__ __forceinline__ typename MM<T>::frag load_kcontig_frag(const T* p) {
  return *reinterpret_cast<const typename MM<T>::frag*>(p);
}

// Operand fragment of product t whose k axis runs along the ROWS of a row-major LDS tile (pitch in
// elements) and whose m/n index (lane % 32) runs along its columns starting at col0. k index of slot s
// follows the accumulator register order (r = t * E + s -> 8 (r / 4) + 4 (lane / 32) + r % 4), offset by
// row0. bf16 uses two transposing LDS reads; float reads one element.
template <typename T>
__device__ __forceinline__ typename MM<T>::frag load_kmajor_frag(const T* tile, int pitch, int row0, int col0,
                                                               int t, int lane);

template <>
__device__ __forceinline__ bf16x8 load_kmajor_frag<bf16>(const bf16* tile, int pitch, int row0, int col0, int t,
                                                        int lane) {
  const int g = lane >> 5;
  const int s = lane & 15;
  const int col = col0 + (lane & 16) + 4 * (s & 3);
  const int row = row0 + 16 * t + 4 * g + (s >> 2);
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(tile + row * pitch + col));
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(tile + (row + 8) * pitch + col));
  bf16x8 f;
  f[0] = lo[0]; f[1] = lo[1]; f[2] = lo[2]; f[3] = lo[3];
  f[4] = hi[0]; f[5] = hi[1]; f[6] = hi[2]; f[7] = hi[3];
  return f;
}

template <>
__device__ __forceinline__ float load_kmajor_frag<float>(const float* tile, int pitch, int row0, int col0, int t,
                                                        int lane) {
  const int g = lane >> 5;
  const int row = row0 + 8 * (t >> 2) + 4 * g + (t & 3);
  return tile[row * pitch + col0 + (lane & 31)];
}

// Fragment of product t taken from an accumulator (registers t * E .. t * E + E - 1), rounded to T.
template <typename T>
__device__ __forceinline__ typename MM<T>::frag acc_frag(const f32x16& acc, int t);

template <>
__device__ __forceinline__ bf16x8 acc_frag<bf16>(const f32x16& acc, int t) {
  bf16x8 f;
#pragma unroll
  for (int s = 0; s < 8; ++s) f[s] = (bf16)acc[8 * t + s];
  return f;
}

template <>
__device__ __forceinline__ float acc_frag<float>(const f32x16& acc, int t) {
  return acc[t];
}

// Scheduling hint for a block of NM matrix products fed by NR LDS reads: LEAD reads first, then each
// product followed by its share of the remaining reads, so that the reads stay a few products ahead
// instead of being issued all at once. Must sit at the end of the block (same basic block).
template <int NM, int NR, int LEAD>
__device__ __forceinline__ void interleave_reads() {
  __builtin_amdgcn_sched_group_barrier(0x100, LEAD, 0);
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, (NR - LEAD + NM - 1) / NM, 0);
  }
}

// ------------------------------------------------------------------ swizzled bf16 tiles
// A bf16 tile with rows of D elements (D * 2 bytes, unpadded) stores 16-byte chunk c of row r at chunk
// position c ^ swz_key<D>(r). With 64 LDS banks of 4 bytes this makes both access patterns of the kernels
// conflict-free: 16 lanes reading the same chunk of 16 consecutive rows (operand fragments with k along
// the row), and 32 lanes reading 64 bytes of 4 consecutive rows (transposing reads, k along the rows).
template <int D>
__device__ __forceinline__ int swz_key(int r) {
  static_assert(D == 64 || D == 128, "swizzled tiles are defined for 64 and 128 columns");
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// Byte offset of element `col` (a multiple of 4) of row r in a swizzled tile.
template <int D>
__device__ __forceinline__ int swz_off(int r, int col) {
  return r * (D * 2) + (((col >> 3) ^ swz_key<D>(r)) << 4) + ((col & 7) << 1);
}

// Precomputed per-lane byte offsets for the two read patterns of a swizzled tile. Because swz_key
// depends only on the low four row bits, moving by 32 rows (row reads) or 16 rows (transposing reads)
// keeps every offset, so the loops add compile-time row strides to a handful of lane constants.
template <int D>
struct SwzRowReads {  // operand with k along the row: lane reads row rb * 32 + lane % 32, chunk 2 c + lane / 32
  int off[D / 16];
  __device__ __forceinline__ void init(int lane) {
    const int r = lane & 31, g = lane >> 5;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) off[c] = swz_off<D>(r, c * 16 + g * 8);
  }
  __device__ __forceinline__ bf16x8 read(const bf16* tile, int rb, int c) const {
    return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(tile) + rb * 32 * (D * 2) + off[c]);
  }
};

// SwzColReads<D, NB> covers the NB 32-column blocks db_first .. db_first + NB - 1 (db_first may be a run-time
// value); read() takes the block's index within that range and must be given compile-time indices, so
// that the offsets stay in registers (a dynamically indexed private array may be placed in LDS).
template <int D, int NB = D / 32>
struct SwzColReads {  // operand with k along the rows (the load_kmajor_frag pattern), one 32-column block db
  int lo[NB], hi[NB];
  __device__ __forceinline__ void init(int lane, int db_first = 0) {
    const int g = lane >> 5, s = lane & 15;
    const int row = 4 * g + (s >> 2);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int col = (db_first + i) * 32 + (lane & 16) + 4 * (s & 3);
      lo[i] = swz_off<D>(row, col);
      hi[i] = swz_off<D>(row + 8, col);
    }
  }
  __device__ __forceinline__ bf16x8 read(const bf16* tile, int t, int db) const {
    typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
    const char* base = reinterpret_cast<const char*>(tile) + t * 16 * (D * 2);
    const bf16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base + lo[db]));
    const bf16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base + hi[db]));
    bf16x8 f;
    f[0] = x[0]; f[1] = x[1]; f[2] = x[2]; f[3] = x[3];
    f[4] = y[0]; f[5] = y[1]; f[6] = y[2]; f[7] = y[3];
    return f;
  }
};

// One direct global-to-LDS copy instruction: each lane fetches 16 bytes from gbase + voff and the wave
// writes them lane-linearly at LDS byte address lds (wave-uniform). Issued as inline assembly: the
// compiler's wait-count pass models the builtin as a store to an unknown LDS location and would then
// wait for every copy in flight before any later LDS read, which serialises each prefetch with the
// compute it should overlap. Callers wait themselves (s_waitcnt vmcnt(0) and a barrier) before reading
// the tile; the compiler only ever over-waits for its own loads because of these untracked ones.
__device__ __forceinline__ void lds_copy16(const void* gbase, uint32_t voff, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(gbase), "{m0}"(lds) : "memory");
}

// lds_copy16 for data read once (streaming): the non-temporal hint keeps it from displacing reused lines.
__device__ __forceinline__ void lds_copy16_nt(const void* gbase, uint32_t voff, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(gbase), "{m0}"(lds) : "memory");
}

// Direct global-to-LDS load of 4 bytes per lane (256 bytes per wave instruction, lane-linear at `lds`).
__device__ __forceinline__ void lds_copy4(const void* gbase, uint32_t voff, uint32_t lds) {
  asm volatile("global_load_lds_dword %0, %1" ::"v"(voff), "s"(gbase), "{m0}"(lds) : "memory");
}

// LDS byte address of a pointer into shared memory, made wave-uniform.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p);
}

// Asynchronous copy of rows [row0, row0 + ROWS) of a [*, D] bf16 matrix into a swizzled LDS tile with
// direct global-to-LDS loads: each wave instruction moves 1 KB (16 bytes per lane, written lane-linearly
// at the instruction's LDS address), and lane l of the instruction fetches the global chunk that the
// swizzle places at its position. Rows at or past nrows read row nrows - 1 (finite data the kernels
// mask). NW waves take part. The caller waits with s_waitcnt vmcnt(0) and a barrier before reading.
template <int D, int ROWS, int NW>
__device__ __forceinline__ void copy_tile_async(bf16* tile, const bf16* __restrict__ g, int row0, int nrows,
                                                int wave, int lane) {
  constexpr int RB = D * 2;        // bytes per row
  constexpr int RPI = 1024 / RB;   // rows per instruction
  constexpr int NI = ROWS / RPI;   // instructions per tile
  constexpr int CPW = RB / 16;     // 16-byte chunks per row
  static_assert(ROWS % RPI == 0 && NI % NW == 0, "the tile must split evenly over the waves");
  // A wave's instructions step NW * RPI rows, a multiple of 16, so the swizzle key (a function of the
  // row's low four bits) and hence the lane's source chunk stay the same for all of them.
  static_assert((NW * RPI) % 16 == 0, "the swizzle key of a lane's row must not change between instructions");
  const int rl = wave * RPI + lane / CPW;                            // lane's row for the first instruction
  const int col = ((lane % CPW) ^ swz_key<D>(rl)) << 4;              // byte offset of its chunk in the row
  const char* gb = reinterpret_cast<const char*>(g + (size_t)row0 * D);  // uniform
  const int lim = nrows - 1 - row0;                                   // last valid row of the tile
  const uint32_t lds0 = lds_addr(tile) + (uint32_t)__builtin_amdgcn_readfirstlane(wave) * 1024u;
  if (lim >= ROWS - 1) {
    // whole tile in range: uniform base plus a constant 32-bit lane offset per instruction
    const uint32_t off = (uint32_t)(rl * RB + col);
#pragma unroll
    for (int k = 0; k < NI / NW; ++k) lds_copy16(gb + k * NW * RPI * RB, off, lds0 + k * NW * 1024);
  } else {
    // ragged last tile: rows past nrows read row nrows - 1 (finite data the kernels mask)
#pragma unroll
    for (int k = 0; k < NI / NW; ++k) {
      const uint32_t off = (uint32_t)(min(rl + k * NW * RPI, lim) * RB + col);
      lds_copy16(gb, off, lds0 + k * NW * 1024);
    }
  }
}

// Direct global-to-LDS copy of the 64 columns c0 .. c0 + 63 of one mask vector row into dst[64]; columns
// at or past n read column n - 1 (the kernels mask columns past n). `row` must be wave-uniform.
__device__ __forceinline__ void copy_vector_slice(int* dst, const int* row, int c0, int n, int lane) {
  lds_copy4(row, (uint32_t)min(c0 + lane, n - 1) * 4u, lds_addr(dst));
}

// One wave per vector: wave w of the first four copies LTS, LTE, UTS, UTE (as present) of the BCOLS columns
// from c0 into vec[w][BCOLS], 64 columns per instruction. `w` must be wave-uniform.
template <int BCOLS = 64>
__device__ __forceinline__ void copy_tile_vectors(int (*vec)[BCOLS], const int* lts, const int* lte, const int* uts,
                                                  const int* ute, size_t vrow, int c0, int n, int w, int lane) {
  const int* src = w == 0 ? lts : w == 1 ? lte : w == 2 ? uts : ute;
  if constexpr (BCOLS == 64) {
    if (w < 4 && src != nullptr) copy_vector_slice(vec[w], src + vrow, c0, n, lane);
  } else {
    if (w < 4 && src != nullptr) {
#pragma unroll
      for (int h = 0; h < BCOLS / 64; ++h) copy_vector_slice(vec[w] + 64 * h, src + vrow, c0 + 64 * h, n, lane);
    }
  }
}

// The same copy as copy_tile_async, split into this wave's instructions so that the caller can spread
// them between matrix products: prep() computes the addresses, issue(k) sends instruction k (k a
// compile-time value after unrolling). Every lane's offset is clamped to its chunk of row nrows - 1,
// which covers the ragged last tile without a branch.
template <int D, int ROWS, int NW>
struct TileCopy {
  static constexpr int RB = D * 2;
  static constexpr int RPI = 1024 / RB;
  static constexpr int NI = ROWS / RPI;
  static constexpr int NK = NI / NW;  // instructions per wave
  static constexpr int CPW = RB / 16;
  static constexpr uint32_t STEP = NW * RPI * RB;
  static_assert(ROWS % RPI == 0 && NI % NW == 0, "the tile must split evenly over the waves");
  static_assert((NW * RPI) % 16 == 0, "the swizzle key of a lane's row must not change between instructions");
  const char* gb;  // wave-uniform: the tile's first row
  uint32_t lds0;   // wave-uniform: LDS address of this wave's first instruction
  uint32_t off0;   // lane: byte offset of its chunk for instruction 0
  uint32_t lim;    // lane: byte offset of the same chunk position in row nrows - 1
  __device__ __forceinline__ void prep(bf16* tile, const bf16* __restrict__ g, int row0, int nrows, int wave,
                                       int lane) {
    prep_at(lds_addr(tile), g, row0, nrows, wave, lane);
  }
  // The same with the tile's LDS byte address given (wave-uniform).
  __device__ __forceinline__ void prep_at(uint32_t tile_lds, const bf16* __restrict__ g, int row0, int nrows, int wave,
                                          int lane) {
    const int rl = wave * RPI + lane / CPW;
    const int col = ((lane % CPW) ^ swz_key<D>(rl)) << 4;
    gb = reinterpret_cast<const char*>(g + (size_t)row0 * D);
    lds0 = tile_lds + (uint32_t)__builtin_amdgcn_readfirstlane(wave) * 1024u;
    off0 = (uint32_t)(rl * RB + col);
    lim = (uint32_t)((nrows - 1 - row0) * RB + col);
  }
  __device__ __forceinline__ void issue(int k) const {
    lds_copy16(gb, min(off0 + (uint32_t)k * STEP, lim), lds0 + (uint32_t)k * (NW * 1024u));
  }
  // Instruction k of the same copy for another matrix of the same shape and rows (its own tile base and
  // LDS address, same lane offsets).
  __device__ __forceinline__ void issue_to(const char* gb2, uint32_t lds2, int k) const {
    lds_copy16(gb2, min(off0 + (uint32_t)k * STEP, lim), lds2 + (uint32_t)k * (NW * 1024u));
  }
};

// 16-byte global/LDS copy helpers.
__device__ __forceinline__ i32x4 ld16(const void* p) { return *reinterpret_cast<const i32x4*>(p); }
__device__ __forceinline__ void st16(void* p, i32x4 v) { *reinterpret_cast<i32x4*>(p) = v; }

// Copy rows [row0, row0 + ROWS) of a [*, D] row-major global matrix into an LDS tile of pitch PITCH
// elements, zero-filling rows at or past nrows. All NT threads of the block take part.
template <typename T, int ROWS, int D, int PITCH, int NT>
__device__ __forceinline__ void load_tile(T* lds, const T* __restrict__ g, int row0, int nrows, int tid) {
  constexpr int CHUNKS_PER_ROW = D * (int)sizeof(T) / 16;
  constexpr int TOTAL = ROWS * CHUNKS_PER_ROW;
  static_assert(TOTAL % NT == 0, "tile copy must divide evenly");
#pragma unroll
  for (int it = 0; it < TOTAL / NT; ++it) {
    const int c = it * NT + tid;
    const int r = c / CHUNKS_PER_ROW;
    const int cc = c % CHUNKS_PER_ROW;
    i32x4 v = {0, 0, 0, 0};
    if (row0 + r < nrows) v = ld16(reinterpret_cast<const char*>(g + (size_t)(row0 + r) * D) + cc * 16);
    st16(reinterpret_cast<char*>(lds + r * PITCH) + cc * 16, v);
  }
}


// Output rows of one wave, from accumulators in the matrix-core layout (lane l: row l % 32; register r of
// block db: column 32 db + 8 (r / 4) + 4 (l / 32) + r % 4) to a row-major [*, D] bf16 tensor. Stored
// directly, each store instruction writes 8 bytes into each of 32 rows, which costs one memory request per
// 16 bytes. Staged instead through a wave-private LDS area of 32 rows (16-byte chunks XOR-swizzled by row,
// conflict-free reads), each instruction writes 16 contiguous bytes per lane and whole rows per wave.
// `mul` scales the lane's own row; rows at or past `nrows` are not stored. `stage` must hold 32 * D bf16
// (16-byte aligned) that no other wave touches until this returns.
template <int D>
__device__ __forceinline__ void store_rows_staged(char* stage, const f32x16 (&acc)[D / 32], float mul,
                                                  bf16* dst, int nrows, int lane) {
  constexpr int CH = D / 8;        // 16-byte chunks per row
  constexpr int RPI = 64 / CH;     // rows per read instruction
  const int g = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      bf16x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = (bf16)(acc[db][4 * q4 + e] * mul);
      const int c = (4 * db + q4) ^ (l32 & (CH - 1));
      *reinterpret_cast<bf16x4*>(stage + l32 * (D * 2) + c * 16 + g * 8) = w;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int c = lane % CH;
#pragma unroll
  for (int it = 0; it < 32 / RPI; ++it) {
    const int rr = it * RPI + lane / CH;
    const i32x4 v = *reinterpret_cast<const i32x4*>(stage + rr * (D * 2) + ((c ^ (rr & (CH - 1))) * 16));
    if (rr < nrows) *reinterpret_cast<i32x4*>(reinterpret_cast<char*>(dst) + (size_t)rr * (D * 2) + c * 16) = v;
  }
}

}  // namespace fm
