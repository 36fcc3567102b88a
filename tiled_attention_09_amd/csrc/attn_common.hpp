// Building blocks shared by the attention kernels for gfx950 (MI355X): vector
// types, the LDS tile of 64 rows x d with its XOR swizzle, buffer resources,
// the direct HBM/L2 -> LDS tile copy, the half-wave exchange and the
// XCD-aware workgroup order.
//
// LDS tile: 64 rows of d bf16 values, row-major, the 16-byte chunks of row r
// stored at chunk index (c ^ swz(r)).  Row-wise operand reads (16 consecutive
// rows per 16 lanes) and LDS transpose reads (4 rows per half-wave) are then
// free of bank conflicts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace tiledattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;
constexpr int kWaves = 4;
constexpr int kThreads = kWave * kWaves;
constexpr int kBM = 128;          // rows owned by one workgroup (32 per wave)
constexpr int kBN = 64;           // rows per LDS tile
constexpr float kLog2e = 1.44269504088896340736f;
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit data format
constexpr float kLn2 = 0.69314718055994530942f;

#define TA_LDS __attribute__((address_space(3)))

template <int D>
struct Tile {
  // 64 and 128: bf16 rows of Q, K, V.  32: the geometry of the 64-byte rows of
  // FP8 codes at d = 64 (a bf16 row of 32 values is 64 bytes).
  static_assert(D == 32 || D == 64 || D == 128, "row width");
  static constexpr int KS = D / 16;                 // MFMA k-steps over d for S^T
  static constexpr int DB = D / 32;                 // 32-row blocks of O^T
  static constexpr int DCH = D / 8;                 // 16-byte chunks per key row
  static constexpr int BYTES = kBN * D * 2;         // one tile
  static constexpr int LOADS = BYTES / (kThreads * 16);   // 16-byte loads per thread per tile
  static_assert(LOADS * kThreads * 16 == BYTES, "tile split");

  // XOR applied to the chunk index of key row r.  d=128 (16 chunks): bijective
  // on any 16 aligned rows, and rows 4a..4a+3 get 4 different 64-byte groups.
  // d=64 (8 chunks, two rows per 256-byte bank window): bijective on the rows
  // of one parity within 16 rows, and rows 4a, 4a+2 (and 4a+1, 4a+3) get
  // different 64-byte groups.  32 (4 chunks of 16 bytes, four rows per
  // 256-byte bank window): rows r and r + 4 k differ in (r >> 2) & 3, so 16
  // consecutive rows at one chunk index fill 16 different 16-byte slots.
  __device__ static __forceinline__ int swz(int r) {
    if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    else if constexpr (D == 64) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
    else return (r >> 2) & 3;
  }
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kRsrcWord3);
}

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

// Both halves of a wave hold partial results for the same 32 queries; the
// swap (v_permlane32_swap) gives every lane the other half's value without a
// trip through LDS.
__device__ __forceinline__ float other_half(float x) {
  const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false,
                                                   false);
  // lanes 0-31: pr[1] holds lanes 32-63; lanes 32-63: pr[0] holds lanes 0-31
  return __int_as_float((threadIdx.x & 32) ? pr[0] : pr[1]);
}

// Issue-order recipe for a block of NMFMA matrix products fed by LDS reads:
// PRE reads first, then each product followed by up to PER more reads until
// TOTAL reads are placed (group sizes must be compile-time constants, hence the
// expansion over an index sequence).  Keeps PRE / PER products' worth of reads
// in flight instead of waiting on each operand just before its product.
template <int PRE, int PER, int TOTAL, int... I>
__device__ __forceinline__ void sched_mfma_ds(std::integer_sequence<int, I...>) {
  __builtin_amdgcn_sched_group_barrier(0x100, PRE, 0);
  ((__builtin_amdgcn_sched_group_barrier(0x008, 1, 0),
    __builtin_amdgcn_sched_group_barrier(
        0x100, (TOTAL - PRE - PER * I) >= PER ? PER : ((TOTAL - PRE - PER * I) > 0 ? (TOTAL - PRE - PER * I) : 0),
        0)),
   ...);
}

// Like sched_mfma_ds, with V vector instructions placed after each product.
template <int PRE, int PER, int TOTAL, int V, int... I>
__device__ __forceinline__ void sched_mfma_ds_valu(std::integer_sequence<int, I...>) {
  __builtin_amdgcn_sched_group_barrier(0x100, PRE, 0);
  ((__builtin_amdgcn_sched_group_barrier(0x008, 1, 0),
    __builtin_amdgcn_sched_group_barrier(
        0x100, (TOTAL - PRE - PER * I) >= PER ? PER : ((TOTAL - PRE - PER * I) > 0 ? (TOTAL - PRE - PER * I) : 0),
        0),
    __builtin_amdgcn_sched_group_barrier(0x002, V, 0)),
   ...);
}

// Recipe building blocks: a group of R DS reads, and N repetitions of
// (1 MFMA, R DS reads, V VALU instructions); empty groups are skipped.
template <int R>
__device__ __forceinline__ void sched_reads() {
  if (R) __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
}
template <int R, int V>
__device__ __forceinline__ void sched_step() {
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  if (R) __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
  if (V) __builtin_amdgcn_sched_group_barrier(0x002, V, 0);
}
template <int R, int V, int... I>
__device__ __forceinline__ void sched_rep_impl(std::integer_sequence<int, I...>) {
  ((sched_step<R, V>(), (void)I), ...);
}
template <int R, int V, int N>
__device__ __forceinline__ void sched_rep() {
  sched_rep_impl<R, V>(std::make_integer_sequence<int, N>{});
}

// Store a wave's block of 32 rows x W fp32 results held as 32x32 MFMA
// accumulators (acc[db][4 g + e] is row l32, column 32 db + 8 g + 4 hi + e),
// each row scaled by the lane's s, to global rows blk + r W for r < rows.
// Direct stores from that layout would write 32 bytes into each of 32 rows
// per instruction; instead the block goes through the wave's own LDS region
// reg (32 W 4 bytes) -- chunk c of row r at chunk slot c ^ (r mod W/4),
// conflict-free for the row-wise reads -- and is read back row-contiguous,
// so every store instruction writes whole rows (1 KiB).  The region must not
// be in use by any other wave.
template <int W>
__device__ __forceinline__ void store_rows_lds(TA_LDS uint8_t* reg, const f32x16* acc, float s,
                                               float* blk, int rows, int lane) {
  constexpr int CH = W / 4;             // 16-byte chunks per row
  constexpr uint32_t ROW = W * 4;       // bytes per row
  const int l32 = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int db = 0; db < W / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 val = {acc[db][4 * g] * s, acc[db][4 * g + 1] * s, acc[db][4 * g + 2] * s,
                         acc[db][4 * g + 3] * s};
      const int c = 8 * db + 2 * g + hi;  // chunk of columns 32 db + 8 g + 4 hi + [0, 4)
      *reinterpret_cast<TA_LDS f32x4*>(reg + l32 * ROW + ((c ^ (l32 & (CH - 1))) << 4)) = val;
    }
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int k = 0; k < (int)(32 * ROW / 1024); ++k) {
    const uint32_t f = (uint32_t)k * 1024u + (uint32_t)lane * 16u;
    const int r = (int)(f / ROW);
    const int c = (int)((f % ROW) >> 4);
    const f32x4 val =
        *reinterpret_cast<const TA_LDS f32x4*>(reg + r * ROW + ((c ^ (r & (CH - 1))) << 4));
    if (r < rows) *reinterpret_cast<f32x4*>(blk + (size_t)r * W + 4 * c) = val;
  }
  __builtin_amdgcn_wave_barrier();
}

// Workgroup -> (head, row tile).  Workgroups are handed to the 8 XCDs
// round-robin, so block b runs on XCD b % 8; each XCD is given a contiguous
// eighth of the (head, tile) items, so one head's tiles share that XCD's L2.
// With `reverse` the tiles of a head are taken last to first (causal query
// tiles: the last has the most work).  An XCD normally takes its items head
// by head.  When the work per tile changes monotonically with the tile index
// (`monotone`: causal) and a head has fewer tiles than the XCD runs
// workgroups at once (`slots`: 32 CUs times the workgroups per CU), the
// last heads' longest tiles would start near the end of the queue and
// stretch the tail (16 heads of 16 causal query tiles per XCD: a
// list-scheduling makespan 1.26 times the even share), so the XCD then takes
// tile position t of every one of its heads before position t + 1 (measured
// 9 % faster forward, 8 % faster backward at B=8, H=16, N=2048).  With more
// tiles per head both orders schedule evenly, and head by head keeps fewer
// heads' K and V in L2 at once.
__device__ __forceinline__ void map_block(int bid, int bh_count, int n_t, bool reverse,
                                          bool monotone, int slots, int& bh, int& t_out) {
  int t;
  if (monotone && n_t < slots && (bh_count & 7) == 0) {
    const int hc = bh_count >> 3;         // heads per XCD
    const int i = bid >> 3;               // position in this XCD's queue
    bh = (bid & 7) * hc + i % hc;
    t = i / hc;
  } else {
    const int total = bh_count * n_t;
    int j = bid;
    if ((total & 7) == 0) j = (bid & 7) * (total >> 3) + (bid >> 3);
    bh = j / n_t;
    t = j - bh * n_t;
  }
  t_out = reverse ? n_t - 1 - t : t;
}

// Enqueue the copy of row tile j of two matrices (K and V; Q and dO) into one
// LDS stage; the matrices may have different widths DA, DB (64 or 128).  Load
// i of wave w fills bytes [(W i + w) * 1024, +1024) (W waves) of a stage's
// tile, one 16-byte chunk per lane; src_a / src_b hold each lane's offset
// within a tile (tile_src_offsets).  Copies of the two matrices alternate.
template <int DA, int DB>
__device__ __forceinline__ void issue_pair(__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                           const uint32_t* src_a, const uint32_t* src_b, int j,
                                           int wave, TA_LDS uint16_t* da, TA_LDS uint16_t* db) {
  constexpr int LA = Tile<DA>::LOADS, LB = Tile<DB>::LOADS;
  const uint32_t off_a = (uint32_t)j * (uint32_t)Tile<DA>::BYTES;   // scalar
  const uint32_t off_b = (uint32_t)j * (uint32_t)Tile<DB>::BYTES;
#pragma unroll
  for (int i = 0; i < (LA > LB ? LA : LB); ++i) {
    const int dst = (kWaves * i + wave) * 512;   // uint16 elements, wave-uniform
    if (i < LA)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (TA_LDS void*)(da + dst), 16, src_a[i], off_a,
                                               0, 0);
    if (i < LB)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (TA_LDS void*)(db + dst), 16, src_b[i], off_b,
                                               0, 0);
  }
}

// One matrix's row tile j into an LDS stage (same placement as issue_pair).
template <int D>
__device__ __forceinline__ void issue_rows(__amdgpu_buffer_rsrc_t r, const uint32_t* src, int j,
                                           int wave, TA_LDS uint16_t* dst_tile) {
  const uint32_t off = (uint32_t)j * (uint32_t)Tile<D>::BYTES;   // scalar
#pragma unroll
  for (int i = 0; i < Tile<D>::LOADS; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (TA_LDS void*)(dst_tile + (kWaves * i + wave) * 512),
                                             16, src[i], off, 0, 0);
}

template <int D>
__device__ __forceinline__ void issue_tile(__amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr,
                                           const uint32_t* src_off, int j, int wave,
                                           TA_LDS uint16_t* kd, TA_LDS uint16_t* vd) {
  issue_pair<D, D>(kr, vr, src_off, src_off, j, wave, kd, vd);
}

// Per-lane source offsets of issue_tile: LDS chunk p = (W i + w) * 64 + lane
// holds tile row p / DCH, global chunk (p % DCH) ^ swz(row).
template <int D>
__device__ __forceinline__ void tile_src_offsets(uint32_t* src_off, int wave, int lane) {
  using T = Tile<D>;
#pragma unroll
  for (int i = 0; i < T::LOADS; ++i) {
    const int p = (kWaves * i + wave) * 64 + lane;
    const int row = p / T::DCH;
    const int chunk = (p % T::DCH) ^ T::swz(row);
    src_off[i] = (uint32_t)(row * D + chunk * 8) * 2u;
  }
}

// Row-wise MFMA operand read from a swizzled tile: row `row`, 8 values starting
// at column 16 ks + 8 hi (A operand of a 32x32x16 product, k = columns).
template <int D>
__device__ __forceinline__ bf16x8 read_rows(const TA_LDS uint16_t* t, int row, int ks, int hi,
                                            int rswz) {
  return *reinterpret_cast<const TA_LDS bf16x8*>(t + row * D + (((2 * ks + hi) ^ rswz) << 3));
}

// Transposed MFMA operand from a swizzled tile: the 32 columns [32 db, +32) of
// tile rows 16 g + [0, 16) (A operand of a 32x32x16 product whose k runs over
// tile rows).  Two LDS transpose reads (ds_read_b64_tr_b16); each 16-lane group
// receives a 16 (columns) x 4 (rows) block.  Element e of lane l corresponds to
// tile row 16 g + 8 (e / 4) + 4 (l / 32) + e % 4, matching the rows a 32x32
// accumulator block holds in elements 8 (g % 2) + e.
template <int D>
__device__ __forceinline__ bf16x8 read_cols(const TA_LDS uint16_t* t, int g, int db, int row_lo,
                                            int col_lo) {
  s16x4 part[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int row = 16 * g + 8 * r + row_lo;
    const int col = 32 * db + col_lo;
    const int off = row * D + ((((col >> 3) ^ Tile<D>::swz(row)) << 3) | (col & 7));
    part[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((TA_LDS s16x4*)(t + off));
  }
  return __builtin_bit_cast(bf16x8,
                            __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
}

// The same two reads with the addresses split so that only a per-lane XOR with
// a compile-time constant remains: a row's 16-byte chunk index sits in byte
// bits 4.. (below the row bits), the swizzle only mixes chunk bits, and every
// term that varies by whole rows (the 32-row block, the 16-row group g, the
// LDS stage) is a constant the compiler folds into the ds_read offset field.
// This keeps the lane-dependent address registers to KS + 2 DB instead of one
// per (stage, row block, k-step).
template <int D>
struct LdsReader {
  uint32_t rows;      // byte offset of (row l32, chunk hi ^ swz(l32)) in a tile
  uint32_t cols[2];   // byte offset of the transpose-read source for r = 0, 1

  __device__ __forceinline__ LdsReader(int lane) {
    const int l32 = lane & 31, hi = lane >> 5;
    rows = (uint32_t)(l32 * D * 2) | ((uint32_t)(hi ^ Tile<D>::swz(l32)) << 4);
    const int row_lo = 4 * hi + ((lane & 15) >> 2);               // source row within 8
    const int col_lo = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);   // source column within 32
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int row = 8 * r + row_lo;
      cols[r] = (uint32_t)(row * D * 2) |
                ((uint32_t)((col_lo >> 3) ^ Tile<D>::swz(row)) << 4) | (uint32_t)((col_lo & 7) * 2);
    }
  }

  // A operand from rows 32 rb + l32, columns 16 ks + 8 hi + [0, 8).
  __device__ __forceinline__ bf16x8 row_op(const TA_LDS uint16_t* t, int rb, int ks) const {
    const uint32_t off = (uint32_t)(rb * 32 * D * 2) + (rows ^ (uint32_t)(ks << 5));
    return *reinterpret_cast<const TA_LDS bf16x8*>((const TA_LDS char*)t + off);
  }

  // Transposed A operand: columns [32 db, +32) of rows 16 g + [0, 16).
  __device__ __forceinline__ bf16x8 col_op(const TA_LDS uint16_t* t, int g, int db) const {
    s16x4 part[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const uint32_t off = (uint32_t)(g * 16 * D * 2) + (cols[r] ^ (uint32_t)(db << 6));
      part[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (TA_LDS s16x4*)((const TA_LDS char*)t + off));
    }
    return __builtin_bit_cast(bf16x8,
                              __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
  }
};

// A operands of the FP8 score product (v_mfma_scale_f32_32x32x64_f8f6f4) from
// a tile of ROWB-byte rows (ROWB FP8 values: 128 with the geometry and swizzle
// of a bf16 Tile<64>, 64 with that of a Tile<32>): row 32 rb + l32, bytes
// [64 ks + 32 hi, +32) as two 16-byte reads.  Both operands of the product use
// this byte order, so the k order inside the instruction does not matter.
// Chunk indices 4 ks + 2 hi + part have disjoint bits, so the swizzle is one
// per-lane XOR with a compile-time constant.
template <int ROWB>
struct LdsReaderF8 {
  static_assert(ROWB == 64 || ROWB == 128, "FP8 row bytes");
  using TG = Tile<ROWB / 2>;   // the bf16 tile with the same row geometry
  uint32_t rows;
  __device__ __forceinline__ explicit LdsReaderF8(int lane) {
    const int l32 = lane & 31, hi = lane >> 5;
    rows = (uint32_t)(l32 * ROWB) | ((uint32_t)((2 * hi) ^ TG::swz(l32)) << 4);
  }
  __device__ __forceinline__ i32x8 row_op(const TA_LDS uint8_t* t, int rb, int ks) const {
    const TA_LDS char* base = (const TA_LDS char*)t + rb * 32 * ROWB;
    const u32x4 a = *reinterpret_cast<const TA_LDS u32x4*>(base + (rows ^ (uint32_t)((4 * ks) << 4)));
    const u32x4 b = *reinterpret_cast<const TA_LDS u32x4*>(base + (rows ^ (uint32_t)((4 * ks + 1) << 4)));
    return __builtin_bit_cast(i32x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
  }
};

// Philox-4x32 with 10 rounds (Salmon, Moraes, Dror, Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC 2011): counter (c0..c3), key (k0, k1).  Each
// round multiplies words 0 and 2 by the two round constants into 64-bit
// products whose halves are mixed with words 1 and 3 and the key; the key
// advances by two Weyl constants between rounds.
__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                               uint32_t k0, uint32_t k1) {
  constexpr uint32_t kM0 = 0xD2511F53u, kM1 = 0xCD9E8D57u;
  constexpr uint32_t kW0 = 0x9E3779B9u, kW1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += kW0;
      k1 += kW1;
    }
    const uint64_t p0 = (uint64_t)kM0 * c0, p1 = (uint64_t)kM1 * c2;
    // Three-input exclusive or in one instruction (truth table 0x96 = a ^ b ^ c).
    const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
    const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
  }
  return u32x4{c0, c1, c2, c3};
}

// Dropout parameters: key (seed_lo, seed_hi); an element is kept when its
// random byte is >= t (drop probability t / 256); kept values are scaled by
// keep_scale = 256 / (256 - t).  The byte of (query row i, key j) of head n is
// byte j mod 16 (little endian) of the block for counter (i, j / 16, n, 0).
struct DropoutArgs {
  uint32_t seed_lo, seed_hi, t;
  float keep_scale;
};

// Mask words of one 64-key tile for a lane that holds query row `row` and,
// in 32-key block kb of a score accumulator, keys 32 kb + 8 g + 4 hi + e
// (g, e = 0..3): word mw[kb][g] carries those four keys' bytes, e in byte e.
// The two lanes of a row (one per wave half) need disjoint halves of the
// tile's four 16-key blocks: each generates the two blocks of 32-key block
// `hi` and one half-wave swap per word pair trades what the other needs.
__device__ __forceinline__ void dropout_row_words(uint32_t row, uint32_t tile, uint32_t head,
                                                  const DropoutArgs& dr, int hi,
                                                  uint32_t (&mw)[2][4]) {
  const uint32_t blk = 4u * tile + 2u * (uint32_t)hi;
  const u32x4 b0 = philox4x32_10(row, blk, head, 0u, dr.seed_lo, dr.seed_hi);
  const u32x4 b1 = philox4x32_10(row, blk + 1u, head, 0u, dr.seed_lo, dr.seed_hi);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    // Word 2 (g % 2) of block g / 2 serves the lower half (keys 8 g + 0..3),
    // word 2 (g % 2) + 1 the upper half (keys 8 g + 4..7).  After the swap
    // the first result holds block kb = 0's word for this lane, the second
    // block kb = 1's.
    const uint32_t lo = (g >> 1) ? b1[2 * (g & 1)] : b0[2 * (g & 1)];
    const uint32_t up = (g >> 1) ? b1[2 * (g & 1) + 1] : b0[2 * (g & 1) + 1];
    const auto pr = __builtin_amdgcn_permlane32_swap(lo, up, false, false);
    mw[0][g] = pr[0];
    mw[1][g] = pr[1];
  }
}

// Keep test of element (kb, i) of a score accumulator pair (key
// 32 kb + 8 (i / 4) + 4 hi + i % 4) with the words of dropout_row_words.
__device__ __forceinline__ bool dropout_keep(const uint32_t (&mw)[2][4], int kb, int i,
                                             uint32_t t) {
  return ((mw[kb][i >> 2] >> (8 * (i & 3))) & 0xffu) >= t;
}

}  // namespace tiledattn
