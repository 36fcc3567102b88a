// Attention backward for gfx950 (MI355X): recomputing probabilities from the
// saved per-row log-normaliser, never storing the N x N score matrix.
//
// Method (page "22. GPU Engineering: Correctness, Throughput, and Attention",
// sec. 22.5 and the derivation of sec. 22.7).  With G = dL/dO:
//   dV = P^T G,   dP = G V^T,   dS = P * (dP - D),   D_i = sum_c G[i,c] O[i,c]
//   dQ = scale dS K,   dK = scale dS^T Q,
// where D replaces the row sum of dP * P by the identity the page derives, and
// each block of P is rebuilt as exp(S - LSE).  Base-2 exponentials: with
// c = scale log2(e) and LSE2 = LSE log2(e), P = 2^(c (q.k) - LSE2).
//
// Shapes: Nq query rows at positions offset .. offset + Nq - 1 and Nk keys
// per head (the square case Nq = Nk, offset 0 has instances of its own); Q
// and K rows of width D, V, O and G rows of width DV.
//
// Three kernels, all on the caller's stream:
//  1. attn_bwd_prep_kernel: per row, LSE2 and -D into a workspace of two
//     planes per head (HBM-bound, one pass over O and G).
//  2. attn_bwd_dkdv_kernel: one workgroup owns 128 keys of one head (32 per
//     wave) and streams that head's query rows in tiles of 64; the wave's dK
//     and dV rows stay in registers for the whole loop and are written once,
//     so no two workgroups ever add into the same gradient row (the parallel
//     dK/dV accumulation the page asks for, without atomics).
//  3. attn_bwd_dq_kernel: one workgroup owns 128 query rows (32 per wave) and
//     streams the keys and values in tiles of 64, like the forward; dQ stays
//     in registers.  Recomputing S and dP here instead of adding dQ partial
//     sums atomically from kernel 2 costs two extra products per tile but
//     keeps every gradient deterministic.
//
// Operand layout (CDNA4 MFMA 32x32x16 bf16, fp32 accumulation; lane = l):
//  * dK/dV kernel: S = Q K^T and dP = G V^T for 32 queries x the wave's 32
//    keys per accumulator block, so every lane owns one key column (l % 32)
//    and 16 query rows; K and V of the wave's keys stay in VGPRs as B
//    operands; Q and G rows are read from LDS as A operands.  P and dS, rounded
//    to bf16, are then directly the B operands (k = query) of
//    dV^T += G^T P and dK^T += Q^T dS, with G^T and Q^T read from the same LDS
//    tiles by the transpose read.  LSE2 and D of the 16 query rows a lane
//    holds come from a 512-byte LDS copy of the tile's workspace rows.
//  * dQ kernel: the forward's orientation, S^T = K Q^T and dP^T = V G^T, so a
//    lane owns one query (one LSE2 and D in registers) and dS^T is the B
//    operand of dQ^T += K^T dS^T, K^T by the transpose read.
//  * Tiles reach LDS by buffer_load ... lds copies two stages deep (one
//    barrier per tile), in the swizzled layout of attn_common.hpp.  Rows past
//    the end of a head read as zeros.
//  * Causal: a key tile starts at the first query tile that can see it; the
//    query tiles end at the last key tile they can see; a wave whose rows lie
//    entirely on the hidden side of a tile skips its math; element masks only
//    on tiles crossing the diagonal or the end of the sequence.
#pragma once

#include "attn_common.hpp"

namespace tiledattn {

constexpr int kPrepRowsPerBlock = 16;     // 16 lanes per row, 256 threads

// Row statistics workspace: per head two planes of `stride` floats (stride:
// the rows rounded up to a multiple of 4, so both planes start 16-byte
// aligned): LSE2 of every row, then -D of every row (the starting value of a
// dP accumulator, so the products yield dP - D directly).
//
// Copy LSE2 and -D of the 64 query rows of tile i into LDS (256 bytes each,
// -D after LSE2): lanes 0..15 of wave 0 copy the LSE2 rows, lanes 16..31 the
// -D rows, 16 bytes each.  Each plane has a buffer resource of its own
// covering Nq rows, so rows past the end read as zeros (a finite D keeps the
// masked products finite).
__device__ __forceinline__ void issue_stats(__amdgpu_buffer_rsrc_t srl, __amdgpu_buffer_rsrc_t srd,
                                            int i, int wave, int lane, TA_LDS float* sd) {
  if (wave == 0) {
    if (lane < 16)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(srl, (TA_LDS void*)sd, 16, (uint32_t)lane * 16u,
                                               (uint32_t)i * (kBN * 4u), 0, 0);
    else if (lane < 32)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(srd, (TA_LDS void*)sd, 16,
                                               (uint32_t)(lane - 16) * 16u,
                                               (uint32_t)i * (kBN * 4u), 0, 0);
  }
}

// ---------------------------------------------------------------------------
// 1. -D_i = -sum_c G[i,c] O[i,c] and LSE2_i = LSE_i log2(e), one row per 16 lanes.
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_prep_kernel(const float* __restrict__ O,
                                                            const uint16_t* __restrict__ G,
                                                            const float* __restrict__ LSE,
                                                            float* __restrict__ stats, int N,
                                                            int stats_stride, int64_t rows) {
  constexpr int E = D / 16;                      // values per lane: 8 (d=128) or 4 (d=64)
  const int sub = threadIdx.x & 15;
  const int64_t row = (int64_t)blockIdx.x * kPrepRowsPerBlock + (threadIdx.x >> 4);
  float acc = 0.f;
  if (row < rows) {
    const float* orow = O + row * D + sub * E;
    const uint32_t* grow = reinterpret_cast<const uint32_t*>(G + row * D + sub * E);
#pragma unroll
    for (int e = 0; e < E; e += 4) {
      const f32x4 o = *reinterpret_cast<const f32x4*>(orow + e);
      const uint32_t w0 = grow[e / 2], w1 = grow[e / 2 + 1];   // 4 bf16, little-endian pairs
      acc = __builtin_fmaf(__uint_as_float(w0 << 16), o[0], acc);
      acc = __builtin_fmaf(__uint_as_float(w0 & 0xffff0000u), o[1], acc);
      acc = __builtin_fmaf(__uint_as_float(w1 << 16), o[2], acc);
      acc = __builtin_fmaf(__uint_as_float(w1 & 0xffff0000u), o[3], acc);
    }
  }
  // Sum over the 16 lanes of the row (xor butterfly stays inside the group).
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 16);
  if (row < rows && sub == 0) {
    const int64_t bh = row / N;
    float* head = stats + bh * 2 * stats_stride;
    head[row - bh * N] = LSE[row] * kLog2e;
    head[stats_stride + (row - bh * N)] = -acc;
  }
}

// Dropout mask words for a lane that owns key column k_first + (lane % 32) of
// 32 keys and, in query block qb of a 32 x 32 accumulator pair, tile rows
// 32 qb + 8 g + 4 hi + e (g, e = 0..3): word out[qb][g] carries rows e = 0..3
// in byte e (the byte layout dropout_keep reads).
// Lane L generates the two 16-key blocks (keys k_first .. k_first + 31) of
// tile row qbase + L; a 4 x 4 byte transpose inside each quad of lanes (rows
// 4a .. 4a+3) turns four rows x four keys around, and a 2 KB per-wave LDS block
// (64 bytes per key) hands every lane its column.  In a key's 64 bytes, row
// group a = 8 qb + 2 g + hi sits at word (hi, qb, g), so a reader's eight words
// are two aligned 16-byte chunks; chunk c of key k is stored at chunk
// c ^ ((k / 4) % 4), which keeps the 16-byte reads and the 4-byte writes free
// of bank conflicts.
__device__ __forceinline__ void dropout_col_words(uint32_t qbase, uint32_t k_first, uint32_t head,
                                                  const DropoutArgs& dr, int lane,
                                                  TA_LDS uint32_t* buf, uint32_t (&out)[2][4]) {
  const uint32_t blk = k_first >> 4;
  const u32x4 b0 = philox4x32_10(qbase + (uint32_t)lane, blk, head, 0u, dr.seed_lo, dr.seed_hi);
  const u32x4 b1 = philox4x32_10(qbase + (uint32_t)lane, blk + 1u, head, 0u, dr.seed_lo,
                                 dr.seed_hi);
  // Quad transpose, two exchanges (byte selectors of v_perm_b32: 0-3 pick the
  // second operand's bytes, 4-7 the first's):
  //  1. with lane ^ 1: even lanes keep (own 0, partner 0, own 2, partner 2),
  //     odd lanes (partner 1, own 1, partner 3, own 3);
  //  2. with lane ^ 2: lanes 0, 1 keep (own 0, own 1, partner 0, partner 1),
  //     lanes 2, 3 (partner 2, partner 3, own 2, own 3).
  // Lane 4a + i then holds key 4w + i of rows 4a .. 4a+3 (row 4a + e in byte e).
  const uint32_t sel1 = (lane & 1) ? 0x03070105u : 0x06020400u;
  const uint32_t sel2 = (lane & 2) ? 0x03020706u : 0x05040100u;
  const int a = lane >> 2, i = lane & 3;
  const int pos = ((a & 1) << 3) | ((a >> 3) << 2) | ((a >> 1) & 3);
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    const uint32_t x = (w < 4) ? b0[w] : b1[w - 4];   // keys 4w .. 4w+3 of row qbase + lane
    const uint32_t px = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false);
    const uint32_t y1 = __builtin_amdgcn_perm(px, x, sel1);
    const uint32_t py = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)y1, 0x4E, 0xF, 0xF, false);
    const uint32_t y2 = __builtin_amdgcn_perm(py, y1, sel2);
    const int key = 4 * w + i;
    buf[key * 16 + ((((pos >> 2) ^ (key >> 2)) & 3) << 2) + (pos & 3)] = y2;
  }
  __builtin_amdgcn_wave_barrier();
  const int kk = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int c = (2 * hi + qb) ^ ((kk >> 2) & 3);
    const u32x4 r = *reinterpret_cast<const TA_LDS u32x4*>(buf + kk * 16 + 4 * c);
#pragma unroll
    for (int g = 0; g < 4; ++g) out[qb][g] = r[g];
  }
  __builtin_amdgcn_wave_barrier();
}

// ---------------------------------------------------------------------------
// 2. dK and dV for 128 keys of one head per workgroup.
// D: width of Q and K rows (dK); DV: width of V, O and G rows (dV).  Nq query
// rows at positions offset .. offset + Nq - 1 and Nk keys (causal: key j is
// visible to query i iff j <= i + offset); GENERAL = false is the square case
// (Nk = Nq, offset 0) with those facts known at compile time.
// DROPOUT: the probabilities of the forward were kept or zeroed by the mask of
// `drop` and scaled by keep_scale:  dV = (P M ks)^T G,  dS = P (M ks dP - D).
template <int D, int DV, bool CAUSAL, bool GENERAL, bool DROPOUT = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1)))
void attn_bwd_dkdv_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                          const uint16_t* __restrict__ V, const uint16_t* __restrict__ G,
                          const float* __restrict__ stats, float* __restrict__ dK,
                          float* __restrict__ dV, int bh_count, int Nq, int nk_arg,
                          int offset_arg, int stats_stride, int n_kt, float c, float scale,
                          int skip_floor, DropoutArgs drop) {
  static_assert(GENERAL || D == DV, "square instances have one head width");
  const int Nk = GENERAL ? nk_arg : Nq;
  const int offset = GENERAL ? offset_arg : 0;
  using T = Tile<D>;     // Q and K rows, dK
  using TG = Tile<DV>;   // G and V rows, dV
  __shared__ __attribute__((aligned(1024))) uint16_t q_lds0[kBN * D];
  __shared__ __attribute__((aligned(1024))) uint16_t g_lds0[kBN * DV];
  __shared__ __attribute__((aligned(1024))) uint16_t q_lds1[kBN * D];
  __shared__ __attribute__((aligned(1024))) uint16_t g_lds1[kBN * DV];
  __shared__ __attribute__((aligned(16))) float st_lds0[2 * kBN];   // LSE2 rows, then -D rows
  __shared__ __attribute__((aligned(16))) float st_lds1[2 * kBN];
  __shared__ __attribute__((aligned(16))) uint32_t mk_lds[DROPOUT ? kWaves * 32 * 16 : 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  int bh, kt;
  map_block(blockIdx.x, bh_count, n_kt, false, CAUSAL, 32, bh, kt);   // causal: key tile 0 has most work

  const size_t qhead = (size_t)bh * (size_t)Nq, khead = (size_t)bh * (size_t)Nk;
  const __amdgpu_buffer_rsrc_t qr = make_rsrc(Q + qhead * D, (uint32_t)Nq * D * 2u);
  const __amdgpu_buffer_rsrc_t gr = make_rsrc(G + qhead * DV, (uint32_t)Nq * DV * 2u);
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(K + khead * D, (uint32_t)Nk * D * 2u);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(V + khead * DV, (uint32_t)Nk * DV * 2u);
  const float* st_head = stats + (size_t)bh * 2 * (size_t)stats_stride;
  const __amdgpu_buffer_rsrc_t srl = make_rsrc(st_head, (uint32_t)Nq * 4u);
  const __amdgpu_buffer_rsrc_t srd = make_rsrc(st_head + stats_stride, (uint32_t)Nq * 4u);

  const int k0 = kt * kBM + wave * 32;    // first key of this wave
  const int my_k = k0 + l32;              // this lane's key

  // K and V rows of the wave's keys (B operands, k = d): [my_k][16 ks + 8 hi + 0..7].
  bf16x8 kf[T::KS], vf[TG::KS];
  constexpr int KSM = T::KS > TG::KS ? T::KS : TG::KS;
#pragma unroll
  for (int ks = 0; ks < KSM; ++ks) {
    if (ks < T::KS)
      kf[ks] = __builtin_bit_cast(bf16x8, load16(kr, (uint32_t)(my_k * D + 16 * ks + 8 * hi) * 2u));
    if (ks < TG::KS)
      vf[ks] = __builtin_bit_cast(bf16x8, load16(vr, (uint32_t)(my_k * DV + 16 * ks + 8 * hi) * 2u));
  }

  uint32_t src_q[T::LOADS], src_g[TG::LOADS];
  tile_src_offsets<D>(src_q, wave, lane);
  tile_src_offsets<DV>(src_g, wave, lane);
  const LdsReader<D> rd(lane);
  const LdsReader<DV> rdg(lane);

  f32x16 dk[T::DB], dv[TG::DB];
#pragma unroll
  for (int db = 0; db < T::DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dk[db][i] = 0.f;
#pragma unroll
  for (int db = 0; db < TG::DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dv[db][i] = 0.f;

  const int n_qt = (Nq + kBN - 1) / kBN;
  // First query tile that sees any key here: its last position reaches kt kBM.
  const int i0 = CAUSAL ? (GENERAL ? max(0, kt * kBM - offset) : kt * kBM) / kBN : 0;

  auto compute_tile = [&](int i, const TA_LDS uint16_t* qt, const TA_LDS uint16_t* gt,
                          const TA_LDS float* st) {
    const int qbase = i * kBN;
    // Row statistics of the 16 query rows each lane holds per block: element
    // 4 g4 + t of block qb is tile row 32 qb + 8 g4 + 4 hi + t (four
    // consecutive rows, one 16-byte read per plane).  LSE2 is kept for the
    // exponent; the stored -D is the starting value of the dP accumulator, so
    // the products below yield dP - D directly.
    f32x16 s[2], dp[2];
    float lse2[2][16];
    float nd[DROPOUT ? 2 : 1][16];   // dropout: -D itself, the dP accumulator starts at 0
    uint32_t mk[2][4];
    if constexpr (DROPOUT)
      dropout_col_words((uint32_t)(qbase + offset), (uint32_t)k0, (uint32_t)bh, drop, lane,
                        (TA_LDS uint32_t*)mk_lds + wave * (32 * 16), mk);
    // S and dP - D: 2 blocks of 32 queries x the wave's 32 keys (4 KS products).
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[qb][e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const bf16x8 aq = rd.row_op(qt, qb, ks);
        s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, kf[ks], s[qb], 0, 0, 0);
      }
    // The row statistics (needed from dP on) and the first G operands of dP
    // are read under the S products, after S's own operands.
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int qb = r >> 2, g4 = r & 3;
      const int qrow = 32 * qb + 8 * g4 + 4 * hi;
      const f32x4 l2 = *reinterpret_cast<const TA_LDS f32x4*>(st + qrow);
      const f32x4 n = *reinterpret_cast<const TA_LDS f32x4*>(st + kBN + qrow);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        lse2[qb][4 * g4 + t] = l2[t];
        if constexpr (DROPOUT) {
          nd[qb][4 * g4 + t] = n[t];
          dp[qb][4 * g4 + t] = 0.f;
        } else {
          dp[qb][4 * g4 + t] = n[t];
        }
      }
    }
    constexpr int kGPre = 3;
    static_assert(TG::KS >= kGPre, "dP has at least kGPre operand steps");
    bf16x8 agp[kGPre][2];
#pragma unroll
    for (int ks = 0; ks < kGPre; ++ks)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) agp[ks][qb] = rdg.row_op(gt, qb, ks);
    // Reads: 6 ahead, then two after each product.
    sched_mfma_ds<6, 2, 2 * T::KS + 16 + 2 * kGPre>(std::make_integer_sequence<int, 2 * T::KS>{});
    // S is issued in full before dP, so that the exponent arguments (accumulator
    // reads and FMAs, which need only S) run between the dP products.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < TG::KS; ++ks)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const bf16x8 ag = ks < kGPre ? agp[ks < kGPre ? ks : 0][qb] : rdg.row_op(gt, qb, ks);
        dp[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ag, vf[ks], dp[qb], 0, 0, 0);
      }

    // Exponent arguments c s - LSE2; hidden pairs (query before key, or query
    // past the end) get -inf, which exp2 turns into an exact 0.
    const bool edge = (CAUSAL && qbase + offset < k0 + 31) || (qbase + kBN > Nq);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[qb][e] = __builtin_fmaf(s[qb][e], c, -lse2[qb][e]);
    {
      constexpr int kDP = 2 * TG::KS;
      constexpr int kArgPer = (64 + kDP - 1) / kDP;
      sched_reads<4>();
      sched_rep<1, kArgPer, kDP>();
    }
    if (edge) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int q = qbase + 32 * qb + 8 * (e >> 2) + 4 * hi + (e & 3);
          if ((CAUSAL && my_k > q + offset) || q >= Nq) s[qb][e] = -__builtin_inff();
        }
    }
    // P = 2^arg and dS = P (dP - D), rounded to bf16 as B operands.
    bf16x8 pf[4], sf[4];
    if constexpr (DROPOUT) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
          float pm[2], ds[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const float p = __builtin_amdgcn_exp2f(s[qb][e + u]);
            // dV uses P M (keep_scale is applied to dV once, at the end).
            const bool keep = dropout_keep(mk, qb, e + u, drop.t);
            pm[u] = keep ? p : 0.f;
            const float g = keep ? __builtin_fmaf(drop.keep_scale, dp[qb][e + u], nd[qb][e + u])
                                 : nd[qb][e + u];
            ds[u] = p * g;
          }
          // One packed conversion per pair (after the mask's selects the
          // compiler would otherwise convert each value alone and permute).
          const bf16x2 bp = __builtin_convertvector(f32x2{pm[0], pm[1]}, bf16x2);
          const bf16x2 bs = __builtin_convertvector(f32x2{ds[0], ds[1]}, bf16x2);
          pf[2 * qb + (e >> 3)][e & 7] = bp[0];
          pf[2 * qb + (e >> 3)][(e & 7) + 1] = bp[1];
          sf[2 * qb + (e >> 3)][e & 7] = bs[0];
          sf[2 * qb + (e >> 3)][(e & 7) + 1] = bs[1];
        }
    } else {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = __builtin_amdgcn_exp2f(s[qb][e]);
          pf[2 * qb + (e >> 3)][e & 7] = (__bf16)p;
          sf[2 * qb + (e >> 3)][e & 7] = (__bf16)(p * dp[qb][e]);
        }
    }

    // dV^T (dv x 32 keys) += G^T (dv x 64 queries) P;  dK^T (d x 32) += Q^T dS.
    constexpr int DBM = T::DB > TG::DB ? T::DB : TG::DB;
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int db = 0; db < DBM; ++db) {
        if (db < TG::DB) {
          const bf16x8 ag = rdg.col_op(gt, g, db);
          dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ag, pf[g], dv[db], 0, 0, 0);
        }
        if (db < T::DB) {
          const bf16x8 aq = rd.col_op(qt, g, db);
          dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, sf[g], dk[db], 0, 0, 0);
        }
      }
    sched_mfma_ds<8, 2, 8 * (T::DB + TG::DB)>(std::make_integer_sequence<int, 4 * (T::DB + TG::DB)>{});
  };

  TA_LDS uint16_t* const q0p = (TA_LDS uint16_t*)q_lds0;
  TA_LDS uint16_t* const g0p = (TA_LDS uint16_t*)g_lds0;
  TA_LDS uint16_t* const q1p = (TA_LDS uint16_t*)q_lds1;
  TA_LDS uint16_t* const g1p = (TA_LDS uint16_t*)g_lds1;
  TA_LDS float* const s0p = (TA_LDS float*)st_lds0;
  TA_LDS float* const s1p = (TA_LDS float*)st_lds1;
  // A wave's keys are all hidden from query tile i when its last query
  // precedes the wave's first key.  Without the causal mask the host passes
  // INT_MIN as skip_floor: the test is then always true, but stays a runtime
  // branch, which keeps each tile's products in a scheduling region of its own
  // (merged regions made the compiler spill).
  const int first_key = CAUSAL ? k0 - offset : skip_floor;
  auto active = [&](int i) { return i * kBN + kBN - 1 >= first_key; };
  // Each stage holds the Q and G rows of one query tile and their {LSE2, D}.
  // Pairs of tiles run in the loop (stage 0, stage 1); an odd last tile runs
  // after it, so the loop has a single exit.
  if (i0 < n_qt) {
    issue_pair<D, DV>(qr, gr, src_q, src_g, i0, wave, q0p, g0p);
    issue_stats(srl, srd, i0, wave, lane, s0p);
  }
  int i = i0;
  for (; i + 1 < n_qt; i += 2) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();                       // tile i visible; tile i-1's readers done
    issue_pair<D, DV>(qr, gr, src_q, src_g, i + 1, wave, q1p, g1p);
    issue_stats(srl, srd, i + 1, wave, lane, s1p);
    if (active(i)) compute_tile(i, q0p, g0p, s0p);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (i + 2 < n_qt) {
      issue_pair<D, DV>(qr, gr, src_q, src_g, i + 2, wave, q0p, g0p);
      issue_stats(srl, srd, i + 2, wave, lane, s0p);
    }
    if (active(i + 1)) compute_tile(i + 1, q1p, g1p, s1p);
  }
  if (i < n_qt) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (active(i)) compute_tile(i, q0p, g0p, s0p);
  }

  // Epilogue: lane owns key my_k; accumulator element e of block db is column
  // 32 db + 8 (e / 4) + 4 hi + e % 4.
  const float vs = DROPOUT ? drop.keep_scale : 1.f;
  if constexpr (D == DV) {
    // dK, then dV, through LDS (store_rows_lds): each wave uses one of the
    // now free Q/G stages.
    __syncthreads();                       // every wave is done with the stages
    TA_LDS uint8_t* const reg = wave == 0 ? (TA_LDS uint8_t*)q_lds0
                                : wave == 1 ? (TA_LDS uint8_t*)g_lds0
                                : wave == 2 ? (TA_LDS uint8_t*)q_lds1
                                            : (TA_LDS uint8_t*)g_lds1;
    store_rows_lds<D>(reg, dk, scale, dK + (khead + k0) * D, Nk - k0, lane);
    store_rows_lds<DV>(reg, dv, vs, dV + (khead + k0) * DV, Nk - k0, lane);
  } else if (my_k < Nk) {
    float* dkrow = dK + (khead + my_k) * D;
    float* dvrow = dV + (khead + my_k) * DV;
    constexpr int DBM = T::DB > TG::DB ? T::DB : TG::DB;
#pragma unroll
    for (int db = 0; db < DBM; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if (db < T::DB) {
          f32x4 a = {dk[db][4 * g] * scale, dk[db][4 * g + 1] * scale, dk[db][4 * g + 2] * scale,
                     dk[db][4 * g + 3] * scale};
          *reinterpret_cast<f32x4*>(dkrow + db * 32 + 8 * g + 4 * hi) = a;
        }
        if (db < TG::DB) {
          f32x4 b = {dv[db][4 * g] * vs, dv[db][4 * g + 1] * vs, dv[db][4 * g + 2] * vs,
                     dv[db][4 * g + 3] * vs};
          *reinterpret_cast<f32x4*>(dvrow + db * 32 + 8 * g + 4 * hi) = b;
        }
      }
  }
}

// ---------------------------------------------------------------------------
// 3. dQ for 128 query rows of one head per workgroup.
// Shapes as for the dK/dV kernel (D, DV, Nq, Nk, offset, GENERAL).
// DROPOUT: dS = P (M ks dP - D) with the forward's mask (dropout_row_words).
template <int D, int DV, bool CAUSAL, bool GENERAL, bool DROPOUT = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void attn_bwd_dq_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                        const uint16_t* __restrict__ V, const uint16_t* __restrict__ G,
                        const float* __restrict__ stats, float* __restrict__ dQ, int bh_count,
                        int Nq, int nk_arg, int offset_arg, int stats_stride, int n_qt, float c,
                        float scale, int skip_ceiling, DropoutArgs drop) {
  static_assert(GENERAL || D == DV, "square instances have one head width");
  const int Nk = GENERAL ? nk_arg : Nq;
  const int offset = GENERAL ? offset_arg : 0;
  using T = Tile<D>;     // Q and K rows, dQ
  using TV = Tile<DV>;   // G and V rows
  __shared__ __attribute__((aligned(1024))) uint16_t k_lds0[kBN * D];
  __shared__ __attribute__((aligned(1024))) uint16_t v_lds0[kBN * DV];
  __shared__ __attribute__((aligned(1024))) uint16_t k_lds1[kBN * D];
  __shared__ __attribute__((aligned(1024))) uint16_t v_lds1[kBN * DV];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  int bh, qt;
  map_block(blockIdx.x, bh_count, n_qt, CAUSAL, CAUSAL, 64, bh, qt);

  const size_t qhead = (size_t)bh * (size_t)Nq, khead = (size_t)bh * (size_t)Nk;
  const __amdgpu_buffer_rsrc_t qr = make_rsrc(Q + qhead * D, (uint32_t)Nq * D * 2u);
  const __amdgpu_buffer_rsrc_t gr = make_rsrc(G + qhead * DV, (uint32_t)Nq * DV * 2u);
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(K + khead * D, (uint32_t)Nk * D * 2u);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(V + khead * DV, (uint32_t)Nk * DV * 2u);

  const int q0 = qt * kBM + wave * 32;
  const int my_q = q0 + l32;

  // Q and G rows of the lane's query (B operands of S^T = K Q^T, dP^T = V G^T).
  bf16x8 qf[T::KS], gf[TV::KS];
#pragma unroll
  for (int ks = 0; ks < T::KS; ++ks)
    qf[ks] = __builtin_bit_cast(bf16x8, load16(qr, (uint32_t)(my_q * D + 16 * ks + 8 * hi) * 2u));
#pragma unroll
  for (int ks = 0; ks < TV::KS; ++ks)
    gf[ks] = __builtin_bit_cast(bf16x8, load16(gr, (uint32_t)(my_q * DV + 16 * ks + 8 * hi) * 2u));
  float lse2 = 0.f, nd = 0.f;   // LSE2 and -D of the lane's query
  if (my_q < Nq) {
    const float* st_head = stats + (size_t)bh * 2 * (size_t)stats_stride;
    lse2 = st_head[my_q];
    nd = st_head[stats_stride + my_q];
  }

  uint32_t src_k[T::LOADS], src_v[TV::LOADS];
  tile_src_offsets<D>(src_k, wave, lane);
  tile_src_offsets<DV>(src_v, wave, lane);
  const LdsReader<D> rd(lane);
  const LdsReader<DV> rdv(lane);

  f32x16 dq[T::DB];
#pragma unroll
  for (int db = 0; db < T::DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dq[db][i] = 0.f;

  const int n_kt_all = (Nk + kBN - 1) / kBN;
  // Causal: key tiles up to the last row's position.
  const int n_kt = CAUSAL ? min(n_kt_all, (qt * kBM + kBM + offset + kBN - 1) / kBN) : n_kt_all;

  auto compute_tile = [&](int j, const TA_LDS uint16_t* kt, const TA_LDS uint16_t* vt) {
    const int key0 = j * kBN;
    const bool edge = (CAUSAL && key0 + kBN - 1 > q0 + offset) || (key0 + kBN > Nk);
    uint32_t mw[2][4];
    if constexpr (DROPOUT)
      dropout_row_words((uint32_t)(my_q + offset), (uint32_t)j, (uint32_t)bh, drop, hi, mw);
    // One 32-key block at a time: S^T and dP^T (32 keys x 32 queries), then
    // its dS^T, then its share of dQ^T.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // Without dropout dP^T - D accumulates from -D (the lane's query is the
      // accumulator column, so every element starts at the same -D).
      f32x16 s, dp;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        s[e] = 0.f;
        dp[e] = DROPOUT ? 0.f : nd;
      }
#pragma unroll
      for (int ks = 0; ks < T::KS; ++ks) {
        const bf16x8 ak = rd.row_op(kt, kb, ks);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qf[ks], s, 0, 0, 0);
      }
#pragma unroll
      for (int ks = 0; ks < TV::KS; ++ks) {
        const bf16x8 av = rdv.row_op(vt, kb, ks);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, gf[ks], dp, 0, 0, 0);
      }
      sched_mfma_ds<4, 1, T::KS + TV::KS>(std::make_integer_sequence<int, T::KS + TV::KS>{});

      // Element e is key key0 + 32 kb + 8 (e / 4) + 4 hi + e % 4 of query my_q;
      // hidden keys get exponent -inf (an exact 0).
#pragma unroll
      for (int e = 0; e < 16; ++e) s[e] = __builtin_fmaf(s[e], c, -lse2);
      if (edge) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = key0 + kb * 32 + 8 * (e >> 2) + 4 * hi + (e & 3);
          if ((CAUSAL && key > my_q + offset) || key >= Nk) s[e] = -__builtin_inff();
        }
      }
      bf16x8 sf[2];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float g = dp[e];
        if constexpr (DROPOUT)
          g = dropout_keep(mw, kb, e, drop.t) ? __builtin_fmaf(drop.keep_scale, dp[e], nd) : nd;
        sf[e >> 3][e & 7] = (__bf16)(__builtin_amdgcn_exp2f(s[e]) * g);
      }

      // dQ^T (d x 32 queries) += K^T (d x these 32 keys) dS^T.
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int db = 0; db < T::DB; ++db) {
          const bf16x8 ak = rd.col_op(kt, 2 * kb + h, db);
          dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, sf[h], dq[db], 0, 0, 0);
        }
      sched_mfma_ds<8, 2, 4 * T::DB>(std::make_integer_sequence<int, 2 * T::DB>{});
    }
  };

  // A wave's queries all precede key tile j when its first key is past the
  // wave's last query.  Without the causal mask the host passes INT_MAX as
  // skip_ceiling: always true, but a runtime branch that keeps the two tiles
  // of an iteration in separate scheduling regions.
  const int last_query = CAUSAL ? q0 + 31 + offset : skip_ceiling;
  auto active = [&](int j) { return j * kBN <= last_query; };

  TA_LDS uint16_t* const k0p = (TA_LDS uint16_t*)k_lds0;
  TA_LDS uint16_t* const v0p = (TA_LDS uint16_t*)v_lds0;
  TA_LDS uint16_t* const k1p = (TA_LDS uint16_t*)k_lds1;
  TA_LDS uint16_t* const v1p = (TA_LDS uint16_t*)v_lds1;
  if (n_kt > 0) issue_pair<D, DV>(kr, vr, src_k, src_v, 0, wave, k0p, v0p);
  for (int j = 0; j < n_kt; j += 2) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (j + 1 < n_kt) issue_pair<D, DV>(kr, vr, src_k, src_v, j + 1, wave, k1p, v1p);
    if (active(j)) compute_tile(j, k0p, v0p);
    if (j + 1 >= n_kt) break;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (j + 2 < n_kt) issue_pair<D, DV>(kr, vr, src_k, src_v, j + 2, wave, k0p, v0p);
    if (active(j + 1)) compute_tile(j + 1, k1p, v1p);
  }

  if constexpr (DV >= D) {
    // dQ through LDS (store_rows_lds): each wave uses one of the now free
    // K/V stages.
    __syncthreads();                       // every wave is done with the stages
    TA_LDS uint8_t* const reg = wave == 0 ? (TA_LDS uint8_t*)k0p
                                : wave == 1 ? (TA_LDS uint8_t*)v0p
                                : wave == 2 ? (TA_LDS uint8_t*)k1p
                                            : (TA_LDS uint8_t*)v1p;
    store_rows_lds<D>(reg, dq, scale, dQ + (qhead + q0) * D, Nq - q0, lane);
  } else if (my_q < Nq) {
    float* row = dQ + (qhead + my_q) * D;
#pragma unroll
    for (int db = 0; db < T::DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 a = {dq[db][4 * g] * scale, dq[db][4 * g + 1] * scale, dq[db][4 * g + 2] * scale,
                   dq[db][4 * g + 3] * scale};
        *reinterpret_cast<f32x4*>(row + db * 32 + 8 * g + 4 * hi) = a;
      }
  }
}

}  // namespace tiledattn
