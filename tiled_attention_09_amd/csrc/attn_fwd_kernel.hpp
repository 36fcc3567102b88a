// Fused attention forward for gfx950 (MI355X): one workgroup owns a tile of
// BM query rows of one (batch, head) and streams that head's keys and values
// through LDS in tiles of BN keys, keeping the online-softmax state in
// registers, so the score matrix never reaches HBM.
//
// Method (page "22. GPU Engineering: Correctness, Throughput, and Attention",
// sec. 22.5): per query row a running maximum m, normaliser l and
// unnormalised accumulator o start at -inf, 0, 0; each score tile S updates
//   m' = max(m, max S),  alpha = exp(m - m'),  p = exp(S - m'),
//   l' = alpha l + sum p,  o' = alpha o + p V_tile,
// and the output is o / l.  Hidden (future or non-existent) keys get -inf
// before the maximum and the sum.  A row whose maximum is still -inf uses 0 as
// exponent reference (sec. 22.7 lab).  The per-row log-normaliser m + ln l is
// stored beside O (sec. 22.7: the statistic a recomputing backward needs).
// Exponentials are taken base 2 with log2(e) folded into the score scale; the
// stored LSE is converted back to natural log.
//
// Mapping to CDNA4 (wave64; MFMA 32x32x16 bf16, fp32 accumulation):
//  * 4 waves x 32 query rows.  Scores are computed transposed, S^T = K Q^T,
//    so an accumulator gives each lane one query (lane % 32) and 16 of its
//    keys: the row max/sum is in-lane work plus one exchange between the two
//    wave halves.  Q stays in VGPRs as the B operand for the whole loop.
//  * The same accumulator, rounded to bf16, is the B operand of
//    O^T = V^T P^T; O^T accumulates in fp32 registers and its column is again
//    the lane's own query, so the alpha rescale is lane-local.
//  * K and V tiles are copied HBM/L2 -> LDS by the buffer unit itself
//    (buffer_load ... lds, 16 bytes per lane, no VGPR staging), two stages
//    each, K one tile ahead of V; one barrier per tile.
//  * Software pipeline inside the wave: while the softmax of tile j runs on
//    the vector unit, the score products of tile j+1 run on the matrix unit
//    (an explicit issue recipe interleaves them), then o is rescaled (only
//    when some row moved its maximum) and P_j V_j accumulated.  The buffer
//    range check returns zeros past the end of the head, so a ragged last
//    tile needs no guard (zero V rows also keep 0 * garbage out of the sum).
//  * Both tiles keep the row-major [key][d] layout with the 16-byte chunks of
//    each row XOR-swizzled by the row index.  K is read row-wise as the MFMA A
//    operand (16 consecutive rows per 16 lanes hit 16 different chunk slots);
//    V is read with the LDS transpose read (ds_read_b64_tr_b16): each 16-lane
//    group receives a 16(d) x 4(keys) block transposed, which is exactly the
//    V^T operand, and the 4 key rows of a half-wave land in 4 different 64-byte
//    bank groups.
//  * Causal: a query tile visits key tiles only up to its last row's position
//    (query index plus the offset of the lab's decoding-style subproblems); a
//    wave whose rows all precede a key tile skips its math; element masks are
//    applied only on tiles that cross the diagonal or the end of the keys.
//  * General shapes: Nq queries and Nk keys per head, Q/K rows of width D and
//    V/O rows of width DV; with no keys a row keeps l = 0 and gets O = 0,
//    LSE = -inf (the lab's fully-hidden-row policy).
//  * Split key ranges (decoding over long contexts): workgroups cover key
//    tile ranges of one (head, query tile) and write their own normalised O
//    and LSE; attn_split_merge_kernel combines them by their log-normalisers.
//  * Epilogue: O leaves through LDS (store_rows_lds), so that each store
//    instruction writes whole rows instead of 32-byte pieces of 32 rows.
#pragma once

#include "attn_common.hpp"

namespace tiledattn {

// Vector instructions of the softmax placed after each score product (square
// shapes; the general-shape instances keep 7, with which they do not spill).
constexpr int kValuPerMfma = 5;
constexpr int kValuPerMfmaGeneral = 7;
// Vector instructions of the dropout generator placed after each value product.
constexpr int kDropValuPerMfma = 16;

// D: width of Q and K rows; DV: width of V and O rows.  Nq query rows at
// absolute positions offset .. offset + Nq - 1 attend Nk keys at positions
// 0 .. Nk - 1 (causal: key j visible to query i iff j <= i + offset).
// GENERAL = false is the square case (Nk = Nq, offset 0) with those facts
// known at compile time.  F8: Q and K are FP8 (OCP E4M3) codes with per-head
// descale factors (Q = codes * q_descale[b h], likewise K), the scores use the
// FP8 matrix product, and the descales fold into the exponent scale (d = 64 or 128).
// DROPOUT: each probability is kept or zeroed by the reproducible mask of
// `drop` (DropoutArgs) and the output scaled by keep_scale; the normaliser and
// LSE count every visible key; the mask's row counter is the query's absolute
// position (offset + row), so a query chunk draws the rows of the whole problem.
// SPLIT: the key range is split over workgroups: bh_count counts (split,
// head) pairs, workgroup (s, head) covers key tiles [s split_tiles,
// (s + 1) split_tiles) and writes its own normalised O and LSE at index
// s * heads + head of O and LSE (attn_split_merge_kernel combines them).
template <int D, int DV, bool CAUSAL, bool POS_SCALE, bool GENERAL, bool F8 = false,
          bool DROPOUT = false, bool SPLIT = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void attn_fwd_kernel(const void* __restrict__ Qv, const void* __restrict__ Kv,
                     const uint16_t* __restrict__ V, float* __restrict__ O,
                     float* __restrict__ LSE, int bh_count, int Nq, int nk_arg, int offset_arg,
                     int n_qt, float scale_log2, const float* __restrict__ q_descale,
                     const float* __restrict__ k_descale, DropoutArgs drop, int heads,
                     int split_tiles) {
  static_assert(!F8 || D == 64 || D == 128, "FP8 scores: d = 64 or 128");
  static_assert(!DROPOUT || !F8, "dropout: bf16 scores");
  static_assert(!SPLIT || (GENERAL && !F8 && !DROPOUT), "split key ranges: general bf16 shapes");
  const int Nk = GENERAL ? nk_arg : Nq;
  const int offset = GENERAL ? offset_arg : 0;
  using T = Tile<D>;
  using TV = Tile<DV>;
  // K tile geometry in bytes: an FP8 row of D values is laid out like a bf16
  // row of D / 2 (D bytes).
  constexpr int DK = F8 ? D / 2 : D;
  using TK = Tile<DK>;
  constexpr uint32_t kElemQK = F8 ? 1u : 2u;     // bytes per Q / K value
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds0[TK::BYTES];
  __shared__ __attribute__((aligned(1024))) uint16_t v_lds0[kBN * DV];
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds1[TK::BYTES];
  __shared__ __attribute__((aligned(1024))) uint16_t v_lds1[kBN * DV];
  const char* Q = static_cast<const char*>(Qv);
  const char* K = static_cast<const char*>(Kv);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  int bhs, qt;
  map_block(blockIdx.x, bh_count, n_qt, CAUSAL, CAUSAL, 64, bhs, qt);
  const int split = SPLIT ? bhs / heads : 0;
  const int bh = SPLIT ? bhs - split * heads : bhs;   // (batch, head) of Q, K, V

  const __amdgpu_buffer_rsrc_t qr =
      make_rsrc(Q + (size_t)bh * Nq * D * kElemQK, (uint32_t)Nq * D * kElemQK);
  const __amdgpu_buffer_rsrc_t kr =
      make_rsrc(K + (size_t)bh * Nk * D * kElemQK, (uint32_t)Nk * D * kElemQK);
  if constexpr (F8) scale_log2 *= q_descale[bh] * k_descale[bh];   // online descaling
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(V + (size_t)bh * Nk * DV, (uint32_t)Nk * DV * 2u);

  const int q0 = qt * kBM + wave * 32;   // first query row of this wave
  const int my_q = q0 + l32;             // this lane's query row

  // Q fragment (B operand of S^T = K Q^T): bf16 Q[my_q][16 ks + 8 hi + 0..7];
  // FP8: bytes [64 ks + 32 hi, +32) of row my_q (the byte order of the K reads).
  constexpr int KS8 = D / 64;
  bf16x8 qf[F8 ? 1 : T::KS];
  i32x8 qf8[F8 ? KS8 : 1];
  if constexpr (F8) {
#pragma unroll
    for (int ks = 0; ks < KS8; ++ks) {
      const uint32_t off = (uint32_t)(my_q * D + 64 * ks + 32 * hi);
      qf8[ks] = __builtin_bit_cast(
          i32x8, __builtin_shufflevector(load16(qr, off), load16(qr, off + 16u), 0, 1, 2, 3, 4, 5,
                                         6, 7));
    }
  } else {
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8, load16(qr, (uint32_t)(my_q * D + 16 * ks + 8 * hi) * 2u));
  }
  if constexpr (F8 && POS_SCALE) {
    // The instance takes the row maximum on raw scores, which is right only
    // for a positive effective scale.  A negative descale product is folded
    // into Q instead: negating an E4M3 code flips its sign bit, so with every
    // Q code negated and the scale's magnitude the scaled scores are unchanged.
    if (scale_log2 < 0.f) {
      scale_log2 = -scale_log2;
#pragma unroll
      for (int ks = 0; ks < KS8; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) qf8[ks][e] ^= (int)0x80808080u;
    }
  }

  // Tile copy offsets: the same for every tile (K and V differ only when D != DV).
  uint32_t src_k[TK::LOADS], src_v[TV::LOADS];
  tile_src_offsets<DK>(src_k, wave, lane);
  tile_src_offsets<DV>(src_v, wave, lane);
  // Operand reads: K row-wise (A operand of S^T), V transposed (A operand of
  // O^T), with lane offsets whose row/stage parts fold into the instruction.
  const LdsReader<D> rd(lane);
  const LdsReaderF8<D> rd8(lane);
  const LdsReader<DV> rdv(lane);

  f32x16 oacc[TV::DB];
#pragma unroll
  for (int db = 0; db < TV::DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  // Running max: raw-score domain when the scale is positive (max commutes
  // with the scale), scaled log2 domain otherwise.
  float m = -__builtin_inff();
  float l = 0.f;               // running normaliser (this wave half's keys)

  // Key tiles this query tile can see (causal: up to its last row's position).
  const int n_kt_all = (Nk + kBN - 1) / kBN;
  const int n_kt_vis = CAUSAL ? min(n_kt_all, (qt * kBM + kBM + offset + kBN - 1) / kBN) : n_kt_all;
  // Key tiles of this workgroup: [kt_lo, n_kt) (kt_lo is even, so the stage
  // parity of tile j is still j % 2).
  const int kt_lo = SPLIT ? split * split_tiles : 0;
  const int n_kt = SPLIT ? min(n_kt_vis, kt_lo + split_tiles) : n_kt_vis;
  const int q_last = q0 + 31 + offset;   // position of the wave's last query row

  // Tiles this wave takes part in: key tiles whose first key is not past the
  // wave's last query position (a prefix of 0 .. n_kt - 1); none when all of
  // its rows lie past the last query (a ragged last tile, a decoding step):
  // such a wave only shares the tile copies and barriers.
  const int n_w = (q0 >= Nq) ? 0 : (CAUSAL ? min(n_kt, q_last / kBN + 1) : n_kt);

  // S^T (64 keys x 32 queries) of the key tile in `kt`: block kb covers tile
  // keys 32 kb + [0, 32).
  auto scores = [&](const TA_LDS uint8_t* kt, f32x16 (&s)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
    if constexpr (F8) {
      // 32x32x64 FP8 products (unit block scales: exponent 127 = 2^0).
#pragma unroll
      for (int ks = 0; ks < KS8; ++ks)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(rd8.row_op(kt, kb, ks), qf8[ks],
                                                                  s[kb], 0, 0, 0, 127, 0, 127);
    } else {
#pragma unroll
      for (int ks = 0; ks < T::KS; ++ks)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              rd.row_op((const TA_LDS uint16_t*)kt, kb, ks), qf[ks], s[kb], 0, 0, 0);
    }
  };
  // Score products per tile and the LDS reads that feed them.
  constexpr int kScoreMfma = F8 ? 2 * KS8 : 2 * T::KS;
  constexpr int kScoreReads = F8 ? 2 * kScoreMfma : kScoreMfma;
  constexpr int kValuPerScore = F8 ? 16 : (GENERAL ? kValuPerMfmaGeneral : kValuPerMfma);

  // Scale (non-positive scales only) and hide future / non-existent keys of key
  // tile j in s; only tiles crossing the diagonal or the end of the keys need
  // the mask.
  auto prepare = [&](int j, f32x16 (&s)[2]) __attribute__((always_inline)) {
    const int key0 = j * kBN;
    if (!POS_SCALE) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][i] *= scale_log2;
    }
    if ((CAUSAL && key0 + kBN - 1 > q0 + offset) || (key0 + kBN > Nk)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = key0 + kb * 32 + 8 * (i >> 2) + 4 * hi + (i & 3);
          if ((CAUSAL && key > my_q + offset) || key >= Nk) s[kb][i] = -__builtin_inff();
        }
    }
  };

  // Online-softmax update from a tile's prepared scores s:
  // m' = max(m, max S), alpha = exp(m - m'), p = exp(S - m'), l' = alpha l + sum p.
  // Returns alpha; p goes to pf as the bf16 B operand of the value product.
  // In the square instances without dropout the sum is formed in `values`
  // from the fp32 p kept in pe (the adds then run under the value products,
  // where the vector unit is otherwise idle); the general-shape and dropout
  // instances keep it here (the live p would make them spill).
  constexpr bool kSumInValues = !GENERAL && !DROPOUT;
  // With the fp32 p kept, its bf16 rounding for the value products also moves
  // there (each operand converted just before its products): the score region
  // is bound by the vector unit, the value region is not.
  constexpr bool kCvtInValues = kSumInValues;
  // Dropout mask words of the tile whose softmax runs next (dropout_row_words).
  uint32_t mw[2][4];
  float pe[32];
  auto softmax = [&](f32x16 (&s)[2], bf16x8 (&pf)[4]) __attribute__((always_inline)) {
    // Row maximum: 32 in-lane values (a chain of 3-input maxima), then the
    // other wave half.
    float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int i = 2; i < 32; i += 2)
      mx = fmaxf(fmaxf(mx, s[i >> 4][i & 15]), s[(i + 1) >> 4][(i + 1) & 15]);
    mx = fmaxf(mx, other_half(mx));
    // The safe reference keeps a row with no visible key yet away from -inf - -inf.
    const float m_new = fmaxf(m, mx);
    const float ref = (m_new == -__builtin_inff()) ? 0.f : m_new;
    const float cref = POS_SCALE ? ref * scale_log2 : ref;
    // alpha is exactly 1 while the maximum stays put.  (Formed as
    // exp2(c m - cref), it would be 1 only up to the rounding of cref: the
    // subtraction contracts into a fused multiply-add, and a factor 1 - 2^-24
    // applied on every tile of a long row drifts l by 0.6 % over 5e4 tiles.)
    const float alpha = (m_new == m) ? 1.f
                                     : __builtin_amdgcn_exp2f((POS_SCALE ? m * scale_log2 : m) - cref);
    m = m_new;
    // p = 2^(c s - c m'); positive scale: one fused multiply-add per element.
    // For the row maximum itself the argument is only the rounding residual of
    // c m (|r| <= 2^-24 |c m|), so its p rounds to exactly 1 in bf16: the
    // dominant weight carries no bf16 rounding into the value product.
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        float pv[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float arg = POS_SCALE ? __builtin_fmaf(s[kb][i + e], scale_log2, -cref)
                                      : s[kb][i + e] - cref;
          const float p = __builtin_amdgcn_exp2f(arg);
          if constexpr (kSumInValues) pe[kb * 16 + i + e] = p;
          else psum += p;
          // Dropout zeroes the weight in the value product only: the
          // normaliser keeps every visible key.
          pv[e] = (DROPOUT && !dropout_keep(mw, kb, i + e, drop.t)) ? 0.f : p;
        }
        if constexpr (DROPOUT) {
          // Spelled as one packed conversion per key pair: after the mask's
          // selects the compiler would otherwise convert each value alone and
          // pack the halves with a permute.
          const bf16x2 b = __builtin_convertvector(f32x2{pv[0], pv[1]}, bf16x2);
          pf[kb * 2 + (i >> 3)][i & 7] = b[0];
          pf[kb * 2 + (i >> 3)][(i & 7) + 1] = b[1];
        } else if constexpr (!kCvtInValues) {
          pf[kb * 2 + (i >> 3)][i & 7] = (__bf16)pv[0];
          pf[kb * 2 + (i >> 3)][(i & 7) + 1] = (__bf16)pv[1];
        }
      }
    if constexpr (!kSumInValues) l = __builtin_fmaf(l, alpha, psum);
    return alpha;
  };

  // (l = alpha l + sum p,) o = alpha o, then O^T (dv x 32 queries) += V^T (dv x
  // 64 keys) P^T (64 keys x 32 queries).  Without dropout the transposed V operands of the first
  // four products are read before the rescale, so that when some row moved
  // its maximum the 16 DV / 32 multiplies per block run under the latency of
  // those reads instead of ahead of them.  With dropout (whose mask generator
  // needs those registers) the reads follow the rescale, and the mask words
  // of tile j + 1 are generated during the products (the vector unit is
  // otherwise idle there).
  auto values = [&](int j, const TA_LDS uint16_t* vt, const bf16x8 (&pf)[4], float alpha)
                    __attribute__((always_inline)) {
    if constexpr (kSumInValues) {
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) psum += pe[i];
      l = __builtin_fmaf(l, alpha, psum);
    }
    constexpr int NPRE = DROPOUT ? 0 : TV::DB;   // operands read before the rescale
    bf16x8 vpre[TV::DB];
#pragma unroll
    for (int db = 0; db < NPRE; ++db) vpre[db] = rdv.col_op(vt, 0, db);
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < TV::DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x8 pg = pf[g];
      if constexpr (kCvtInValues) {
        // Keys 8 g .. 8 g + 7 of the lane's 32: element i of 32-key block kb
        // is pe[16 kb + i], operand g holds block g / 2, elements 8 (g % 2) + t.
#pragma unroll
        for (int t = 0; t < 8; ++t) pg[t] = (__bf16)pe[8 * g + t];
      }
#pragma unroll
      for (int db = 0; db < TV::DB; ++db)
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            (g == 0 && NPRE) ? vpre[db] : rdv.col_op(vt, g, db), pg, oacc[db], 0, 0, 0);
    }
    if constexpr (DROPOUT) {
      dropout_row_words((uint32_t)(my_q + offset), (uint32_t)(j + 1), (uint32_t)bh, drop, hi, mw);
      // Eight transposed V reads in flight, then two more per product.
      sched_mfma_ds_valu<8, 2, 8 * TV::DB, kDropValuPerMfma>(
          std::make_integer_sequence<int, 4 * TV::DB>{});
    } else {
      // The remaining reads, two after each product (eight in flight).
      sched_mfma_ds<0, 2, 6 * TV::DB>(std::make_integer_sequence<int, 4 * TV::DB>{});
    }
  };

  // Pipeline (the matrix work of the next tile runs under the softmax of this
  // one, inside the wave): K runs one tile ahead of V.  At iteration j, LDS
  // holds K_{j+1} (for S_{j+1}) and V_j (for P_j V_j); the barrier at its start
  // also frees K_j's and V_{j-1}'s stages, which receive K_{j+2} and V_{j+1}.
  // Each iteration: S_{j+1} = K_{j+1} Q^T interleaved with the softmax of S_j,
  // the alpha rescale of o (only when some row moved its maximum), then P_j V_j.
  TA_LDS uint8_t* const k0 = (TA_LDS uint8_t*)k_lds0;
  TA_LDS uint16_t* const v0 = (TA_LDS uint16_t*)v_lds0;
  TA_LDS uint8_t* const k1 = (TA_LDS uint8_t*)k_lds1;
  TA_LDS uint16_t* const v1 = (TA_LDS uint16_t*)v_lds1;
  f32x16 sa[2], sb[2];
  bf16x8 pf[4];

  auto step = [&](int j, const TA_LDS uint8_t* k_next, const TA_LDS uint16_t* v_cur,
                  f32x16 (&s_cur)[2], f32x16 (&s_next)[2]) __attribute__((always_inline)) {
    prepare(j, s_cur);
    // The shared region runs at raised wave priority, so the other wave on
    // this SIMD (in its own value products) does not hold back its issue.
    __builtin_amdgcn_s_setprio(1);
    float alpha;
    if (j + 1 < n_w) {
      // S_{j+1} only for a tile this wave visits (its K stage was filled).
      scores(k_next, s_next);
      alpha = softmax(s_cur, pf);
      // Issue order: four K operand reads ahead, then each product followed by
      // one read and a share of the softmax's vector instructions.
      sched_reads<4>();
      sched_rep<(kScoreReads - 4) / (kScoreMfma - 4 > 0 ? kScoreMfma - 4 : kScoreMfma),
                kValuPerScore, (kScoreMfma - 4 > 0 ? kScoreMfma - 4 : kScoreMfma)>();
      sched_rep<0, kValuPerScore, (kScoreMfma - 4 > 0 ? 4 : 0)>();
      // The probabilities must be complete here, inside the region shared with
      // the score products: without this use the compiler sinks the
      // exponentials below the rescale branch, out of reach of the interleave.
      if constexpr (kCvtInValues) {
#pragma unroll
        for (int i = 0; i < 32; i += 4)
          asm volatile("" ::"v"(pe[i]), "v"(pe[i + 1]), "v"(pe[i + 2]), "v"(pe[i + 3]));
      } else {
        asm volatile("" ::"v"(pf[0]), "v"(pf[1]), "v"(pf[2]), "v"(pf[3]));
      }
    } else {
      alpha = softmax(s_cur, pf);   // the wave's last tile: nothing to overlap
    }
    __builtin_amdgcn_s_setprio(0);
    values(j, v_cur, pf, alpha);
  };
  // Iteration j with the stage parity P = j % 2 fixed at compile time.
  auto iter = [&](int j, auto pc) __attribute__((always_inline)) {
    constexpr int P = decltype(pc)::value;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();                 // K_{j+1}, V_j visible; K_j, V_{j-1} stages free
    if (j + 2 < n_kt)
      issue_rows<DK>(kr, src_k, j + 2, wave, (TA_LDS uint16_t*)(P ? k1 : k0));
    if (j + 1 < n_kt) issue_rows<DV>(vr, src_v, j + 1, wave, P ? v0 : v1);
    if (j < n_w) {
      if constexpr (P == 0)
        step(j, k1, v0, sa, sb);
      else
        step(j, k0, v1, sb, sa);
    }
  };

  if (n_kt > kt_lo) {
    issue_rows<DK>(kr, src_k, kt_lo, wave, (TA_LDS uint16_t*)k0);
    issue_rows<DV>(vr, src_v, kt_lo, wave, v0);
    if (n_kt > kt_lo + 1) issue_rows<DK>(kr, src_k, kt_lo + 1, wave, (TA_LDS uint16_t*)k1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (n_w > kt_lo) scores(k0, sa);
    if constexpr (DROPOUT)
      dropout_row_words((uint32_t)(my_q + offset), 0u, (uint32_t)bh, drop, hi, mw);
  }
  for (int j = kt_lo; j < n_kt; j += 2) {
    iter(j, std::integral_constant<int, 0>{});
    if (j + 1 >= n_kt) break;
    iter(j + 1, std::integral_constant<int, 1>{});
  }

  // Epilogue: combine the two halves' normalisers, O = o / l, LSE = m + log2 l
  // (as ln).  A row that saw no key (no keys at all) follows the lab's policy:
  // O = 0 and LSE = -inf.
  const float l_row = l + other_half(l);
  const bool live = l_row > 0.f;
  const float inv = live ? (DROPOUT ? drop.keep_scale : 1.f) / l_row : 0.f;
  if constexpr (!F8 && D >= DV) {
    // O goes out through LDS (store_rows_lds), each wave through one of the
    // now free K/V stages.
    __syncthreads();                        // every wave is done with the stages
    TA_LDS uint8_t* const reg = wave == 0 ? k0
                                : wave == 1 ? (TA_LDS uint8_t*)v0
                                : wave == 2 ? k1
                                            : (TA_LDS uint8_t*)v1;
    store_rows_lds<DV>(reg, oacc, inv, O + ((size_t)bhs * Nq + q0) * DV, Nq - q0, lane);
  } else {
    if (my_q < Nq) {
      float* orow = O + ((size_t)bhs * Nq + my_q) * DV;
#pragma unroll
      for (int db = 0; db < TV::DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 val = {oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv,
                             oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv};
          *reinterpret_cast<f32x4*>(orow + db * 32 + 8 * g + 4 * hi) = val;
        }
    }
  }
  if (my_q < Nq && hi == 0) {
    const float mlog2 = POS_SCALE ? m * scale_log2 : m;
    LSE[(size_t)bhs * Nq + my_q] = live ? (mlog2 + __log2f(l_row)) * kLn2 : -__builtin_inff();
  }
}

// Combination of the partial results of a split key range, each normalised by
// its own l: LSE = log sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s (the
// online-softmax recurrence of the tiles, applied once to whole key ranges).
// Os: [n_split][rows][DV], Ls: [n_split][rows]; one wave per row.  A row
// whose partial LSEs are all -inf saw no key: O = 0, LSE = -inf.
template <int DV>
__global__ __launch_bounds__(256) void attn_split_merge_kernel(const float* __restrict__ Os,
                                                               const float* __restrict__ Ls,
                                                               float* __restrict__ O,
                                                               float* __restrict__ LSE,
                                                               int64_t rows, int n_split) {
  constexpr int C = DV / 64;   // output columns per lane
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  float m = -__builtin_inff();
  for (int sp = 0; sp < n_split; ++sp) m = fmaxf(m, Ls[sp * rows + row]);
  float acc[C] = {};
  float den = 0.f;
  if (m != -__builtin_inff()) {
    for (int sp = 0; sp < n_split; ++sp) {
      const float w = expf(Ls[sp * rows + row] - m);
      den += w;
      const float* src = Os + (sp * rows + row) * DV + lane * C;
#pragma unroll
      for (int c = 0; c < C; ++c) acc[c] = __builtin_fmaf(w, src[c], acc[c]);
    }
  }
  const bool live = den > 0.f;
  float* dst = O + row * DV + lane * C;
#pragma unroll
  for (int c = 0; c < C; ++c) dst[c] = live ? acc[c] / den : 0.f;
  if (lane == 0) LSE[row] = live ? m + logf(den) : -__builtin_inff();
}

}  // namespace tiledattn
