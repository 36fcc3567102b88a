// Fused attention forward for gfx950 (MI355X): one workgroup owns a tile of
// BM query rows of one (batch, head) and streams that head's keys and values
// through LDS in tiles of BN, keeping the online-softmax state in registers.
//
// Method (page "22. GPU Engineering: Correctness, Throughput, and Attention",
// sec. 22.5): per query row a running maximum m, normaliser l and
// unnormalised accumulator o start at -inf, 0, 0; each score tile S updates
//   m' = max(m, max S),  alpha = exp(m - m'),  p = exp(S - m'),
//   l' = alpha l + sum p,  o' = alpha o + p V_tile,
// and the output is o / l.  Hidden (future or non-existent) keys are set to
// -inf before the maximum and the sum.  A row whose maximum is still -inf uses
// 0 as exponent reference (sec. 22.7 lab).  The per-row log-normaliser
// m + ln l is stored beside O (sec. 22.7: the statistic a recomputing backward
// needs).  Exponentials are taken base 2 with log2(e) folded into the score
// scale; the stored LSE is converted back to natural log.
//
// Mapping to CDNA4 (wave64, MFMA 32x32x16 bf16 with fp32 accumulation):
//  * Each of the 4 waves owns 32 query rows.  Scores are computed transposed,
//    S^T = K Q^T, so an MFMA accumulator gives each lane one query (lane%32)
//    and 16 keys of it; the row max/sum is then 15 in-lane ops plus one
//    exchange between the two wave halves (instead of a 32-lane reduction).
//  * The same accumulator, rounded to bf16, is directly the B operand of
//    O^T = V^T P^T; O^T accumulates in fp32 registers for the whole loop, and
//    its lane%32 column is again the lane's own query, so the alpha rescale is
//    lane-local.
//  * K is staged row-major in LDS, rows padded by 16 bytes (conflict-free
//    128-bit reads of 16 consecutive rows).  V is staged transposed (V^T,
//    keys contiguous) with a key permutation inside each group of 16 keys so
//    that the 8 keys a wave half needs for one MFMA are contiguous.
//  * Global tiles are read with 128-bit buffer loads whose range check
//    returns zeros past the end of the head (ragged N: zero K rows are then
//    masked, zero V rows keep 0 * garbage out of the sum).  The next tile's
//    loads are issued before the current tile's math (register double
//    buffering), so HBM/L2 latency hides under MFMA work.
//  * Causal: a query tile only visits key tiles up to its last row; a wave
//    whose rows are all before a key tile skips that tile's math; element
//    masks are applied only on tiles that straddle the diagonal or the end.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tiledattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kWaves = 4;
constexpr int kThreads = kWave * kWaves;
constexpr int kBM = 128;          // query rows per workgroup (32 per wave)
constexpr int kBN = 64;           // keys per LDS tile
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit data format
constexpr float kLn2 = 0.69314718055994530942f;

template <int D>
struct Tile {
  static_assert(D == 64 || D == 128, "head dim");
  static constexpr int KS = D / 16;                 // MFMA k-steps over d for S^T
  static constexpr int DB = D / 32;                 // 32-row blocks of O^T
  static constexpr int KSTR = D + 8;                // bf16 per K row in LDS
  static constexpr int VSTR = kBN + 8;              // bf16 per V^T row in LDS
  static constexpr int CHUNKS = kBN * D / 8;        // 16-byte chunks per tile
  static constexpr int CPT = CHUNKS / kThreads;     // chunks per thread (4 or 2)
  static constexpr int DCH = D / 8;                 // 16-byte chunks per row
  static_assert(CPT * kThreads == CHUNKS, "tile split");
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kRsrcWord3);
}

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

// Position of key r (0..15) inside its 16-key group of the V^T tile: bits 2
// and 3 exchanged, so keys {0-3, 8-11} fill slots 0-7 and {4-7, 12-15} slots
// 8-15 -- the two halves of a wave each read 8 contiguous slots.
__device__ __forceinline__ int vpos(int key) {
  const int r = key & 15;
  return (key & ~15) | (r & 3) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// Workgroup -> (head, query tile).  Workgroups are handed to the 8 XCDs
// round-robin, so block b runs on XCD b % 8; consecutive logical indices are
// given to the same XCD so one head's query tiles share that XCD's L2.
// Causal: within a head the longest (last) query tiles go first.
__device__ __forceinline__ void map_block(int bid, int bh_count, int n_qt, bool causal,
                                          int& bh, int& qt) {
  const int total = bh_count * n_qt;
  int j = bid;
  if ((total & 7) == 0) j = (bid & 7) * (total >> 3) + (bid >> 3);
  bh = j / n_qt;
  const int t = j - bh * n_qt;
  qt = causal ? n_qt - 1 - t : t;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void attn_fwd_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                     const uint16_t* __restrict__ V, float* __restrict__ O,
                     float* __restrict__ LSE, int bh_count, int N, int n_qt, float scale_log2) {
  using T = Tile<D>;
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[kBN * T::KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[D * T::VSTR];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  int bh, qt;
  map_block(blockIdx.x, bh_count, n_qt, CAUSAL, bh, qt);

  const size_t head = (size_t)bh * (size_t)N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2u;
  const __amdgpu_buffer_rsrc_t qr = make_rsrc(Q + head, head_bytes);
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(K + head, head_bytes);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(V + head, head_bytes);

  const int q0 = qt * kBM + wave * 32;   // first query row of this wave
  const int my_q = q0 + l32;             // this lane's query row

  // Q fragment (B operand of S^T = K Q^T): Q[my_q][16 ks + 8 hi + 0..7].
  bf16x8 qf[T::KS];
#pragma unroll
  for (int ks = 0; ks < T::KS; ++ks)
    qf[ks] = __builtin_bit_cast(bf16x8, load16(qr, (uint32_t)(my_q * D + 16 * ks + 8 * hi) * 2u));

  f32x16 oacc[T::DB];
#pragma unroll
  for (int db = 0; db < T::DB; ++db)
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m = -__builtin_inff();   // running max of log2-domain scores (whole row)
  float l = 0.f;                 // running normaliser (this wave half's keys)

  const int n_kt_all = (N + kBN - 1) / kBN;
  const int n_kt = CAUSAL ? min(n_kt_all, (qt + 1) * (kBM / kBN)) : n_kt_all;

  // Staging assignment.  K: chunk c = tid + 256 i -> key c / DCH, chunk c % DCH.
  // V: this thread owns CPT consecutive keys at one 8-wide d chunk.
  const int v_dc = tid % T::DCH;
  const int v_k0 = (tid / T::DCH) * T::CPT;

  u32x4 kreg[T::CPT], vreg[T::CPT];
  auto load_tile = [&](int j) {
    const int key0 = j * kBN;
#pragma unroll
    for (int i = 0; i < T::CPT; ++i) {
      const int c = tid + kThreads * i;
      const int key = key0 + c / T::DCH;
      kreg[i] = load16(kr, (uint32_t)(key * D + (c % T::DCH) * 8) * 2u);
    }
#pragma unroll
    for (int i = 0; i < T::CPT; ++i)
      vreg[i] = load16(vr, (uint32_t)((key0 + v_k0 + i) * D + v_dc * 8) * 2u);
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < T::CPT; ++i) {
      const int c = tid + kThreads * i;
      *reinterpret_cast<u32x4*>(&k_lds[(c / T::DCH) * T::KSTR + (c % T::DCH) * 8]) = kreg[i];
    }
    // Transpose V: d row (8 v_dc + e) receives this thread's CPT keys.
    const int col = vpos(v_k0);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if constexpr (T::CPT == 4) {
        const u32x2 ev = {(vreg[0][w] & 0xffffu) | (vreg[1][w] << 16),
                          (vreg[2][w] & 0xffffu) | (vreg[3][w] << 16)};
        const u32x2 od = {(vreg[0][w] >> 16) | (vreg[1][w] & 0xffff0000u),
                          (vreg[2][w] >> 16) | (vreg[3][w] & 0xffff0000u)};
        *reinterpret_cast<u32x2*>(&v_lds[(v_dc * 8 + 2 * w) * T::VSTR + col]) = ev;
        *reinterpret_cast<u32x2*>(&v_lds[(v_dc * 8 + 2 * w + 1) * T::VSTR + col]) = od;
      } else {
        const uint32_t ev = (vreg[0][w] & 0xffffu) | (vreg[1][w] << 16);
        const uint32_t od = (vreg[0][w] >> 16) | (vreg[1][w] & 0xffff0000u);
        *reinterpret_cast<uint32_t*>(&v_lds[(v_dc * 8 + 2 * w) * T::VSTR + col]) = ev;
        *reinterpret_cast<uint32_t*>(&v_lds[(v_dc * 8 + 2 * w + 1) * T::VSTR + col]) = od;
      }
    }
  };

  load_tile(0);
  for (int j = 0; j < n_kt; ++j) {
    __syncthreads();                 // all waves are done reading tile j-1
    store_tile();
    __syncthreads();                 // tile j is visible in LDS
    if (j + 1 < n_kt) load_tile(j + 1);

    const int key0 = j * kBN;
    if (CAUSAL && key0 > q0 + 31) continue;   // every key of this tile is in this wave's future

    // S^T (64 keys x 32 queries): block kb covers keys key0 + 32 kb + [0, 32).
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < T::KS; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(
            &k_lds[(kb * 32 + l32) * T::KSTR + 16 * ks + 8 * hi]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[kb], 0, 0, 0);
      }
    }

    // Scale into the log2 domain; hide future / non-existent keys.
    const bool edge = (CAUSAL && key0 + kBN - 1 > q0) || (key0 + kBN > N);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float t = s[kb][i] * scale_log2;
        if (edge) {
          const int key = key0 + kb * 32 + 8 * (i >> 2) + 4 * hi + (i & 3);
          if ((CAUSAL && key > my_q) || key >= N) t = -__builtin_inff();
        }
        s[kb][i] = t;
      }

    // Row maximum: 32 in-lane values, then the other wave half.
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));

    const float m_new = fmaxf(m, mx);
    const float ref = (m_new == -__builtin_inff()) ? 0.f : m_new;   // safe reference
    const float alpha = __builtin_amdgcn_exp2f(m - ref);
    m = m_new;

    float psum = 0.f;
    bf16x8 pf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(s[kb][i] - ref);
        psum += p;
        pf[kb][i >> 3][i & 7] = (__bf16)p;
      }
    l = alpha * l + psum;

#pragma unroll
    for (int db = 0; db < T::DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;

    // O^T (d x 32 queries) += V^T (d x 64 keys) P^T (64 keys x 32 queries).
#pragma unroll
    for (int db = 0; db < T::DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(
            &v_lds[(db * 32 + l32) * T::VSTR + g * 16 + 8 * hi]);
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[g >> 1][g & 1], oacc[db], 0, 0, 0);
      }
  }

  // Epilogue: combine the two halves' normalisers, O = o / l, LSE = m + log2 l (as ln).
  const float l_row = l + __shfl_xor(l, 32);
  if (my_q < N) {
    const float inv = 1.f / l_row;
    float* orow = O + head + (size_t)my_q * D;
#pragma unroll
    for (int db = 0; db < T::DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 val = {oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv,
                     oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv};
        *reinterpret_cast<f32x4*>(orow + db * 32 + 8 * g + 4 * hi) = val;
      }
    if (hi == 0) LSE[(size_t)bh * N + my_q] = (m + __log2f(l_row)) * kLn2;
  }
}

}  // namespace tiledattn
