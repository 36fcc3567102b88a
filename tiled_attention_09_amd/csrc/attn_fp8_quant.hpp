// Per-head FP8 (OCP E4M3) quantisation of bf16 rows for the FP8-score forward
// (page "Chapter 7 GPU Kernels: CUDA, HIP & Triton", sec. 7.6.2: FP8 Q K^T
// with online descaling; page "22. GPU Engineering: Correctness, Throughput,
// and Attention", sec. 22.3: compare against a reference on the same
// quantised inputs).
//
// For each head h (a contiguous block of n_per_head values):
//   amax_h    = max |x|                       (1. init, 2. block maxima + atomic max)
//   code      = RNE_e4m3(clamp(x * (448 / amax_h), -448, 448))     (3.)
//   descale_h = amax_h / 448  (1 when amax_h = 0)                   (4.)
// in float32, one operation per step, so x ~= e4m3(code) * descale_h and the
// codes are reproducible bit for bit.  While steps 1-3 run, descale[h] holds
// the bit pattern of amax_h (a non-negative float orders like its bits, so an
// unsigned atomic max is a float max); step 4 replaces it by the descale.
#pragma once

#include "attn_common.hpp"

namespace tiledattn {

constexpr int kQuantThreads = 256;
constexpr int kQuantPerThread = 16;                        // bf16 values per thread
constexpr int kQuantPerBlock = kQuantThreads * kQuantPerThread;
constexpr float kE4M3Max = 448.f;

__global__ __launch_bounds__(256) void fp8_amax_init_kernel(uint32_t* amax_bits, int heads) {
  const int h = blockIdx.x * 256 + threadIdx.x;
  if (h < heads) amax_bits[h] = 0u;
}

// Amax pass: each thread reads kAmaxPerThread bf16 values per chunk of
// kAmaxPerBlock (eight independent 16-byte loads in flight), and a block
// strides over the head's chunks, so a head takes at most kAmaxBlocksPerHead
// blocks and as many atomics on its amax word (atomics on one word serialise
// in L2).  Grid: (min(chunks, kAmaxBlocksPerHead), heads).  A wave covers 64
// kAmaxPerThread consecutive values of a chunk, load v of lane l the 8 values
// at 512 v + 8 l of them: every load instruction reads 1 KB contiguous.
// n_per_head is a multiple of 8, so each 8-value load is all in range or all
// past the end.
constexpr int kAmaxPerThread = 64;
constexpr int kAmaxPerBlock = kQuantThreads * kAmaxPerThread;
constexpr int kAmaxBlocksPerHead = 16;

__global__ __launch_bounds__(kQuantThreads) void fp8_amax_kernel(const uint16_t* __restrict__ x,
                                                                 uint32_t* amax_bits,
                                                                 int64_t n_per_head) {
  __shared__ uint32_t part[kQuantThreads / 64];
  const int64_t base = (int64_t)blockIdx.y * n_per_head;
  const int lane = threadIdx.x & 63;
  uint32_t m = 0u;   // |x| as bits: bf16 bits << 16 with the sign cleared
  for (int64_t c0 = (int64_t)blockIdx.x * kAmaxPerBlock; c0 < n_per_head;
       c0 += (int64_t)gridDim.x * kAmaxPerBlock) {
    const int64_t w0 = c0 + (int64_t)(threadIdx.x >> 6) * (64 * kAmaxPerThread);
    u32x4 w[kAmaxPerThread / 8];
#pragma unroll
    for (int v = 0; v < kAmaxPerThread / 8; ++v) {
      const int64_t i = w0 + 512 * v + 8 * lane;
      w[v] = i < n_per_head ? *reinterpret_cast<const u32x4*>(x + base + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int v = 0; v < kAmaxPerThread / 8; ++v)
#pragma unroll
      for (int t = 0; t < 4; ++t) m = max(m, max((w[v][t] << 16) & 0x7fffffffu, w[v][t] & 0x7fff0000u));
  }
  // Wave maximum, then the block's four waves through LDS, then one atomic.
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t b = max(max(part[0], part[1]), max(part[2], part[3]));
    atomicMax(amax_bits + blockIdx.y, b);
  }
}

__device__ __forceinline__ float e4m3_scale_of(uint32_t amax_bits) {
  const float amax = __uint_as_float(amax_bits);
  return amax > 0.f ? kE4M3Max / amax : 1.f;
}

// Grid: (chunks, heads).  Each thread: 16 bf16 in, 16 codes out.
__global__ __launch_bounds__(kQuantThreads) void fp8_quant_kernel(const uint16_t* __restrict__ x,
                                                                  uint8_t* __restrict__ out,
                                                                  const uint32_t* amax_bits,
                                                                  int64_t n_per_head) {
  const int64_t base = (int64_t)blockIdx.y * n_per_head;
  const int64_t i0 = (int64_t)blockIdx.x * kQuantPerBlock + (int64_t)threadIdx.x * kQuantPerThread;
  if (i0 >= n_per_head) return;
  const float inv = e4m3_scale_of(amax_bits[blockIdx.y]);
  const u32x4* src = reinterpret_cast<const u32x4*>(x + base + i0);
  u32x4 codes;
#pragma unroll
  for (int v = 0; v < 2; ++v) {
    const u32x4 w = src[v];
#pragma unroll
    for (int t = 0; t < 4; t += 2) {
      // four values -> one 32-bit word of codes (two packed conversions)
      float f[4] = {__uint_as_float(w[t] << 16), __uint_as_float(w[t] & 0xffff0000u),
                    __uint_as_float(w[t + 1] << 16), __uint_as_float(w[t + 1] & 0xffff0000u)};
#pragma unroll
      for (int e = 0; e < 4; ++e) f[e] = fminf(fmaxf(f[e] * inv, -kE4M3Max), kE4M3Max);
      int word = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
      word = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], word, true);
      codes[2 * v + t / 2] = (uint32_t)word;
    }
  }
  *reinterpret_cast<u32x4*>(out + base + i0) = codes;
}

__global__ __launch_bounds__(256) void fp8_descale_kernel(uint32_t* amax_bits, int heads) {
  const int h = blockIdx.x * 256 + threadIdx.x;
  if (h < heads) {
    const float amax = __uint_as_float(amax_bits[h]);
    amax_bits[h] = __float_as_uint(amax > 0.f ? amax / kE4M3Max : 1.f);
  }
}

}  // namespace tiledattn
