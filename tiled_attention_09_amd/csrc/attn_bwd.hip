// C ABI of the attention backward (declarations and contract in
// include/tiledattn.h).  Validates arguments before touching the HIP runtime,
// then enqueues the row-statistics kernel, the dK/dV kernel and the dQ kernel
// on the caller's stream.  attn_bwd_dropout runs the same kernels with the
// forward's dropout mask regenerated from its seed (attn_common.hpp).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "attn_bwd_kernel.hpp"
#include "tiledattn.h"

namespace {

constexpr int kMaxN = 1 << 22;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Rows of one head in the workspace, padded to an even count (16-byte heads).
int64_t stats_stride(int N) { return ((int64_t)N + 1) & ~(int64_t)1; }

template <int D, bool CAUSAL, bool DROPOUT>
int launch(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* o,
           const float* lse, const uint16_t* g, float* dq, float* dk, float* dv,
           tiledattn::f32x2* stats, int bh, int N, float scale, tiledattn::DropoutArgs dr,
           hipStream_t stream) {
  using namespace tiledattn;
  const int stride = (int)stats_stride(N);
  const int64_t rows = (int64_t)bh * N;
  const unsigned prep_blocks = (unsigned)((rows + kPrepRowsPerBlock - 1) / kPrepRowsPerBlock);
  const int n_t = (N + kBM - 1) / kBM;
  const float c = (float)((double)scale * 1.4426950408889634073599);
  attn_bwd_prep_kernel<D><<<dim3(prep_blocks), dim3(256), 0, stream>>>(o, g, lse, stats, N,
                                                                       stride, rows);
  attn_bwd_dkdv_kernel<D, CAUSAL, DROPOUT>
      <<<dim3((unsigned)(bh * n_t)), dim3(kThreads), 0, stream>>>(
          q, k, v, g, stats, dk, dv, bh, N, stride, n_t, c, scale, INT32_MIN, dr);
  attn_bwd_dq_kernel<D, CAUSAL, DROPOUT><<<dim3((unsigned)(bh * n_t)), dim3(kThreads), 0, stream>>>(
      q, k, v, g, stats, dq, bh, N, stride, n_t, c, scale, INT32_MAX, dr);
  return hipGetLastError() == hipSuccess ? TA_OK : TA_ERR_HIP;
}

bool valid_sizes(int B, int H, int N) {
  if (B < 1 || H < 1 || N < 1 || N > kMaxN) return false;
  const int64_t bh = (int64_t)B * H;
  const int64_t n_t = (N + tiledattn::kBM - 1) / tiledattn::kBM;
  if (bh * n_t > INT32_MAX) return false;
  // The row-statistics grid (16 rows per workgroup) stays below 2^32 workgroups.
  return bh * stats_stride(N) <= ((int64_t)1 << 34);
}

// Shared by attn_bwd (DROPOUT = false) and attn_bwd_dropout: every check happens
// before any HIP call.
template <bool DROPOUT>
int backward(const void* q, const void* k, const void* v, const float* o, const float* lse,
             const void* dout, float* dq, float* dk, float* dv, void* workspace, int B, int H,
             int N, int d, float scale, int causal, tiledattn::DropoutArgs dr, void* stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !workspace)
    return TA_ERR_INVALID_ARG;
  if (!valid_sizes(B, H, N)) return TA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return TA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return TA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return TA_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
      !aligned(workspace, 16) || !aligned(lse, 4))
    return TA_ERR_MISALIGNED;

  const int bh = B * H;
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto* qq = static_cast<const uint16_t*>(q);
  auto* kk = static_cast<const uint16_t*>(k);
  auto* vv = static_cast<const uint16_t*>(v);
  auto* gg = static_cast<const uint16_t*>(dout);
  auto* st = static_cast<tiledattn::f32x2*>(workspace);
  if (d == 64)
    return causal
               ? launch<64, true, DROPOUT>(qq, kk, vv, o, lse, gg, dq, dk, dv, st, bh, N, scale, dr, s)
               : launch<64, false, DROPOUT>(qq, kk, vv, o, lse, gg, dq, dk, dv, st, bh, N, scale, dr,
                                            s);
  return causal
             ? launch<128, true, DROPOUT>(qq, kk, vv, o, lse, gg, dq, dk, dv, st, bh, N, scale, dr, s)
             : launch<128, false, DROPOUT>(qq, kk, vv, o, lse, gg, dq, dk, dv, st, bh, N, scale, dr,
                                           s);
}

}  // namespace

extern "C" int attn_bwd(const void* q, const void* k, const void* v, const float* o,
                        const float* lse, const void* dout, float* dq, float* dk, float* dv,
                        void* workspace, int B, int H, int N, int d, float scale, int causal,
                        void* stream) {
  return backward<false>(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, H, N, d, scale, causal,
                         tiledattn::DropoutArgs{}, stream);
}

extern "C" int attn_bwd_dropout(const void* q, const void* k, const void* v, const float* o,
                                const float* lse, const void* dout, float* dq, float* dk,
                                float* dv, void* workspace, int B, int H, int N, int d,
                                float scale, int causal, uint64_t seed, int drop_t,
                                void* stream) {
  if (drop_t < 0 || drop_t > 255) return TA_ERR_INVALID_ARG;
  tiledattn::DropoutArgs dr;
  dr.seed_lo = (uint32_t)seed;
  dr.seed_hi = (uint32_t)(seed >> 32);
  dr.t = (uint32_t)drop_t;
  dr.keep_scale = (float)(256.0 / (256.0 - (double)drop_t));
  return backward<true>(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, H, N, d, scale, causal,
                        dr, stream);
}

extern "C" size_t attn_bwd_workspace_size(int B, int H, int N) {
  if (!valid_sizes(B, H, N)) return 0;
  return (size_t)B * (size_t)H * (size_t)stats_stride(N) * 8u;
}
