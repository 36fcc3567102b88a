// C ABI of attention with dropout on the probabilities (declarations and
// contract in include/tiledattn.h).  Same validation and kernel choice as the
// square forward and backward, plus the mask's seed and threshold.
//
// Dropout (page "22. GPU Engineering: Correctness, Throughput, and Attention",
// sec. 22.5: only with reproducible masks): the mask is a pure function of
// (seed, head, query row, key), drawn from Philox-4x32-10 (attn_common.hpp),
// so the forward and every backward kernel regenerate the same bits without
// storing them.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "attn_fwd_kernel.hpp"
#include "tiledattn.h"

namespace {

constexpr int kMaxN = 1 << 22;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

tiledattn::DropoutArgs make_args(uint64_t seed, int t) {
  tiledattn::DropoutArgs a;
  a.seed_lo = (uint32_t)seed;
  a.seed_hi = (uint32_t)(seed >> 32);
  a.t = (uint32_t)t;
  a.keep_scale = (float)(256.0 / (256.0 - (double)t));
  return a;
}

template <int D, bool CAUSAL>
int launch_fwd(const void* q, const void* k, const void* v, float* o, float* lse, int bh, int N,
               float scale_log2, tiledattn::DropoutArgs dr, hipStream_t stream) {
  const int n_qt = (N + tiledattn::kBM - 1) / tiledattn::kBM;
  const dim3 grid((unsigned)(bh * n_qt));
  const dim3 block(tiledattn::kThreads);
  const uint16_t* vv = static_cast<const uint16_t*>(v);
  if (scale_log2 > 0.f)
    tiledattn::attn_fwd_kernel<D, D, CAUSAL, true, false, false, true><<<grid, block, 0, stream>>>(
        q, k, vv, o, lse, bh, N, N, 0, n_qt, scale_log2, nullptr, nullptr, dr);
  else
    tiledattn::attn_fwd_kernel<D, D, CAUSAL, false, false, false, true><<<grid, block, 0, stream>>>(
        q, k, vv, o, lse, bh, N, N, 0, n_qt, scale_log2, nullptr, nullptr, dr);
  return hipGetLastError() == hipSuccess ? TA_OK : TA_ERR_HIP;
}

}  // namespace

extern "C" int attn_fwd_dropout(const void* q, const void* k, const void* v, float* o, float* lse,
                                int B, int H, int N, int d, float scale, int causal,
                                uint64_t seed, int drop_t, void* stream) {
  if (!q || !k || !v || !o || !lse) return TA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || N < 1 || N > kMaxN) return TA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return TA_ERR_INVALID_ARG;
  if (drop_t < 0 || drop_t > 255) return TA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return TA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return TA_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return TA_ERR_MISALIGNED;
  const int64_t bh = (int64_t)B * H;
  const int64_t n_qt = (N + tiledattn::kBM - 1) / tiledattn::kBM;
  if (bh * n_qt > INT32_MAX) return TA_ERR_INVALID_ARG;
  const float scale_log2 = (float)((double)scale * 1.4426950408889634073599);
  const tiledattn::DropoutArgs dr = make_args(seed, drop_t);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int ibh = (int)bh;
  if (d == 64)
    return causal ? launch_fwd<64, true>(q, k, v, o, lse, ibh, N, scale_log2, dr, s)
                  : launch_fwd<64, false>(q, k, v, o, lse, ibh, N, scale_log2, dr, s);
  return causal ? launch_fwd<128, true>(q, k, v, o, lse, ibh, N, scale_log2, dr, s)
                : launch_fwd<128, false>(q, k, v, o, lse, ibh, N, scale_log2, dr, s);
}
