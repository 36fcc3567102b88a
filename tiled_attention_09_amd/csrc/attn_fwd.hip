// C ABI of the fused attention forward (declarations and contract in
// include/tiledattn.h).  Validates arguments before touching the HIP runtime,
// picks the kernel instance for (head dim, causal) and enqueues it on the
// caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "attn_fwd_kernel.hpp"
#include "tiledattn.h"

namespace {

constexpr int kMaxN = 1 << 22;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

template <int D, bool CAUSAL>
int launch(const void* q, const void* k, const void* v, float* o, float* lse, int bh, int N,
           int n_qt, float scale_log2, hipStream_t stream) {
  const dim3 grid((unsigned)(bh * n_qt));
  const dim3 block(tiledattn::kThreads);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(k);
  const uint16_t* vv = static_cast<const uint16_t*>(v);
  // A positive scale lets the row maximum be taken on raw scores (one fused
  // multiply-add per exponent); zero or negative scales take the scaled path.
  if (scale_log2 > 0.f)
    tiledattn::attn_fwd_kernel<D, CAUSAL, true><<<grid, block, 0, stream>>>(
        qq, kk, vv, o, lse, bh, N, n_qt, scale_log2);
  else
    tiledattn::attn_fwd_kernel<D, CAUSAL, false><<<grid, block, 0, stream>>>(
        qq, kk, vv, o, lse, bh, N, n_qt, scale_log2);
  return hipGetLastError() == hipSuccess ? TA_OK : TA_ERR_HIP;
}

}  // namespace

extern "C" int attn_fwd(const void* q, const void* k, const void* v, float* o, float* lse, int B,
                        int H, int N, int d, float scale, int causal, void* stream) {
  if (!q || !k || !v || !o || !lse) return TA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || N < 1 || N > kMaxN) return TA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return TA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return TA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return TA_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return TA_ERR_MISALIGNED;
  const int64_t bh = (int64_t)B * H;
  const int64_t n_qt = (N + tiledattn::kBM - 1) / tiledattn::kBM;
  if (bh * n_qt > INT32_MAX) return TA_ERR_INVALID_ARG;

  // Scores enter exp2: fold log2(e) into the scale once, in double.
  const float scale_log2 = (float)((double)scale * 1.4426950408889634073599);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int ibh = (int)bh, iqt = (int)n_qt;
  if (d == 64)
    return causal ? launch<64, true>(q, k, v, o, lse, ibh, N, iqt, scale_log2, s)
                  : launch<64, false>(q, k, v, o, lse, ibh, N, iqt, scale_log2, s);
  return causal ? launch<128, true>(q, k, v, o, lse, ibh, N, iqt, scale_log2, s)
                : launch<128, false>(q, k, v, o, lse, ibh, N, iqt, scale_log2, s);
}

extern "C" const char* attn_status_string(int status) {
  switch (status) {
    case TA_OK: return "ok";
    case TA_ERR_INVALID_ARG: return "invalid argument (size, flag, pointer or scale out of range)";
    case TA_ERR_UNSUPPORTED: return "unsupported head dimension (64 or 128 only)";
    case TA_ERR_MISALIGNED: return "misaligned pointer (q, k, v, o need 16 bytes; lse 4 bytes)";
    case TA_ERR_HIP: return "HIP runtime error at launch";
    default: return "unknown status";
  }
}
