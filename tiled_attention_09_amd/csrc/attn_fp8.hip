// C ABI of the FP8-score forward and of the per-head FP8 quantiser
// (declarations and contract in include/tiledattn.h).  Arguments are checked
// before any HIP call.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "attn_fp8_quant.hpp"
#include "attn_fwd_kernel.hpp"
#include "tiledattn.h"

namespace {

constexpr int kMaxN = 1 << 22;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

template <int D, int DV, bool CAUSAL, bool GENERAL>
int launch_fp8(const void* q8, const void* k8, const void* v, float* o, float* lse,
               const float* qd, const float* kd, int bh, int Nq, int Nk, int offset,
               float scale_log2, hipStream_t stream) {
  const int n_qt = (Nq + tiledattn::kBM - 1) / tiledattn::kBM;
  const dim3 grid((unsigned)(bh * n_qt));
  const dim3 block(tiledattn::kThreads);
  const uint16_t* vv = static_cast<const uint16_t*>(v);
  if (scale_log2 > 0.f)
    tiledattn::attn_fwd_kernel<D, DV, CAUSAL, true, GENERAL, true><<<grid, block, 0, stream>>>(
        q8, k8, vv, o, lse, bh, Nq, Nk, offset, n_qt, scale_log2, qd, kd, tiledattn::DropoutArgs{},
        bh, 0);
  else
    tiledattn::attn_fwd_kernel<D, DV, CAUSAL, false, GENERAL, true><<<grid, block, 0, stream>>>(
        q8, k8, vv, o, lse, bh, Nq, Nk, offset, n_qt, scale_log2, qd, kd, tiledattn::DropoutArgs{},
        bh, 0);
  return hipGetLastError() == hipSuccess ? TA_OK : TA_ERR_HIP;
}

template <int D, int DV, bool GENERAL>
int launch_fp8_mask(const void* q8, const void* k8, const void* v, float* o, float* lse,
                    const float* qd, const float* kd, int bh, int Nq, int Nk, int offset,
                    float scale_log2, int causal, hipStream_t s) {
  return causal ? launch_fp8<D, DV, true, GENERAL>(q8, k8, v, o, lse, qd, kd, bh, Nq, Nk,
                                                   offset, scale_log2, s)
                : launch_fp8<D, DV, false, GENERAL>(q8, k8, v, o, lse, qd, kd, bh, Nq, Nk,
                                                    offset, scale_log2, s);
}

}  // namespace

extern "C" int attn_fwd_fp8(const void* q8, const void* k8, const void* v, float* o, float* lse,
                            const float* q_descale, const float* k_descale, int B, int H, int N,
                            int d, float scale, int causal, void* stream) {
  if (!q8 || !k8 || !v || !o || !lse || !q_descale || !k_descale) return TA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || N < 1 || N > kMaxN) return TA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return TA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return TA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return TA_ERR_UNSUPPORTED;
  if (!aligned(q8, 16) || !aligned(k8, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(lse, 4) || !aligned(q_descale, 4) || !aligned(k_descale, 4))
    return TA_ERR_MISALIGNED;
  const int64_t bh = (int64_t)B * H;
  const int64_t n_qt = (N + tiledattn::kBM - 1) / tiledattn::kBM;
  if (bh * n_qt > INT32_MAX) return TA_ERR_INVALID_ARG;
  const float scale_log2 = (float)((double)scale * 1.4426950408889634073599);
  hipStream_t s = static_cast<hipStream_t>(stream);
  return d == 64 ? launch_fp8_mask<64, 64, false>(q8, k8, v, o, lse, q_descale, k_descale,
                                                  (int)bh, N, N, 0, scale_log2, causal, s)
                 : launch_fp8_mask<128, 128, false>(q8, k8, v, o, lse, q_descale, k_descale,
                                                    (int)bh, N, N, 0, scale_log2, causal, s);
}

extern "C" int attn_fwd_fp8_ex(const void* q8, const void* k8, const void* v, float* o,
                               float* lse, const float* q_descale, const float* k_descale, int B,
                               int H, int Nq, int Nk, int d, int dv, int query_offset, float scale,
                               int causal, void* stream) {
  if (B < 1 || H < 1 || Nq < 0 || Nq > kMaxN || Nk < 0 || Nk > kMaxN) return TA_ERR_INVALID_ARG;
  // A pointer may be NULL only where its tensor is empty; the descales are per head.
  if ((Nq > 0 && (!q8 || !o || !lse || !q_descale || !k_descale)) || (Nk > 0 && (!k8 || !v)))
    return TA_ERR_INVALID_ARG;
  if (query_offset < 0 || query_offset > (1 << 30)) return TA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return TA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return TA_ERR_INVALID_ARG;
  if ((d != 64 && d != 128) || (dv != 64 && dv != 128)) return TA_ERR_UNSUPPORTED;
  if (!aligned(q8, 16) || !aligned(k8, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(lse, 4) || !aligned(q_descale, 4) || !aligned(k_descale, 4))
    return TA_ERR_MISALIGNED;
  const int64_t bh = (int64_t)B * H;
  const int64_t n_qt = (Nq + tiledattn::kBM - 1) / tiledattn::kBM;
  if (bh * n_qt > INT32_MAX) return TA_ERR_INVALID_ARG;
  if (Nq == 0) return TA_OK;
  const float scale_log2 = (float)((double)scale * 1.4426950408889634073599);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int bhi = (int)bh;
  if (d == 64)
    return dv == 64 ? launch_fp8_mask<64, 64, true>(q8, k8, v, o, lse, q_descale, k_descale, bhi,
                                                    Nq, Nk, query_offset, scale_log2, causal, s)
                    : launch_fp8_mask<64, 128, true>(q8, k8, v, o, lse, q_descale, k_descale, bhi,
                                                     Nq, Nk, query_offset, scale_log2, causal, s);
  return dv == 64 ? launch_fp8_mask<128, 64, true>(q8, k8, v, o, lse, q_descale, k_descale, bhi,
                                                   Nq, Nk, query_offset, scale_log2, causal, s)
                  : launch_fp8_mask<128, 128, true>(q8, k8, v, o, lse, q_descale, k_descale, bhi,
                                                    Nq, Nk, query_offset, scale_log2, causal, s);
}

extern "C" int attn_quantize_fp8(const void* x, void* out, float* descale, int heads, int rows,
                                 int d, void* stream) {
  if (!x || !out || !descale) return TA_ERR_INVALID_ARG;
  if (heads < 1 || rows < 1 || rows > kMaxN) return TA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return TA_ERR_UNSUPPORTED;
  if (!aligned(x, 16) || !aligned(out, 16) || !aligned(descale, 4)) return TA_ERR_MISALIGNED;
  const int64_t n = (int64_t)rows * d;          // a multiple of 64
  const int64_t chunks = (n + tiledattn::kQuantPerBlock - 1) / tiledattn::kQuantPerBlock;
  if (heads > 65535 || chunks > INT32_MAX) return TA_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto* bits = reinterpret_cast<uint32_t*>(descale);
  const auto* xx = static_cast<const uint16_t*>(x);
  const unsigned hb = (unsigned)((heads + 255) / 256);
  tiledattn::fp8_amax_init_kernel<<<dim3(hb), dim3(256), 0, s>>>(bits, heads);
  const int64_t amax_chunks = (n + tiledattn::kAmaxPerBlock - 1) / tiledattn::kAmaxPerBlock;
  const int64_t amax_blocks = amax_chunks < tiledattn::kAmaxBlocksPerHead
                                  ? amax_chunks : tiledattn::kAmaxBlocksPerHead;
  tiledattn::fp8_amax_kernel<<<dim3((unsigned)amax_blocks, (unsigned)heads),
                               dim3(tiledattn::kQuantThreads), 0, s>>>(xx, bits, n);
  const dim3 grid((unsigned)chunks, (unsigned)heads);
  tiledattn::fp8_quant_kernel<<<grid, dim3(tiledattn::kQuantThreads), 0, s>>>(
      xx, static_cast<uint8_t*>(out), bits, n);
  tiledattn::fp8_descale_kernel<<<dim3(hb), dim3(256), 0, s>>>(bits, heads);
  return hipGetLastError() == hipSuccess ? TA_OK : TA_ERR_HIP;
}
