// C ABI of the fused attention forward (declarations and contract in
// include/tiledattn.h).  Validates arguments before touching the HIP runtime,
// picks the kernel instance for (head dims, causal, sign of the scale,
// dropout) and enqueues it on the caller's stream.
//
// Dropout (page "22. GPU Engineering: Correctness, Throughput, and Attention",
// sec. 22.5: only with reproducible masks): the mask is a pure function of
// (seed, head, query row, key), drawn from Philox-4x32-10 (attn_common.hpp),
// so the backward regenerates the same bits without storing them.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "attn_fwd_kernel.hpp"
#include "tiledattn.h"

namespace {

constexpr int kMaxN = 1 << 22;
constexpr int kMaxOffset = 1 << 30;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

template <int D, int DV, bool CAUSAL, bool GENERAL>
int launch(const void* q, const void* k, const void* v, float* o, float* lse, int bh, int Nq,
           int Nk, int offset, float scale_log2, const tiledattn::DropoutArgs* dr,
           hipStream_t stream) {
  const int n_qt = (Nq + tiledattn::kBM - 1) / tiledattn::kBM;
  const dim3 grid((unsigned)(bh * n_qt));
  const dim3 block(tiledattn::kThreads);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(k);
  const uint16_t* vv = static_cast<const uint16_t*>(v);
  // A positive scale lets the row maximum be taken on raw scores (one fused
  // multiply-add per exponent); zero or negative scales take the scaled path.
  if constexpr (!GENERAL && D == DV) {
    if (dr) {
      if (scale_log2 > 0.f)
        tiledattn::attn_fwd_kernel<D, D, CAUSAL, true, false, false, true>
            <<<grid, block, 0, stream>>>(qq, kk, vv, o, lse, bh, Nq, Nk, 0, n_qt, scale_log2,
                                         nullptr, nullptr, *dr);
      else
        tiledattn::attn_fwd_kernel<D, D, CAUSAL, false, false, false, true>
            <<<grid, block, 0, stream>>>(qq, kk, vv, o, lse, bh, Nq, Nk, 0, n_qt, scale_log2,
                                         nullptr, nullptr, *dr);
      return hipGetLastError() == hipSuccess ? TA_OK : TA_ERR_HIP;
    }
  }
  if (scale_log2 > 0.f)
    tiledattn::attn_fwd_kernel<D, DV, CAUSAL, true, GENERAL><<<grid, block, 0, stream>>>(
        qq, kk, vv, o, lse, bh, Nq, Nk, offset, n_qt, scale_log2, nullptr, nullptr,
        tiledattn::DropoutArgs{});
  else
    tiledattn::attn_fwd_kernel<D, DV, CAUSAL, false, GENERAL><<<grid, block, 0, stream>>>(
        qq, kk, vv, o, lse, bh, Nq, Nk, offset, n_qt, scale_log2, nullptr, nullptr,
        tiledattn::DropoutArgs{});
  return hipGetLastError() == hipSuccess ? TA_OK : TA_ERR_HIP;
}

template <int D, int DV, bool GENERAL>
int launch_mask(const void* q, const void* k, const void* v, float* o, float* lse, int bh,
                int Nq, int Nk, int offset, float scale_log2, int causal,
                const tiledattn::DropoutArgs* dr, hipStream_t s) {
  return causal
             ? launch<D, DV, true, GENERAL>(q, k, v, o, lse, bh, Nq, Nk, offset, scale_log2, dr, s)
             : launch<D, DV, false, GENERAL>(q, k, v, o, lse, bh, Nq, Nk, offset, scale_log2, dr, s);
}

// Shared by attn_fwd (square = true: the instance with Nk = Nq and offset 0
// fixed at compile time), attn_fwd_dropout (square, dr set) and attn_fwd_ex:
// every check happens before any HIP call.
int forward(const void* q, const void* k, const void* v, float* o, float* lse, int B, int H,
            int Nq, int Nk, int d, int dv, int offset, float scale, int causal, void* stream,
            bool square, const tiledattn::DropoutArgs* dr = nullptr) {
  if (B < 1 || H < 1 || Nq < 0 || Nq > kMaxN || Nk < 0 || Nk > kMaxN) return TA_ERR_INVALID_ARG;
  // A pointer may be NULL only where its tensor is empty.
  if ((Nq > 0 && (!q || !o || !lse)) || (Nk > 0 && (!k || !v))) return TA_ERR_INVALID_ARG;
  if (offset < 0 || offset > kMaxOffset) return TA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return TA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return TA_ERR_INVALID_ARG;
  if ((d != 64 && d != 128) || (dv != 64 && dv != 128)) return TA_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return TA_ERR_MISALIGNED;
  const int64_t bh = (int64_t)B * H;
  const int64_t n_qt = (Nq + tiledattn::kBM - 1) / tiledattn::kBM;
  if (bh * n_qt > INT32_MAX) return TA_ERR_INVALID_ARG;
  if (Nq == 0) return TA_OK;                       // nothing to compute

  // Scores enter exp2: fold log2(e) into the scale once, in double.
  const float scale_log2 = (float)((double)scale * 1.4426950408889634073599);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int ibh = (int)bh;
  if (square)
    return d == 64
               ? launch_mask<64, 64, false>(q, k, v, o, lse, ibh, Nq, Nk, 0, scale_log2, causal, dr, s)
               : launch_mask<128, 128, false>(q, k, v, o, lse, ibh, Nq, Nk, 0, scale_log2, causal, dr,
                                              s);
  if (d == 64)
    return dv == 64 ? launch_mask<64, 64, true>(q, k, v, o, lse, ibh, Nq, Nk, offset, scale_log2,
                                                causal, nullptr, s)
                    : launch_mask<64, 128, true>(q, k, v, o, lse, ibh, Nq, Nk, offset, scale_log2,
                                                 causal, nullptr, s);
  return dv == 64 ? launch_mask<128, 64, true>(q, k, v, o, lse, ibh, Nq, Nk, offset, scale_log2,
                                               causal, nullptr, s)
                  : launch_mask<128, 128, true>(q, k, v, o, lse, ibh, Nq, Nk, offset, scale_log2,
                                                causal, nullptr, s);
}

}  // namespace

extern "C" int attn_fwd(const void* q, const void* k, const void* v, float* o, float* lse, int B,
                        int H, int N, int d, float scale, int causal, void* stream) {
  if (N < 1) return TA_ERR_INVALID_ARG;
  return forward(q, k, v, o, lse, B, H, N, N, d, d, 0, scale, causal, stream, true);
}

extern "C" int attn_fwd_dropout(const void* q, const void* k, const void* v, float* o, float* lse,
                                int B, int H, int N, int d, float scale, int causal,
                                uint64_t seed, int drop_t, void* stream) {
  if (N < 1 || drop_t < 0 || drop_t > 255) return TA_ERR_INVALID_ARG;
  tiledattn::DropoutArgs dr;
  dr.seed_lo = (uint32_t)seed;
  dr.seed_hi = (uint32_t)(seed >> 32);
  dr.t = (uint32_t)drop_t;
  dr.keep_scale = (float)(256.0 / (256.0 - (double)drop_t));
  return forward(q, k, v, o, lse, B, H, N, N, d, d, 0, scale, causal, stream, true, &dr);
}

extern "C" int attn_fwd_ex(const void* q, const void* k, const void* v, float* o, float* lse,
                           int B, int H, int Nq, int Nk, int d, int dv, int query_offset,
                           float scale, int causal, void* stream) {
  return forward(q, k, v, o, lse, B, H, Nq, Nk, d, dv, query_offset, scale, causal, stream, false);
}

extern "C" const char* attn_status_string(int status) {
  switch (status) {
    case TA_OK: return "ok";
    case TA_ERR_INVALID_ARG:
      return "invalid argument (size, offset, flag, pointer or scale out of range)";
    case TA_ERR_UNSUPPORTED: return "unsupported head dimension (64 or 128 only)";
    case TA_ERR_MISALIGNED: return "misaligned pointer (q, k, v, o need 16 bytes; lse 4 bytes)";
    case TA_ERR_HIP: return "HIP runtime error at launch";
    default: return "unknown status";
  }
}
