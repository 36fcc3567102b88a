// C ABI of the attention backward (declarations and contract in
// include/tiledattn.h).  Validates arguments before touching the HIP runtime,
// then enqueues the row-statistics kernel, the dK/dV kernel and the dQ kernel
// on the caller's stream.  attn_bwd_dropout runs the same kernels with the
// forward's dropout mask regenerated from its seed (attn_common.hpp);
// attn_bwd_ex runs their general-shape instances (Nq != Nk, a query offset,
// dv != d).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "attn_bwd_kernel.hpp"
#include "tiledattn.h"

namespace {

constexpr int kMaxN = 1 << 22;
constexpr int kMaxOffset = 1 << 30;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Rows of one head's statistics planes, padded to a multiple of 4 (each
// plane 16-byte aligned).
int64_t stats_stride(int N) { return ((int64_t)N + 3) & ~(int64_t)3; }

struct Shape {
  int bh, Nq, Nk, offset;
};

template <int D, int DV, bool CAUSAL, bool GENERAL, bool DROPOUT>
int launch(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* o,
           const float* lse, const uint16_t* g, float* dq, float* dk, float* dv,
           float* stats, Shape sh, float scale, tiledattn::DropoutArgs dr,
           hipStream_t stream) {
  using namespace tiledattn;
  const int stride = (int)stats_stride(sh.Nq);
  const int64_t rows = (int64_t)sh.bh * sh.Nq;
  const float c = (float)((double)scale * 1.4426950408889634073599);
  // A grid of zero workgroups is a launch error: with no query rows the
  // statistics and dQ kernels have nothing to do, and with no keys dK/dV is
  // empty (the dK/dV kernel still writes zeros for every key when Nq = 0).
  if (rows > 0) {
    const unsigned prep_blocks = (unsigned)((rows + kPrepRowsPerBlock - 1) / kPrepRowsPerBlock);
    attn_bwd_prep_kernel<DV><<<dim3(prep_blocks), dim3(256), 0, stream>>>(o, g, lse, stats,
                                                                          sh.Nq, stride, rows);
  }
  if (sh.Nk > 0) {
    const int n_kt = (sh.Nk + kBM - 1) / kBM;
    attn_bwd_dkdv_kernel<D, DV, CAUSAL, GENERAL, DROPOUT>
        <<<dim3((unsigned)(sh.bh * n_kt)), dim3(kThreads), 0, stream>>>(
            q, k, v, g, stats, dk, dv, sh.bh, sh.Nq, sh.Nk, sh.offset, stride, n_kt, c, scale,
            INT32_MIN, dr);
  }
  if (sh.Nq > 0) {
    const int n_qt = (sh.Nq + kBM - 1) / kBM;
    attn_bwd_dq_kernel<D, DV, CAUSAL, GENERAL, DROPOUT>
        <<<dim3((unsigned)(sh.bh * n_qt)), dim3(kThreads), 0, stream>>>(
            q, k, v, g, stats, dq, sh.bh, sh.Nq, sh.Nk, sh.offset, stride, n_qt, c, scale,
            INT32_MAX, dr);
  }
  return hipGetLastError() == hipSuccess ? TA_OK : TA_ERR_HIP;
}

template <int D, int DV, bool GENERAL, bool DROPOUT>
int launch_mask(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* o,
                const float* lse, const uint16_t* g, float* dq, float* dk, float* dv,
                float* st, Shape sh, float scale, int causal,
                tiledattn::DropoutArgs dr, hipStream_t s) {
  return causal ? launch<D, DV, true, GENERAL, DROPOUT>(q, k, v, o, lse, g, dq, dk, dv, st, sh,
                                                        scale, dr, s)
                : launch<D, DV, false, GENERAL, DROPOUT>(q, k, v, o, lse, g, dq, dk, dv, st, sh,
                                                         scale, dr, s);
}

// Row counts a call may take: grids stay within int32 workgroups and the
// row-statistics grid (16 rows per workgroup) below 2^32 workgroups.
bool valid_rows(int B, int H, int N, bool allow_empty) {
  if (B < 1 || H < 1 || N < (allow_empty ? 0 : 1) || N > kMaxN) return false;
  const int64_t bh = (int64_t)B * H;
  const int64_t n_t = (N + tiledattn::kBM - 1) / tiledattn::kBM;
  if (bh * n_t > INT32_MAX) return false;
  return bh * stats_stride(N) <= ((int64_t)1 << 34);
}

// Argument checks of every backward entry point (no HIP call).
int check_backward(const void* q, const void* k, const void* v, const float* o, const float* lse,
                   const void* dout, float* dq, float* dk, float* dv, const void* workspace,
                   int B, int H, int Nq, int Nk, int d, int dvw, int offset, float scale,
                   int causal, bool square) {
  if (!valid_rows(B, H, Nq, !square) || !valid_rows(B, H, Nk, !square)) return TA_ERR_INVALID_ARG;
  // A pointer may be NULL only where its tensor is empty.
  if ((Nq > 0 && (!q || !o || !lse || !dout || !dq || !workspace)) ||
      (Nk > 0 && (!k || !v || !dk || !dv)))
    return TA_ERR_INVALID_ARG;
  if (offset < 0 || offset > kMaxOffset) return TA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return TA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return TA_ERR_INVALID_ARG;
  if ((d != 64 && d != 128) || (dvw != 64 && dvw != 128)) return TA_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
      !aligned(workspace, 16) || !aligned(lse, 4))
    return TA_ERR_MISALIGNED;
  return TA_OK;
}

// Shared by attn_bwd and attn_bwd_dropout (square = true: the instances with
// Nk = Nq, offset 0 and dv = d fixed at compile time), attn_bwd_ex and
// attn_bwd_noalloc: every check happens before any HIP call.
template <bool DROPOUT>
int backward(const void* q, const void* k, const void* v, const float* o, const float* lse,
             const void* dout, float* dq, float* dk, float* dv, void* workspace, int B, int H,
             int Nq, int Nk, int d, int dvw, int offset, float scale, int causal,
             tiledattn::DropoutArgs dr, void* stream, bool square) {
  const int chk = check_backward(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, H, Nq, Nk, d,
                                 dvw, offset, scale, causal, square);
  if (chk != TA_OK) return chk;
  if (Nq == 0 && Nk == 0) return TA_OK;

  const Shape sh{B * H, Nq, Nk, offset};
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto* qq = static_cast<const uint16_t*>(q);
  auto* kk = static_cast<const uint16_t*>(k);
  auto* vv = static_cast<const uint16_t*>(v);
  auto* gg = static_cast<const uint16_t*>(dout);
  auto* st = static_cast<float*>(workspace);
  if (square)
    return d == 64 ? launch_mask<64, 64, false, DROPOUT>(qq, kk, vv, o, lse, gg, dq, dk, dv, st,
                                                         sh, scale, causal, dr, s)
                   : launch_mask<128, 128, false, DROPOUT>(qq, kk, vv, o, lse, gg, dq, dk, dv, st,
                                                           sh, scale, causal, dr, s);
  if (d == 64)
    return dvw == 64 ? launch_mask<64, 64, true, DROPOUT>(qq, kk, vv, o, lse, gg, dq, dk, dv, st,
                                                          sh, scale, causal, dr, s)
                     : launch_mask<64, 128, true, DROPOUT>(qq, kk, vv, o, lse, gg, dq, dk, dv, st,
                                                           sh, scale, causal, dr, s);
  return dvw == 64 ? launch_mask<128, 64, true, DROPOUT>(qq, kk, vv, o, lse, gg, dq, dk, dv, st,
                                                         sh, scale, causal, dr, s)
                   : launch_mask<128, 128, true, DROPOUT>(qq, kk, vv, o, lse, gg, dq, dk, dv, st,
                                                          sh, scale, causal, dr, s);
}

tiledattn::DropoutArgs dropout_args(uint64_t seed, int drop_t) {
  tiledattn::DropoutArgs dr;
  dr.seed_lo = (uint32_t)seed;
  dr.seed_hi = (uint32_t)(seed >> 32);
  dr.t = (uint32_t)drop_t;
  dr.keep_scale = (float)(256.0 / (256.0 - (double)drop_t));
  return dr;
}

// The library's own device scratch for attn_bwd_noalloc: the row statistics
// live here instead of in a caller workspace.  Each device that runs the
// library holds its own copy for the life of the process.  In host code the
// name `scratch` is only a stand-in for the symbol; its device address comes
// from hipGetSymbolAddress, once per device, and only that address is used.
constexpr size_t kScratchBytes = (size_t)16 << 20;
constexpr int kMaxDevices = 64;
__device__ __attribute__((aligned(256))) uint8_t scratch[kScratchBytes];

int scratch_address(void** out) {
  static std::mutex mu;
  static void* table[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TA_ERR_HIP;
  std::lock_guard<std::mutex> lock(mu);
  if (!table[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TA_ERR_HIP;
    table[dev] = p;
  }
  *out = table[dev];
  return TA_OK;
}

}  // namespace

extern "C" size_t attn_bwd_workspace_size(int B, int H, int N) {
  if (!valid_rows(B, H, N, true)) return 0;
  return (size_t)B * (size_t)H * (size_t)stats_stride(N) * 8u;
}

extern "C" int attn_bwd(const void* q, const void* k, const void* v, const float* o,
                        const float* lse, const void* dout, float* dq, float* dk, float* dv,
                        void* workspace, int B, int H, int N, int d, float scale, int causal,
                        void* stream) {
  return backward<false>(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, H, N, N, d, d, 0, scale,
                         causal, tiledattn::DropoutArgs{}, stream, true);
}

extern "C" int attn_bwd_ex(const void* q, const void* k, const void* v, const float* o,
                           const float* lse, const void* dout, float* dq, float* dk, float* dv,
                           void* workspace, int B, int H, int Nq, int Nk, int d, int dv_width,
                           int query_offset, float scale, int causal, void* stream) {
  return backward<false>(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, H, Nq, Nk, d, dv_width,
                         query_offset, scale, causal, tiledattn::DropoutArgs{}, stream, false);
}

extern "C" int attn_bwd_dropout_ex(const void* q, const void* k, const void* v, const float* o,
                                   const float* lse, const void* dout, float* dq, float* dk,
                                   float* dv, void* workspace, int B, int H, int Nq, int Nk, int d,
                                   int dv_width, int query_offset, float scale, int causal,
                                   uint64_t seed, int drop_t, void* stream) {
  if (drop_t < 0 || drop_t > 255) return TA_ERR_INVALID_ARG;
  return backward<true>(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, H, Nq, Nk, d, dv_width,
                        query_offset, scale, causal, dropout_args(seed, drop_t), stream, false);
}

extern "C" int attn_bwd_dropout(const void* q, const void* k, const void* v, const float* o,
                                const float* lse, const void* dout, float* dq, float* dk,
                                float* dv, void* workspace, int B, int H, int N, int d,
                                float scale, int causal, uint64_t seed, int drop_t,
                                void* stream) {
  if (drop_t < 0 || drop_t > 255) return TA_ERR_INVALID_ARG;
  return backward<true>(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, H, N, N, d, d, 0, scale,
                        causal, dropout_args(seed, drop_t), stream, true);
}

extern "C" int attn_bwd_noalloc(const void* q, const void* k, const void* v, const float* o,
                                const float* lse, const void* dout, float* dq, float* dk,
                                float* dv, int B, int H, int N, int d, float scale, int causal,
                                void* stream) {
  // Every argument check before any HIP call; the scratch stands in for the
  // workspace (a non-NULL, aligned placeholder address for the checks, never
  // dereferenced).
  const void* placeholder = reinterpret_cast<const void*>((uintptr_t)256);
  const int chk = check_backward(q, k, v, o, lse, dout, dq, dk, dv, placeholder, B, H, N, N, d, d,
                                 0, scale, causal, true);
  if (chk != TA_OK) return chk;
  if ((size_t)B * (size_t)H * (size_t)stats_stride(N) * 8u > kScratchBytes)
    return TA_ERR_TOO_LARGE;
  void* ws = nullptr;
  const int st = scratch_address(&ws);
  if (st != TA_OK) return st;
  return backward<false>(q, k, v, o, lse, dout, dq, dk, dv, ws, B, H, N, N, d, d, 0, scale, causal,
                         tiledattn::DropoutArgs{}, stream, true);
}
