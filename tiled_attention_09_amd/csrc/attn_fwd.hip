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
  if (dr) {
    if (scale_log2 > 0.f)
      tiledattn::attn_fwd_kernel<D, DV, CAUSAL, true, GENERAL, false, true>
          <<<grid, block, 0, stream>>>(qq, kk, vv, o, lse, bh, Nq, Nk, offset, n_qt, scale_log2,
                                       nullptr, nullptr, *dr, bh, 0);
    else
      tiledattn::attn_fwd_kernel<D, DV, CAUSAL, false, GENERAL, false, true>
          <<<grid, block, 0, stream>>>(qq, kk, vv, o, lse, bh, Nq, Nk, offset, n_qt, scale_log2,
                                       nullptr, nullptr, *dr, bh, 0);
    return hipGetLastError() == hipSuccess ? TA_OK : TA_ERR_HIP;
  }
  if (scale_log2 > 0.f)
    tiledattn::attn_fwd_kernel<D, DV, CAUSAL, true, GENERAL><<<grid, block, 0, stream>>>(
        qq, kk, vv, o, lse, bh, Nq, Nk, offset, n_qt, scale_log2, nullptr, nullptr,
        tiledattn::DropoutArgs{}, bh, 0);
  else
    tiledattn::attn_fwd_kernel<D, DV, CAUSAL, false, GENERAL><<<grid, block, 0, stream>>>(
        qq, kk, vv, o, lse, bh, Nq, Nk, offset, n_qt, scale_log2, nullptr, nullptr,
        tiledattn::DropoutArgs{}, bh, 0);
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

// Argument checks of every forward entry point, before any HIP call.
int check(const void* q, const void* k, const void* v, float* o, float* lse, int B, int H,
          int Nq, int Nk, int d, int dv, int offset, float scale, int causal) {
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
  return TA_OK;
}

// Shared by attn_fwd (square = true: the instance with Nk = Nq and offset 0
// fixed at compile time), attn_fwd_dropout (square, dr set), attn_fwd_ex and
// attn_fwd_dropout_ex (general, dr set).
int forward(const void* q, const void* k, const void* v, float* o, float* lse, int B, int H,
            int Nq, int Nk, int d, int dv, int offset, float scale, int causal, void* stream,
            bool square, const tiledattn::DropoutArgs* dr = nullptr) {
  const int st = check(q, k, v, o, lse, B, H, Nq, Nk, d, dv, offset, scale, causal);
  if (st != TA_OK) return st;
  const int64_t bh = (int64_t)B * H;
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
                                                causal, dr, s)
                    : launch_mask<64, 128, true>(q, k, v, o, lse, ibh, Nq, Nk, offset, scale_log2,
                                                 causal, dr, s);
  return dv == 64 ? launch_mask<128, 64, true>(q, k, v, o, lse, ibh, Nq, Nk, offset, scale_log2,
                                               causal, dr, s)
                  : launch_mask<128, 128, true>(q, k, v, o, lse, ibh, Nq, Nk, offset, scale_log2,
                                                causal, dr, s);
}

tiledattn::DropoutArgs dropout_args(uint64_t seed, int drop_t) {
  tiledattn::DropoutArgs dr;
  dr.seed_lo = (uint32_t)seed;
  dr.seed_hi = (uint32_t)(seed >> 32);
  dr.t = (uint32_t)drop_t;
  dr.keep_scale = (float)(256.0 / (256.0 - (double)drop_t));
  return dr;
}

// Split key ranges (attn_fwd_split): when the (head, query tile) grid is too
// small to fill the chip -- a decoding step of a few sequences over a long
// context -- the keys are split over workgroups, each covering an even number
// (>= 4) of key tiles.  Grids below one workgroup per compute unit are split
// up to kSplitFill workgroups (one per CU streaming a long key range measured
// best: 16 queries over 32768 keys in 16 heads reached 5.2 TB/s with 256
// workgroups, 4.5 with 512, 3.6 with 1024, 3.7 with 128).  Grids below
// kSplitTwo are split in two only when the partial results are small next to
// the keys and values: two fp32 partial rows of dv values, written and read
// back, per query cost 16 Nq dv bytes against 2 Nk dv bytes of V, so Nq <= Nk/64
// keeps them under an eighth (a chunk of 1024 queries over 8192 keys, which
// moved 2.4x its algorithmic bytes split, runs unsplit).
constexpr int64_t kSplitFill = 256;
constexpr int64_t kSplitTwo = 1024;

struct SplitPlan {
  int n_split, tiles;
};

SplitPlan plan_split(int64_t bh, int Nq, int Nk) {
  const int64_t grid = bh * ((Nq + tiledattn::kBM - 1) / tiledattn::kBM);
  const int n_kt = (Nk + tiledattn::kBN - 1) / tiledattn::kBN;
  if (grid == 0 || grid >= kSplitTwo || n_kt < 8) return {1, n_kt};
  if (grid >= kSplitFill && (int64_t)Nq * 64 > (int64_t)Nk) return {1, n_kt};
  const int64_t want = grid < kSplitFill ? (kSplitFill + grid - 1) / grid : 2;
  int n = (int)(want < n_kt / 4 ? want : n_kt / 4);
  int tiles = (n_kt + n - 1) / n;
  tiles += tiles & 1;
  n = (n_kt + tiles - 1) / tiles;
  return {n, tiles};
}

// Workspace of a split call: the partial O ([n_split][B H Nq][dv] fp32) and
// LSE ([n_split][B H Nq]), each 256-byte aligned; 0 when no split is planned.
size_t split_bytes(int64_t bh, int Nq, int dv, SplitPlan p) {
  if (p.n_split <= 1) return 0;
  const size_t rows = (size_t)p.n_split * (size_t)bh * (size_t)Nq;
  return ((rows * (size_t)dv * 4u + 255u) & ~(size_t)255u) + ((rows * 4u + 255u) & ~(size_t)255u);
}

template <int D, int DV, bool CAUSAL>
int launch_split(const void* q, const void* k, const void* v, float* o, float* lse, int bh,
                 int Nq, int Nk, int offset, float scale_log2, SplitPlan p, float* ws,
                 hipStream_t stream) {
  const int n_qt = (Nq + tiledattn::kBM - 1) / tiledattn::kBM;
  const int64_t rows = (int64_t)bh * Nq;
  float* part_o = ws;
  float* part_l = ws + ((((size_t)p.n_split * rows * DV * 4u + 255u) & ~(size_t)255u) / 4u);
  tiledattn::attn_fwd_kernel<D, DV, CAUSAL, true, true, false, false, true>
      <<<dim3((unsigned)(p.n_split * bh * n_qt)), dim3(tiledattn::kThreads), 0, stream>>>(
          q, k, static_cast<const uint16_t*>(v), part_o, part_l, p.n_split * bh, Nq, Nk, offset,
          n_qt, scale_log2, nullptr, nullptr, tiledattn::DropoutArgs{}, bh, p.tiles);
  tiledattn::attn_split_merge_kernel<DV><<<dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream>>>(
      part_o, part_l, o, lse, rows, p.n_split);
  return hipGetLastError() == hipSuccess ? TA_OK : TA_ERR_HIP;
}

template <int D, int DV>
int launch_split_mask(const void* q, const void* k, const void* v, float* o, float* lse, int bh,
                      int Nq, int Nk, int offset, float scale_log2, int causal, SplitPlan p,
                      float* ws, hipStream_t s) {
  return causal ? launch_split<D, DV, true>(q, k, v, o, lse, bh, Nq, Nk, offset, scale_log2, p, ws, s)
                : launch_split<D, DV, false>(q, k, v, o, lse, bh, Nq, Nk, offset, scale_log2, p, ws,
                                             s);
}

}  // namespace

extern "C" size_t attn_fwd_split_workspace_size(int B, int H, int Nq, int Nk, int dv) {
  if (B < 1 || H < 1 || Nq < 0 || Nq > kMaxN || Nk < 0 || Nk > kMaxN) return 0;
  if (dv != 64 && dv != 128) return 0;
  const int64_t bh = (int64_t)B * H;
  if (bh * ((Nq + tiledattn::kBM - 1) / tiledattn::kBM) > INT32_MAX) return 0;
  return split_bytes(bh, Nq, dv, plan_split(bh, Nq, Nk));
}

extern "C" int attn_fwd_split(const void* q, const void* k, const void* v, float* o, float* lse,
                              int B, int H, int Nq, int Nk, int d, int dv, int query_offset,
                              float scale, int causal, void* workspace, size_t workspace_bytes,
                              void* stream) {
  const int st = check(q, k, v, o, lse, B, H, Nq, Nk, d, dv, query_offset, scale, causal);
  if (st != TA_OK) return st;
  const int64_t bh = (int64_t)B * H;
  const SplitPlan p = plan_split(bh, Nq, Nk);
  const size_t need = split_bytes(bh, Nq, dv, p);
  // Without a split (or with a non-positive scale) this is attn_fwd_ex.
  if (need == 0 || !(scale > 0.f))
    return forward(q, k, v, o, lse, B, H, Nq, Nk, d, dv, query_offset, scale, causal, stream, false);
  if (!workspace || workspace_bytes < need) return TA_ERR_INVALID_ARG;
  if (!aligned(workspace, 256)) return TA_ERR_MISALIGNED;
  if ((int64_t)p.n_split * bh * ((Nq + tiledattn::kBM - 1) / tiledattn::kBM) > INT32_MAX)
    return TA_ERR_INVALID_ARG;
  const float scale_log2 = (float)((double)scale * 1.4426950408889634073599);
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* ws = static_cast<float*>(workspace);
  const int ibh = (int)bh;
  if (d == 64)
    return dv == 64 ? launch_split_mask<64, 64>(q, k, v, o, lse, ibh, Nq, Nk, query_offset,
                                                scale_log2, causal, p, ws, s)
                    : launch_split_mask<64, 128>(q, k, v, o, lse, ibh, Nq, Nk, query_offset,
                                                 scale_log2, causal, p, ws, s);
  return dv == 64 ? launch_split_mask<128, 64>(q, k, v, o, lse, ibh, Nq, Nk, query_offset,
                                               scale_log2, causal, p, ws, s)
                  : launch_split_mask<128, 128>(q, k, v, o, lse, ibh, Nq, Nk, query_offset,
                                                scale_log2, causal, p, ws, s);
}

extern "C" int attn_fwd(const void* q, const void* k, const void* v, float* o, float* lse, int B,
                        int H, int N, int d, float scale, int causal, void* stream) {
  if (N < 1) return TA_ERR_INVALID_ARG;
  return forward(q, k, v, o, lse, B, H, N, N, d, d, 0, scale, causal, stream, true);
}

extern "C" int attn_fwd_dropout(const void* q, const void* k, const void* v, float* o, float* lse,
                                int B, int H, int N, int d, float scale, int causal,
                                uint64_t seed, int drop_t, void* stream) {
  if (N < 1 || drop_t < 0 || drop_t > 255) return TA_ERR_INVALID_ARG;
  const tiledattn::DropoutArgs dr = dropout_args(seed, drop_t);
  return forward(q, k, v, o, lse, B, H, N, N, d, d, 0, scale, causal, stream, true, &dr);
}

extern "C" int attn_fwd_dropout_ex(const void* q, const void* k, const void* v, float* o,
                                   float* lse, int B, int H, int Nq, int Nk, int d, int dv,
                                   int query_offset, float scale, int causal, uint64_t seed,
                                   int drop_t, void* stream) {
  if (drop_t < 0 || drop_t > 255) return TA_ERR_INVALID_ARG;
  const tiledattn::DropoutArgs dr = dropout_args(seed, drop_t);
  return forward(q, k, v, o, lse, B, H, Nq, Nk, d, dv, query_offset, scale, causal, stream, false,
                 &dr);
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
    case TA_ERR_TOO_LARGE:
      return "sizes exceed the fixed device scratch of attn_bwd_noalloc (16 MiB: B*H*N <= 2^21)";
    default: return "unknown status";
  }
}
