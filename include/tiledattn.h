/*
 * tiledattn.h -- C ABI of the fused attention library (forward and backward)
 * for AMD Instinct MI355X (gfx950).  Library file: libtiledattn.so.
 *
 * The operation is softmax attention with an online (tiled) softmax: for
 * every (batch, head) and query row i,
 *
 *     S[i,j] = scale * <q_i, k_j>          (hidden when causal and j > i)
 *     O[i,:] = sum_j softmax_j(S[i,:]) v_j
 *     LSE[i] = ln sum_j exp(S[i,j])        (natural log, scaled scores)
 *
 * computed tile by tile with a running maximum, normaliser and unnormalised
 * accumulator, so the N x N score matrix is never stored.  Definitions:
 * page "22. GPU Engineering: Correctness, Throughput, and Attention",
 * sec. 22.5 (the recurrence, masking before max and sum) and sec. 22.7 (the
 * causal rule on absolute positions and the saved per-row log-normaliser);
 * page "GPU Programming & Kernel Development" (FlashAttention: tiles streamed
 * on chip, the score matrix never written).
 *
 * Nothing here depends on HIP headers; a stream is passed as an opaque
 * pointer (a hipStream_t; NULL selects the default stream).
 */
#ifndef TILEDATTN_H
#define TILEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
typedef enum {
  TA_OK = 0,              /* enqueued (or nothing to do)                          */
  TA_ERR_INVALID_ARG = 1, /* a size, offset, flag, pointer or scale is out of range */
  TA_ERR_UNSUPPORTED = 2, /* head dimension other than 64 or 128                  */
  TA_ERR_MISALIGNED = 3,  /* q, k, v or o not 16-byte aligned, lse not 4-byte     */
  TA_ERR_HIP = 4,         /* the HIP runtime reported an error at launch          */
  TA_ERR_TOO_LARGE = 5    /* sizes exceed attn_bwd_noalloc's fixed device scratch */
} ta_status;

/*
 * attn_fwd -- enqueue one fused attention forward on `stream`.
 *
 *   q, k, v : device pointers, bfloat16, contiguous row-major [B, H, N, d]
 *             (the head's rows are consecutive, d fastest).  Read only.
 *   o       : device pointer, float32, [B, H, N, d], written.
 *   lse     : device pointer, float32, [B, H, N], written: natural-log
 *             log-sum-exp of the scaled (and masked) scores of each row.
 *   B, H, N : batch, heads, sequence length (queries = keys = N); each >= 1,
 *             N <= 2^22 and B*H*ceil(N/128) <= 2^31-1.
 *   d       : head dimension, 64 or 128.
 *   scale   : multiplies Q K^T before the softmax; any finite float (callers
 *             usually pass 1/sqrt(d)).
 *   causal  : 0 = every key visible; 1 = key j visible to query i iff j <= i.
 *   stream  : hipStream_t to enqueue on (NULL = default stream).
 *
 * Ownership: the caller allocates and frees every buffer; the library keeps no
 * state and allocates nothing, so concurrent calls on different streams are
 * safe.  o and lse must not overlap q, k or v.
 *
 * Synchronisation: the call only enqueues; results are valid once `stream`
 * has been synchronised.  Q, K and V are expected to be finite (not checked
 * on the device: a non-finite input makes the affected rows non-finite).
 *
 * Errors: argument errors are found before any HIP call, nothing is enqueued
 * and the matching TA_ERR_* code is returned.  A launch rejected by the
 * runtime returns TA_ERR_HIP (hipGetLastError is consumed).  Device faults
 * surface at the caller's next synchronisation, as for any HIP kernel.
 */
int attn_fwd(const void* q, const void* k, const void* v, float* o, float* lse,
             int B, int H, int N, int d, float scale, int causal, void* stream);

/*
 * attn_fwd_ex -- attn_fwd for general shapes: Nq queries attending Nk keys,
 * value width dv, and queries placed at absolute positions query_offset ..
 * query_offset + Nq - 1 (the decoding-style subproblems of the lab on page
 * "22. GPU Engineering: Correctness, Throughput, and Attention", sec. 22.7:
 * a nonnegative query-position offset, the causal rule on absolute
 * positions, and the policy for rows that see no key).
 *
 *     S[i,j] = scale * <q_i, k_j>     hidden when causal and j > i + query_offset
 *     O[i,:] = sum_j softmax_j(S[i,:]) v_j,   LSE[i] = ln sum_j exp(S[i,j])
 *     a row with no visible key (only possible when Nk = 0): O[i,:] = 0, LSE[i] = -inf
 *
 *   q   : device bf16 [B, H, Nq, d];  k: device bf16 [B, H, Nk, d];
 *   v   : device bf16 [B, H, Nk, dv]; read only, contiguous, rows of a head consecutive.
 *   o   : device fp32 [B, H, Nq, dv], written;  lse: device fp32 [B, H, Nq], written.
 *   Nq, Nk       : 0 .. 2^22 each (Nq = 0: nothing is enqueued, TA_OK).  q, o and
 *                  lse may be NULL when Nq = 0, k and v when Nk = 0.
 *   d, dv        : 64 or 128 each (TA_ERR_UNSUPPORTED otherwise).
 *   query_offset : 0 .. 2^30 (the lab requires it nonnegative); ignored when causal = 0.
 *   B, H, scale, causal, stream, ownership, alignment and errors: as for attn_fwd.
 *
 * attn_fwd(q, k, v, o, lse, B, H, N, d, ...) computes exactly
 * attn_fwd_ex(q, k, v, o, lse, B, H, N, N, d, d, 0, ...).
 */
int attn_fwd_ex(const void* q, const void* k, const void* v, float* o, float* lse,
                int B, int H, int Nq, int Nk, int d, int dv, int query_offset,
                float scale, int causal, void* stream);

/*
 * attn_quantize_fp8 -- per-head FP8 quantisation of bf16 rows (the input side of
 * attn_fwd_fp8).  For each head h of x (heads x rows x d, contiguous):
 *
 *     amax      = max |x[h]|
 *     out[h]    = RNE_e4m3(clamp(x[h] * (448 / amax), -448, 448))   OCP E4M3 codes
 *     descale[h] = amax / 448        (1 when amax = 0)
 *
 * each step one float32 operation, so x ~= e4m3(out) * descale.  (Page
 * "Chapter 7 GPU Kernels: CUDA, HIP & Triton", sec. 7.6.2: FP8 Q K^T with
 * online descaling; the per-head amax recipe is this library's choice.)
 *
 *   x       : device bf16 [heads, rows, d], read only, 16-byte aligned.
 *   out     : device uint8 [heads, rows, d], written, 16-byte aligned.
 *   descale : device float32 [heads], written (used as scratch while running).
 *   heads   : 1 .. 65535;  rows: 1 .. 2^22;  d: 64 or 128 (TA_ERR_UNSUPPORTED).
 *   stream  : as for attn_fwd.  Finite inputs are a precondition.
 * Errors, ownership and synchronisation as for attn_fwd.
 */
int attn_quantize_fp8(const void* x, void* out, float* descale, int heads, int rows, int d,
                      void* stream);

/*
 * attn_fwd_fp8 -- attn_fwd with FP8 scores: Q and K arrive as OCP E4M3 codes
 * with per-(batch, head) descale factors, so the scores are
 *
 *     S[i,j] = scale * q_descale[b,h] * k_descale[b,h] * <q8_i, k8_j>
 *
 * computed on the FP8 matrix unit (32x32x64 products at twice the bf16 rate)
 * with the descales folded into the softmax's exponent scale; P V stays in
 * bf16 with fp32 accumulation; O and LSE as for attn_fwd.
 *
 *   q8, k8    : device uint8 [B, H, N, d] E4M3 codes (attn_quantize_fp8 output).
 *   v         : device bf16 [B, H, N, d].
 *   q_descale, k_descale : device float32 [B, H].
 *   d         : 64 or 128 (TA_ERR_UNSUPPORTED otherwise); dv = d.
 *   o, lse, B, H, N, scale, causal, stream, errors: as for attn_fwd
 *   (q8, k8, v, o 16-byte aligned; lse and the descales 4-byte aligned).
 */
int attn_fwd_fp8(const void* q8, const void* k8, const void* v, float* o, float* lse,
                 const float* q_descale, const float* k_descale, int B, int H, int N, int d,
                 float scale, int causal, void* stream);

/*
 * attn_fwd_fp8_ex -- attn_fwd_fp8 for the general shapes of attn_fwd_ex:
 * q8 [B, H, Nq, d] and k8 [B, H, Nk, d] E4M3 codes, v bf16 [B, H, Nk, dv],
 * o fp32 [B, H, Nq, dv], lse [B, H, Nq]; query r at position query_offset + r.
 *   d, dv   : 64 or 128 each (TA_ERR_UNSUPPORTED otherwise).
 *   q_descale, k_descale, scale: as for attn_fwd_fp8; everything else as for
 *   attn_fwd_ex (Nq, Nk in 0 .. 2^22; no keys gives O = 0, LSE = -inf).
 */
int attn_fwd_fp8_ex(const void* q8, const void* k8, const void* v, float* o, float* lse,
                    const float* q_descale, const float* k_descale, int B, int H, int Nq, int Nk,
                    int d, int dv, int query_offset, float scale, int causal, void* stream);

/*
 * attn_fwd_split_workspace_size -- bytes of device workspace attn_fwd_split
 * uses for these sizes (0: no split is planned, and attn_fwd_split is
 * attn_fwd_ex).  Returns 0 also for sizes out of range.
 */
size_t attn_fwd_split_workspace_size(int B, int H, int Nq, int Nk, int dv);

/*
 * attn_fwd_split -- attn_fwd_ex with the key range split over workgroups when
 * the (batch, head, 128-query tile) grid alone would leave most of the chip
 * idle (a decoding step of a few sequences over a long context).  Workgroup
 * (s, head, tile) runs the online softmax over key tiles [s T, (s + 1) T) and
 * writes its own normalised O_s and LSE_s to the workspace; a second kernel
 * combines them exactly:
 *
 *     LSE = log sum_s exp(LSE_s),   O = sum_s exp(LSE_s - LSE) O_s
 *
 * (the recurrence of page "22. GPU Engineering: Correctness, Throughput, and
 * Attention", sec. 22.5, applied once to whole key ranges).  The split count
 * is chosen from the sizes alone (grids under 256 workgroups are split up to
 * about 256; grids under 1024 in two when Nq <= Nk / 64, where the partial
 * results stay small next to the keys and values read; >= 4 key tiles of 64
 * per split), so results are deterministic for given sizes.
 *
 *   workspace       : device, 256-byte aligned, >= attn_fwd_split_workspace_size
 *                     bytes (TA_ERR_INVALID_ARG if smaller, TA_ERR_MISALIGNED if
 *                     misaligned); owned by the caller, overwritten.  May be
 *                     NULL when that size is 0.  Concurrent calls need
 *                     separate workspaces.
 *   scale <= 0      : runs unsplit (as attn_fwd_ex).
 *   everything else : as for attn_fwd_ex.
 */
int attn_fwd_split(const void* q, const void* k, const void* v, float* o, float* lse, int B,
                   int H, int Nq, int Nk, int d, int dv, int query_offset, float scale, int causal,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_fwd_dropout -- attn_fwd with dropout on the probabilities (page
 * "22. GPU Engineering: Correctness, Throughput, and Attention", sec. 22.5:
 * dropout only with reproducible masks).  For head n = b * H + h, query row i
 * and key j the mask byte is
 *
 *     byte(i, j) = byte (j mod 16) of Philox-4x32-10(counter = (i, j / 16, n, 0),
 *                                                    key = (seed mod 2^32, seed / 2^32))
 *
 * (the generator's four 32-bit output words read as 16 little-endian bytes;
 * Salmon, Moraes, Dror, Shaw, SC 2011), P[i, j] is kept when byte >= drop_t,
 * and
 *
 *     O[i,:] = 256 / (256 - drop_t) * sum_j keep(i, j) softmax_j(S[i,:]) v_j
 *     LSE[i] = ln sum_j exp(S[i,j])         (every visible key, kept or not)
 *
 * so the drop probability is drop_t / 256 and drop_t = 0 is attn_fwd.  The
 * mask is a pure function of (seed, n, i, j): attn_bwd_dropout regenerates it.
 *
 *   seed   : any 64-bit value.
 *   drop_t : 0 .. 255 (TA_ERR_INVALID_ARG otherwise).
 *   q, k, v, o, lse, B, H, N, d, scale, causal, stream, errors: as for attn_fwd.
 */
int attn_fwd_dropout(const void* q, const void* k, const void* v, float* o, float* lse, int B,
                     int H, int N, int d, float scale, int causal, uint64_t seed, int drop_t,
                     void* stream);

/*
 * attn_fwd_dropout_ex -- attn_fwd_dropout for the general shapes of
 * attn_fwd_ex (Nq queries at positions query_offset .. query_offset + Nq - 1,
 * Nk keys, value width dv).  The mask byte of query row r is that of absolute
 * position i = query_offset + r in the formula of attn_fwd_dropout, so a chunk
 * of queries gets exactly the rows of the whole problem with the same seed
 * (the lab's decoding-style subproblems, page "22. GPU Engineering:
 * Correctness, Throughput, and Attention", sec. 22.7).
 *   seed, drop_t: as for attn_fwd_dropout; everything else as for attn_fwd_ex.
 */
int attn_fwd_dropout_ex(const void* q, const void* k, const void* v, float* o, float* lse,
                        int B, int H, int Nq, int Nk, int d, int dv, int query_offset,
                        float scale, int causal, uint64_t seed, int drop_t, void* stream);

/*
 * attn_bwd_workspace_size -- bytes of device workspace attn_bwd needs for
 * (B, H, N): 8 * B * H * (N rounded up to a multiple of 4); for attn_bwd_ex pass
 * N = Nq.
 * Returns 0 when the sizes are out of the range the backward accepts (N = 0
 * gives 0 bytes, valid for attn_bwd_ex only).
 */
size_t attn_bwd_workspace_size(int B, int H, int N);

/*
 * attn_bwd -- enqueue the gradients of attn_fwd on `stream`.
 *
 * For a loss L with G = dL/dO, with P the softmax of the scaled (and masked)
 * scores of each row:
 *
 *     dV = P^T G,   dP = G V^T,   dS = P * (dP - D),   D_i = sum_c G[i,c] O[i,c]
 *     dQ = scale dS K,   dK = scale dS^T Q
 *
 * (page "22. GPU Engineering: Correctness, Throughput, and Attention",
 * sec. 22.5 for the formulas, sec. 22.7 for the derivation: the row sum of
 * dP * P equals D, so only O and the per-row log-normaliser are kept from the
 * forward, and every probability block is recomputed as exp(S - LSE)).
 *
 *   q, k, v   : device, bfloat16, [B, H, N, d] -- the forward's inputs. Read only.
 *   o, lse    : device, float32, [B, H, N, d] and [B, H, N] -- the forward's
 *               outputs for the same q, k, v, scale and causal flag.  Read only.
 *   dout      : device, bfloat16, [B, H, N, d] -- G, the gradient of the loss
 *               with respect to O, given at the precision of the matrix-unit
 *               operands.  Read only.
 *   dq, dk, dv: device, float32, [B, H, N, d], written (every element).
 *   workspace : device, attn_bwd_workspace_size(B, H, N) bytes, 16-byte
 *               aligned, owned by the caller; overwritten (per-row D and
 *               LSE log2(e)).  Calls that run concurrently need separate
 *               workspaces.
 *   B, H, N, d, scale, causal, stream: as for attn_fwd.
 *
 * Every gradient row is written by exactly one workgroup (no atomics): the
 * result is deterministic, bit for bit, for a given input.
 *
 * Ownership and synchronisation as for attn_fwd: nothing is allocated or kept;
 * the call only enqueues.  Outputs must not overlap any input or each other.
 *
 * Errors: as for attn_fwd; q, k, v, o, dout, dq, dk, dv and workspace need
 * 16-byte alignment, lse 4 bytes (TA_ERR_MISALIGNED otherwise).
 */
int attn_bwd(const void* q, const void* k, const void* v, const float* o,
             const float* lse, const void* dout, float* dq, float* dk, float* dv,
             void* workspace, int B, int H, int N, int d, float scale, int causal,
             void* stream);

/*
 * attn_bwd_ex -- the gradients of attn_fwd_ex: general shapes, with the same
 * formulas as attn_bwd.  Query i sits at position query_offset + i and (when
 * causal) sees key j iff j <= i + query_offset.
 *
 *   q, dout   : device bf16, [B, H, Nq, d] and [B, H, Nq, dv].
 *   k, v      : device bf16, [B, H, Nk, d] and [B, H, Nk, dv].
 *   o, lse    : device fp32, [B, H, Nq, dv] and [B, H, Nq] -- attn_fwd_ex's
 *               outputs for the same inputs, scale, causal flag and offset.
 *   dq        : device fp32 [B, H, Nq, d]; dk: [B, H, Nk, d]; dv: [B, H, Nk, dv];
 *               written (every element; dK = dV = 0 for Nq = 0, dQ = 0 for
 *               Nk = 0).
 *   workspace : attn_bwd_workspace_size(B, H, Nq) bytes (per query row).
 *   Nq, Nk    : 0 .. 2^22;  query_offset: 0 .. 2^30;  d, dv: 64 or 128.
 *   A pointer may be NULL only where its tensors are empty.  Other arguments,
 *   ownership, determinism and errors as for attn_bwd.
 */
int attn_bwd_ex(const void* q, const void* k, const void* v, const float* o, const float* lse,
                const void* dout, float* dq, float* dk, float* dv, void* workspace, int B, int H,
                int Nq, int Nk, int d, int dv_width, int query_offset, float scale, int causal,
                void* stream);

/*
 * attn_bwd_dropout -- the gradients of attn_fwd_dropout (same seed, drop_t,
 * scale and causal flag).  With M the keep mask (regenerated from the seed,
 * never stored) and ks = 256 / (256 - drop_t):
 *
 *     dV = (P * M ks)^T G,   dP = (G V^T) * M ks,   dS = P * (dP - D),
 *     D_i = sum_c G[i,c] O[i,c]   (O: attn_fwd_dropout's output)
 *     dQ = scale dS K,   dK = scale dS^T Q
 *
 * (the chain rule of attn_bwd through the mask; the row sum of dP * P still
 * equals D).  Arguments, workspace (attn_bwd_workspace_size), ownership,
 * determinism and errors as for attn_bwd; drop_t outside 0 .. 255 gives
 * TA_ERR_INVALID_ARG.
 */
int attn_bwd_dropout(const void* q, const void* k, const void* v, const float* o,
                     const float* lse, const void* dout, float* dq, float* dk, float* dv,
                     void* workspace, int B, int H, int N, int d, float scale, int causal,
                     uint64_t seed, int drop_t, void* stream);

/*
 * attn_bwd_dropout_ex -- the gradients of attn_fwd_dropout_ex (same shapes,
 * offset, seed and drop_t; the mask is regenerated from the absolute query
 * positions).  Arguments, workspace (attn_bwd_workspace_size(B, H, Nq)),
 * determinism and errors as for attn_bwd_ex.
 */
int attn_bwd_dropout_ex(const void* q, const void* k, const void* v, const float* o,
                        const float* lse, const void* dout, float* dq, float* dk, float* dv,
                        void* workspace, int B, int H, int Nq, int Nk, int d, int dv_width,
                        int query_offset, float scale, int causal, uint64_t seed, int drop_t,
                        void* stream);

/*
 * attn_bwd_noalloc -- attn_bwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results (bit for bit) as attn_bwd, with
 * the per-row statistics kept in the library's own device scratch instead of
 * a caller workspace.  The call allocates nothing, neither does the library.
 *
 *   scratch : a fixed 16 MiB array per device, held until the process ends;
 *             it needs 8 * B * H * (N rounded up to a multiple of 4) bytes, so
 *             B * H * N <= 2^21 rows (sizes beyond it: TA_ERR_TOO_LARGE,
 *             before any HIP call).  Nothing in it needs to start at zero.
 *   Every call on one device shares that device's scratch: calls that may
 *   overlap on one device (different streams, or threads) race and must be
 *   serialised by the caller.  The first call on a device (with that device
 *   current) looks up the scratch address once (hipGetSymbolAddress); a
 *   failure there gives TA_ERR_HIP.
 *   q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale, causal, stream, the
 *   other errors, ownership and synchronisation: as for attn_bwd.
 */
int attn_bwd_noalloc(const void* q, const void* k, const void* v, const float* o,
                     const float* lse, const void* dout, float* dq, float* dk, float* dv,
                     int B, int H, int N, int d, float scale, int causal, void* stream);

/* Human-readable text for a ta_status value (static storage; never NULL). */
const char* attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* TILEDATTN_H */
