/*
 * attn_bwd.h - C ABI of the MI355X (gfx950) attention backward.
 *
 * The gradients of the forward of attn_fwd.h, O = softmax(scale * Q K^T) V,
 * with respect to Q, K and V, given the upstream gradient dO, the forward's
 * output O and its log-sum-exp (page 3 "OpenAI Triton from introduction to
 * model practice", section 6: the autograd wrapper saves q, k, v, o and lse
 * in the forward and hands them to the backward).  With s = scale q.k and
 * P = exp(s - lse), for every batch b and head h:
 *
 *   dV = P^T dO
 *   dP = dO V^T,   D_i = sum_c dO_ic O_ic,   dS = P * (dP - D)
 *   dQ = scale * dS K,   dK = scale * dS^T Q
 *
 * computed tile by tile (P and dS are recomputed from Q, K and lse and never
 * reach device memory).  Optionally causal (ATTN_CAUSAL of attn_fwd.h).
 */
#ifndef ATTN_BWD_H
#define ATTN_BWD_H

#include <stddef.h>
#include <stdint.h>

#include "attn_fwd.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Arguments of attn_bwd.  All tensors contiguous [B, H, N, d] (lse [B, H, N]),
 * device memory of the current device, 16-byte aligned (lse 4-byte).
 *
 * q, k, v, o : the forward's inputs and output, element type `dtype`.
 * dout       : dL/dO, element type `dtype`.
 * lse        : the forward's log-sum-exp output, fp32, for the same scale and
 *              flags.
 * dq, dk, dv : written: the gradients, rounded to nearest-even to `dtype`
 *              from fp32 accumulators (for fp32, the accumulators).  They must not overlap each other or
 *              any input.
 * B, H, N, d : as for attn_fwd (d = 64 or 128).
 * scale      : the forward's scale, finite.
 * dtype      : ATTN_DTYPE_F16, ATTN_DTYPE_BF16 or ATTN_DTYPE_F32 (fp32 runs
 *              kernels of its own: VALU products over LDS tiles of 32 rows,
 *              P and dS kept in fp32).
 * flags      : 0 or ATTN_CAUSAL (query i attends keys 0..i).
 * stream     : a hipStream_t (NULL = the null stream).
 */
typedef struct attn_bwd_args {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  int64_t B, H, N, d;
  float scale;
  int dtype;
  unsigned flags;
  void* stream;
} attn_bwd_args_t;

/* Bytes of workspace attn_bwd needs: B*H*N*8 (per query row the pair
 * lse * log2(e) and D = rowsum(dO * O), both fp32), 0 for empty or invalid
 * sizes. */
size_t attn_bwd_workspace(int64_t B, int64_t H, int64_t N, int64_t d);

/*
 * attn_bwd - dQ, dK, dV (see above).  Two kernels queued on args->stream:
 * dQ (blocks over query rows; each block first stores its rows'
 * (lse * log2(e), D) pairs in the workspace), then dK, dV (blocks over keys,
 * reading those pairs), with no atomics (deterministic).
 *
 * workspace : device memory, 16-byte aligned, at least attn_bwd_workspace()
 *             bytes, not overlapping any tensor; owned by the caller.
 * Returns ATTN_OK, or the attn_fwd codes: ATTN_ERR_NULLPTR (args, a pointer
 * or the workspace NULL while B*H*N > 0), ATTN_ERR_SHAPE, ATTN_ERR_HEAD_DIM,
 * ATTN_ERR_DTYPE, ATTN_ERR_SCALE, ATTN_ERR_FLAGS, ATTN_ERR_ALIGN,
 * ATTN_ERR_ALIAS, ATTN_ERR_WORKSPACE, ATTN_ERR_HIP.  Every check but the last
 * runs before any HIP call.  B*H*N == 0 returns ATTN_OK with no launch.
 */
int attn_bwd(const attn_bwd_args_t* args, void* workspace, size_t workspace_bytes);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_BWD_H */
