/*
 * attn_fwd.h - C ABI of the MI355X (gfx950) fused attention forward.
 *
 * The operation (page 3 "OpenAI Triton from introduction to model practice",
 * section 5, the FlashAttention forward kernel that stores the output and the
 * log-sum-exp; section 3 for the plain definition it replaces):
 *
 *   for every batch b < B, head h < H and query row i < N:
 *     s_ij        = scale * sum_c Q[b,h,i,c] * K[b,h,j,c]          (j < N)
 *     O[b,h,i,:]  = sum_j softmax_j(s_i.) * V[b,h,j,:]
 *     lse[b,h,i]  = ln sum_j exp(s_ij)      (natural log, scaled scores)
 *
 * computed tile by tile with an online softmax (page 1 "Triton hand-written
 * kernels", section 4: running row max m, running exp-sum l, rescaled fp32
 * accumulator), so the N x N score matrix never reaches device memory.
 * attn_fwd is the non-causal self-attention call on contiguous tensors
 * (queries and keys share N); attn_fwd_ex adds the causal variant, element
 * strides and a key length Nk of its own (j < Nk above: a few queries against
 * a long key/value history, as when generation scores each new position
 * against all cached keys, which page 3 section 4 names as the
 * memory-bandwidth-bound case of inference), and attn_fwd_splitkv splits
 * each head's keys over several blocks.
 *
 * Everything here is plain C: pointers, sizes and an opaque stream handle.
 */
#ifndef ATTN_FWD_H
#define ATTN_FWD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of Q, K, V and O.  lse is always fp32. */
typedef enum {
  ATTN_DTYPE_F32 = 0,  /* IEEE binary32; QK^T and PV on fp32 MFMA, P kept fp32  */
  ATTN_DTYPE_F16 = 1,  /* IEEE binary16; fp16 MFMA, fp32 accumulate, P -> fp16  */
  ATTN_DTYPE_BF16 = 2  /* bfloat16;      bf16 MFMA, fp32 accumulate, P -> bf16  */
} attn_dtype_t;

/* Return codes.  Every error is detected before any HIP call is made, except
 * ATTN_ERR_HIP; on any error nothing is launched and no output is written. */
enum {
  ATTN_OK = 0,
  ATTN_ERR_NULLPTR = -1,  /* q, k, v or o is NULL while B*H*N > 0              */
  ATTN_ERR_SHAPE = -2,    /* a size is negative, or B*H*N*d overflows int64,
                             or N or Nk exceeds ATTN_MAX_N, or the grid is
                             too large                                          */
  ATTN_ERR_HEAD_DIM = -3, /* d is not 64 or 128                                 */
  ATTN_ERR_DTYPE = -4,    /* dtype is not an attn_dtype_t value                 */
  ATTN_ERR_SCALE = -5,    /* scale is NaN or infinite                           */
  ATTN_ERR_ALIGN = -6,    /* q, k, v, o not 16-byte aligned, or lse not 4-byte  */
  ATTN_ERR_ALIAS = -7,    /* o or lse overlaps an input, or lse overlaps o      */
  ATTN_ERR_HIP = -8,      /* the kernel launch failed (hipGetLastError)         */
  ATTN_ERR_FLAGS = -9,    /* attn_fwd_ex: unknown bits in flags, or
                             ATTN_CAUSAL with Nk != N                           */
  ATTN_ERR_LAYOUT = -10,  /* attn_fwd_ex: a stride is negative, not a multiple
                             of 8 elements, or rows of a head overlap           */
  ATTN_ERR_SPLITS = -11,  /* attn_fwd_splitkv: splits not in 1..ATTN_MAX_SPLITS */
  ATTN_ERR_WORKSPACE = -12, /* attn_fwd_splitkv: workspace_bytes too small      */
  ATTN_ERR_STATIC_LIMIT = -13 /* attn_fwd_splitkv_static: the partial results need
                                 more than ATTN_STATIC_WORKSPACE_BYTES          */
};

/* Largest split count of attn_fwd_splitkv. */
#define ATTN_MAX_SPLITS 64

/* Largest sequence length accepted: per-head byte offsets and buffer sizes
 * are 32-bit in-kernel (N * 2d bytes must stay below 2^31). */
#define ATTN_MAX_N (1 << 22)

/*
 * attn_fwd - O = softmax(scale * Q K^T) V and lse, for all B*H heads.
 *
 * q, k, v : device pointers, [B, H, N, d] contiguous (row-major, d fastest),
 *           element type `dtype`.  Read only.
 * o       : device pointer, [B, H, N, d] contiguous, element type `dtype`.
 *           Written: O rounded to nearest-even from the fp32 accumulator.
 * lse     : device pointer, [B, H, N] fp32, or NULL to skip it.  Written:
 *           m + ln l of the scaled scores.
 * B, H, N : batch, heads, sequence length (queries = keys = N).  Any >= 0;
 *           N need not be a multiple of any tile size (tails are masked:
 *           padded keys get probability 0, padded query rows are not stored).
 * d       : head dimension, 64 or 128.
 * scale   : multiplies Q K^T before the softmax; any finite value (the usual
 *           choice is 1/sqrt(d)).
 * dtype   : an attn_dtype_t value.
 * stream  : a hipStream_t (NULL = the null stream).  The launch is
 *           asynchronous and ordered on this stream; the call never
 *           synchronises, allocates or frees anything, and keeps no state.
 *           It enqueues kernel launches only (no memset or copy), so it may
 *           be captured into a HIP graph and replayed.
 *
 * Ownership: the caller owns every buffer and must keep them alive until the
 * stream work completes.  Pointers must be device memory of the current
 * device (not checked: host pointers fault).  Outputs must not overlap inputs.
 * B*H*N == 0 returns ATTN_OK without launching anything.
 * Results are deterministic: the same inputs give bit-identical outputs.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int64_t B, int64_t H, int64_t N, int64_t d, float scale, int dtype,
             void* stream);

/* Flags of attn_fwd_ex. */
#define ATTN_CAUSAL 1u /* query row i attends keys 0..i only */

/*
 * Arguments of attn_fwd_ex: those of attn_fwd, plus flags, tensor strides and
 * the key length.
 *
 * flags   : 0, or ATTN_CAUSAL for the causal variant (page 1 section 4 notes
 *           that practical kernels add a causal mask; page 3 section 3's
 *           decoder layer masks future positions with -1e9 before the
 *           softmax and section 6's wrapper passes a causal flag).  Query
 *           row i then attends keys 0..i: s_ij for j > i is excluded
 *           (probability exactly 0), and lse covers keys 0..i.
 * *_stride: element strides of the batch, head and row dimensions of q, k,
 *           v and o ({b, h, n}); the head dimension is always contiguous.
 *           All three zero means contiguous [B, H, N, d] (strides
 *           {H*N*d, N*d, d}); a [B, N, H, d] tensor has {N*H*d, d, H*d}.
 *           Every stride must be a multiple of 8 (16-byte aligned rows) and
 *           the (b, h, n) rows of o must not overlap.  lse is always
 *           contiguous [B, H, N].
 * Nk      : key and value rows per head: k and v are [B, H, Nk, d] (with
 *           their own strides; all-zero strides mean {H*Nk*d, Nk*d, d}),
 *           q, o and lse keep N rows.  0 means Nk = N (self-attention); a
 *           softmax over no keys is undefined, so there is no way to ask for
 *           it.  Any value in 1..ATTN_MAX_N, smaller or larger than N.
 *           ATTN_CAUSAL requires Nk == N (ATTN_ERR_FLAGS otherwise): the
 *           pages define the causal mask for one sequence only.
 */
typedef struct attn_fwd_args {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t B, H, N, d;
  float scale;
  int dtype;
  unsigned flags;
  int64_t q_stride[3];
  int64_t k_stride[3];
  int64_t v_stride[3];
  int64_t o_stride[3];
  void* stream;
  int64_t Nk;
} attn_fwd_args_t;

/*
 * attn_fwd_ex - attn_fwd with flags and strides (see attn_fwd_args_t).
 * Same ownership, validation and return codes as attn_fwd, plus
 * ATTN_ERR_FLAGS and ATTN_ERR_LAYOUT; args itself is read during the call
 * only.  args == NULL returns ATTN_ERR_NULLPTR.
 */
int attn_fwd_ex(const attn_fwd_args_t* args);

/*
 * attn_fwd_splitkv - the same result as attn_fwd_ex, with each head's keys
 * split into up to `splits` contiguous ranges handled by separate blocks.
 *
 * For shapes whose B*H*ceil(N/256) query blocks leave compute units idle
 * (few heads, long sequences), this multiplies the parallelism.  Each split
 * s computes a normalised partial output O_s and log-sum-exp lse_s over its
 * keys; a second kernel merges them exactly, lse = ln sum_s exp(lse_s) and
 * O = sum_s exp(lse_s - lse) O_s: the combination of per-block row maxima
 * and sums that page 3 section 1.1 describes, using the log-sum-exp that
 * page 3 section 5 stores.  Keys are cut at multiples of 64; the split count
 * actually used is the number of non-empty ranges (at most `splits`).  With
 * few query rows and many keys (Nk >> N) this is the way to fill the GPU.
 *
 * args      : as for attn_fwd_ex; flags must not contain ATTN_CAUSAL
 *             (ATTN_ERR_FLAGS).
 * splits    : 1 .. ATTN_MAX_SPLITS (ATTN_ERR_SPLITS otherwise).
 * workspace : device memory of the current device, 16-byte aligned, at least
 *             attn_fwd_splitkv_workspace_ex(B, H, N, Nk, d, splits) bytes
 *             (attn_fwd_splitkv_workspace(B, H, N, d, splits) when Nk = N),
 *             owned by
 *             the caller and not overlapping any tensor (ATTN_ERR_NULLPTR,
 *             ATTN_ERR_ALIGN, ATTN_ERR_WORKSPACE, ATTN_ERR_ALIAS).  It holds
 *             fp32 partial results between the two kernels, both queued on
 *             args->stream; calls that share a workspace must be ordered.
 * Returns the codes of attn_fwd_ex plus those above.
 */
int attn_fwd_splitkv(const attn_fwd_args_t* args, int splits, void* workspace,
                     size_t workspace_bytes);

/* Bytes of workspace attn_fwd_splitkv needs (splits_used * B*H*N * (d + 1)
 * * 4, where splits_used depends on the key length), or 0 for empty or
 * invalid sizes.  _ex takes the key length Nk (0 means N); the plain form is
 * the self-attention case Nk = N. */
size_t attn_fwd_splitkv_workspace(int64_t B, int64_t H, int64_t N, int64_t d, int splits);
size_t attn_fwd_splitkv_workspace_ex(int64_t B, int64_t H, int64_t N, int64_t Nk, int64_t d,
                                     int splits);

/* Size of the library's own device array behind attn_fwd_splitkv_static. */
#define ATTN_STATIC_WORKSPACE_BYTES ((size_t)64 << 20)

/*
 * attn_fwd_splitkv_static - attn_fwd_splitkv without a workspace argument and
 * without any allocation, for callers that cannot allocate device memory: code
 * being captured into a HIP graph, serving loops and harnesses that forbid
 * hipMalloc.
 *
 * The fp32 partial results live in a static device array of
 * ATTN_STATIC_WORKSPACE_BYTES (64 MiB) that the library owns; every device
 * the library runs on holds its own copy from the first call on it until the
 * process ends.  The call allocates and frees nothing (no hipMalloc, no
 * allocating library routine); on its first call on a device it looks the
 * array's address up (hipGetSymbolAddress) with that device current.
 *
 * args, splits : as for attn_fwd_splitkv (the same kernels run, so the result
 *                is bit-identical to attn_fwd_splitkv with the same splits).
 * Returns the codes of attn_fwd_splitkv, minus the workspace ones, plus
 * ATTN_ERR_STATIC_LIMIT when attn_fwd_splitkv_workspace_ex(B, H, N, Nk, d,
 * splits) exceeds ATTN_STATIC_WORKSPACE_BYTES; that and every other argument error is
 * detected before any HIP call.
 *
 * Every call on one device shares that device's array, which keeps the last
 * call's contents.  Nothing in it has to start at zero: the first kernel
 * writes every partial row the merge reads.  Calls that overlap in time on
 * one device (different streams, or different host threads without ordering)
 * race on the array and give wrong results; order them on one stream.
 */
int attn_fwd_splitkv_static(const attn_fwd_args_t* args, int splits);

/*
 * attn_fwd_merge - combine results over disjoint key sets into the result over
 * their union (the exact merge of attn_fwd_splitkv, for partial results the
 * caller computed, e.g. with attn_fwd_ex over shards of a long key/value
 * cache, one shard per GPU or per call).  Page 3 section 1.1 merges per-block
 * row maxima and sums into the row's; section 5's stored log-sum-exp makes
 * that a formula:
 *
 *   lse = ln sum_s exp(lse_s),   O = sum_s exp(lse_s - lse) O_s.
 *
 * o_parts   : host array of nparts device pointers, each a contiguous
 *             [B, H, N, d] O_s of element type `dtype`, 16-byte aligned.
 * lse_parts : host array of nparts device pointers, each a contiguous
 *             [B, H, N] fp32 lse_s, 4-byte aligned.  Every part must cover at
 *             least one key (lse_s finite): a row whose parts are all empty
 *             has no value.
 * nparts    : 1 .. ATTN_MAX_SPLITS (ATTN_ERR_SPLITS otherwise).
 * o         : device pointer, contiguous [B, H, N, d], `dtype`; written, O
 *             rounded to nearest-even from fp32.
 * lse       : device pointer, [B, H, N] fp32, or NULL to skip it.
 * B, H, N, d, dtype, stream : as for attn_fwd.
 *
 * The host arrays are read during the call only.  Outputs must not overlap
 * any part (ATTN_ERR_ALIAS) or each other.  Every argument error is detected
 * before any HIP call; B*H*N == 0 returns ATTN_OK without a launch.  One
 * kernel on `stream`; nothing is allocated; the result is deterministic and
 * does not depend on the order of the parts beyond fp32 rounding.
 */
int attn_fwd_merge(const void* const* o_parts, const float* const* lse_parts, int nparts,
                   void* o, float* lse, int64_t B, int64_t H, int64_t N, int64_t d, int dtype,
                   void* stream);

/* Static text for a return code (never NULL). */
const char* attn_strerror(int code);

/* Library version as 10000*major + 100*minor + patch. */
int attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_FWD_H */
