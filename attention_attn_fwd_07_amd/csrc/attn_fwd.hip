// attn_fwd.hip - fused attention forward for AMD MI355X (gfx950, CDNA4).
//
// Method: page 1 "Triton hand-written kernels: from vector add to the
// FlashAttention core", section 4 (online softmax: running max m, running
// exp-sum l, rescaled accumulator), and page 3 "OpenAI Triton from
// introduction to model practice", section 5 (the same forward with a
// (batch, head, query-block) grid and a log-sum-exp output), figure 1-A's
// seven steps.  The pages' kernels are Triton programs for NVIDIA parts; this
// file is a gfx950 design of the same computation.
//
// Kernels (each wave owns 32 query rows of one (b, h) for the whole key loop;
// K/V tiles of 64 keys stream through LDS by direct global->LDS loads):
//   * attn_fwd_pp16   bf16/fp16, d = 128, grids of at least one block per CU:
//                     8 waves, 256 rows, two wave groups taking turns between
//                     an MFMA phase and a softmax phase (ping-pong);
//   * attn_fwd_mfma16 bf16/fp16, d = 64 and small grids: 4 waves, 128 rows,
//                     software-pipelined in each wave; for grids of at most
//                     one block per CU, 8 waves with the keys split between
//                     two waves per row group;
//   * attn_fwd_mfma32 fp32: the same structure on the fp32 MFMA; for grids of
//                     a few blocks, shorter blocks whose four waves split
//                     the keys (four key groups at d = 64, two at d = 128);
//   * attn_fwd_dec    any dtype, at most four query rows per head (decode):
//                     K and V streamed with plain loads, scores on the VALU;
//   * attn_merge      the split-KV merge.
// All take element strides, a key length of their own and a key-range
// split; the three MFMA kernels also a causal flag.
//
// Register layouts (the core of the design).  With the 32x32xK MFMA, the C/D
// fragment of lane l holds column (l % 32) and rows 8*(r/4) + 4*(l/32) + r%4
// for r = 0..15.  The kernel therefore computes the TRANSPOSED scores
//     S^T[key, query] = K * Q^T            (A = K rows, B = Q rows)
// so that lane l holds ONE query row (l % 32) and 16 keys per 32-key block.
// Consequences:
//   * row max / row sum are in-lane reductions plus one exchange with lane
//     l ^ 32 (v_permlane32_swap);
//   * the probabilities P, packed in register order, are already the B
//     operand of the second product, computed as O^T = V^T * P^T;
//   * O^T's C fragment again puts query (l % 32) in lane l, so the per-row
//     rescale by alpha needs no cross-lane traffic;
//   * V^T's A operand needs 4 consecutive keys of one column per register
//     pair: exactly what the gfx950 transposing LDS read ds_read_b64_tr_b16
//     returns from a row-major V tile.
// An MFMA pairs A-slot t of lane half h with B-slot t of the same half, so
// any consistent assignment of the contraction index to (half, slot) is
// correct; the kernel uses contiguous 8-element d runs for Q.K and the
// C-fragment key order for P.V.
//
// Softmax runs in the log2 domain: t = s * (scale * log2 e), p = 2^(t - m),
// v_exp_f32 computes 2^x; lse is converted back to natural log at the end.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "attn_common.h"
#include "attn_fwd.h"

namespace {

// Where one head's rows live: element strides (batch, head, row) of Q, K, V
// and O, the head dimension being contiguous, and H to split a block's
// b * H + h index.  Contiguous [B, H, N, d] tensors have strides
// {H N d, N d, d}.
struct Layout {
  int H;
  long long q[3], k[3], v[3], o[3];
  __device__ __forceinline__ long long base(const long long (&st)[3], int bh) const {
    const int b = bh / H, h = bh - b * H;
    return (long long)b * st[0] + (long long)h * st[1];
  }
};

// The keys of a head and their split over blocks.  nk is the number of key
// (and value) rows per head, which need not equal the number of query rows.
// With len > 0 (the split-KV path), block (x, y) of the grid covers key rows
// y*len .. min(nk, (y+1)*len) - 1 only and writes its own normalised output
// and log-sum-exp, in fp32, to opart[y][b*H+h][row][d] and
// lpart[y][b*H+h][row]; a second kernel merges the splits.  len == 0: one
// block covers all keys and writes the final O and lse.
struct Split {
  int len;
  int nk;
  float* opart;
  float* lpart;
  __device__ __forceinline__ int first_key() const { return len ? (int)blockIdx.y * len : 0; }
  __device__ __forceinline__ int keys() const { return len ? min(nk - first_key(), len) : nk; }
};

// Stores of one query row's result (the lane's 16 columns of each 32-column
// block, rows of O^T's C fragment): the final O rounded to the element type,
// or in split mode the fp32 partial O and lse.
template <class E, int D>
__device__ __forceinline__ void store_row16(uint16_t* __restrict__ Oh, float* __restrict__ LSE,
                                           const Split& sp, const Layout& L, int bh, int nbh,
                                           int N, int qrow, const f32x16 (&acc)[D / 32],
                                           float inv, float lse) {
  const int hh = (threadIdx.x & 63) >> 5;
  if (sp.len) {
    const size_t r = ((size_t)blockIdx.y * nbh + bh) * N + qrow;
    float* op = sp.opart + r * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<f32x4*>(op + 32 * db + 8 * g + 4 * hh) =
            (f32x4){acc[db][4 * g + 0] * inv, acc[db][4 * g + 1] * inv,
                    acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv};
    if (hh == 0) sp.lpart[r] = lse;
    return;
  }
  uint16_t* op = Oh + (size_t)qrow * L.o[2];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int col = 32 * db + 8 * g + 4 * hh;
      const u32x2 w = (u32x2){E::pack2(acc[db][4 * g + 0] * inv, acc[db][4 * g + 1] * inv),
                              E::pack2(acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv)};
      *reinterpret_cast<u32x2*>(op + col) = w;
    }
  if (LSE != nullptr && hh == 0) LSE[(size_t)bh * N + qrow] = lse;
}


// The final O rows of one wave (32 rows) stored through LDS so that each
// global store instruction writes whole rows: the C fragments (lane l: row
// l % 32, columns 32 db + 8 g + 4 (l / 32) .. +3) are normalised, rounded
// and written to the wave's own LDS area of 32 x 2D bytes as row-major rows
// whose 16-byte chunks are XOR-swizzled by the row (so the 32 rows of one
// write instruction spread over the banks), then read back 16 bytes per lane
// and stored, 64 / (D / 8) whole rows per instruction.  Storing straight from
// the fragments would write 16-byte pieces of 32 rows per instruction, four
// times the memory transactions for the same bytes.  lse is written as
// before (lanes of half 0, consecutive rows).
template <class E, int D>
__device__ __forceinline__ void store_rows_lds(lds_u8* area, uint16_t* __restrict__ Oh,
                                               float* __restrict__ LSE, const Layout& L, int bh,
                                               int N, int row0, const f32x16 (&acc)[D / 32],
                                               float inv, float lse) {
  constexpr int ROWB = 2 * D, CH = D / 8, RPI = 64 / CH;
  const int lane = threadIdx.x & 63, li = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c = 4 * db + g;
      const u32x2 w = (u32x2){E::pack2(acc[db][4 * g + 0] * inv, acc[db][4 * g + 1] * inv),
                              E::pack2(acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv)};
      *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(
          area + li * ROWB + ((c ^ (li & (CH - 1))) << 4) + 8 * hh) = w;
    }
  // the wave's LDS operations complete in order; this keeps the compiler
  // from moving the reads above the writes
  __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = i * RPI + lane / CH, c = lane % CH;
    const u32x4 x = *(const lds_u32x4*)(area + r * ROWB + ((c ^ (r & (CH - 1))) << 4));
    if (row0 + r < N) *reinterpret_cast<u32x4*>(Oh + (size_t)(row0 + r) * L.o[2] + 8 * c) = x;
  }
  if (LSE != nullptr && hh == 0 && row0 + li < N) LSE[(size_t)bh * N + row0 + li] = lse;
}

// As store_rows_lds, for NB of the D/32 column blocks (H0 .. H0+NB-1) of the
// wave's 32 rows: each row's NB * 64 bytes go through the wave's LDS area of
// 32 x NB * 64 bytes and are stored as contiguous pieces of the row, 64 / (4 NB)
// rows per instruction.  lse is written when LSE is not null.
template <class E, int D, int H0, int NB>
__device__ __forceinline__ void store_cols_lds(lds_u8* area, uint16_t* __restrict__ Oh,
                                               float* __restrict__ LSE, const Layout& L, int bh,
                                               int N, int row0, const f32x16 (&acc)[D / 32],
                                               float inv, float lse) {
  constexpr int ROWB = 64 * NB, CH = 4 * NB, RPI = 64 / CH;
  const int lane = threadIdx.x & 63, li = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int h = 0; h < NB; ++h)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c = 4 * h + g;
      const u32x2 w = (u32x2){E::pack2(acc[H0 + h][4 * g + 0] * inv, acc[H0 + h][4 * g + 1] * inv),
                              E::pack2(acc[H0 + h][4 * g + 2] * inv, acc[H0 + h][4 * g + 3] * inv)};
      *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(
          area + li * ROWB + ((c ^ (li & (CH - 1))) << 4) + 8 * hh) = w;
    }
  __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = i * RPI + lane / CH, c = lane % CH;
    const u32x4 x = *(const lds_u32x4*)(area + r * ROWB + ((c ^ (r & (CH - 1))) << 4));
    if (row0 + r < N)
      *reinterpret_cast<u32x4*>(Oh + (size_t)(row0 + r) * L.o[2] + 32 * H0 + 8 * c) = x;
  }
  if (LSE != nullptr && hh == 0 && row0 + li < N) LSE[(size_t)bh * N + row0 + li] = lse;
}

// --- pieces of one K/V tile -------------------------------------------------

// S^T = K Q^T for the two 32-key halves of a 64-key tile.  s[sb][r] is the
// raw score of key 32 sb + 8 (r/4) + 4 hh + r%4 (tile-relative) for query row
// li of the wave, hh = lane / 32.
template <class E, int D>
__device__ __forceinline__ void qk16(const lds_u8* kb, const u32x4 (&qf)[Geo16<D>::KS],
                                     f32x16 (&s)[2]) {
  using G = Geo16<D>;
  const int lane = threadIdx.x & 63;
  const int li = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    s[sb] = (f32x16){};
    const int row = sb * 32 + li;
    const lds_u8* rp = kb + row * G::ROWB;
    const int sw = swz_k<D>(row);
#pragma unroll
    for (int ks = 0; ks < G::KS; ++ks) {
      const u32x4 a = *(const lds_u32x4*)(rp + (((2 * ks + hh) ^ sw) << 4));
      s[sb] = E::mfma(a, qf[ks], s[sb]);
    }
  }
}

// The keys a query row may see: j <= lim with lim = N - 1, and for causal
// attention also lim <= the row's own index (query i attends keys 0..i).
// lane_lim is the lane's limit, wave_lim the smallest over the wave (uniform);
// a key tile needs masking only if it reaches past wave_lim.
template <bool CAUSAL>
struct KeyLimit {
  int lane_lim, wave_lim;
  __device__ __forceinline__ KeyLimit(int N, int qrow, int qrow0) {
    lane_lim = CAUSAL ? min(N - 1, qrow) : N - 1;
    wave_lim = CAUSAL ? min(N - 1, qrow0) : N - 1;
  }
  __device__ __forceinline__ bool partial(int j0, int bn) const { return j0 + bn - 1 > wave_lim; }
};

// Number of key tiles of width bn that a block of query rows q0 .. q0+bm-1
// visits: all of them, or for causal attention those up to its last row.
template <bool CAUSAL>
__device__ __forceinline__ int key_tiles(int N, int q0, int bm, int bn) {
  const int nk = CAUSAL ? min(N, q0 + bm) : N;
  return (nk + bn - 1) / bn;
}

// (head, query tile) of a block.  For causal attention the last query tile
// of a head visits the most key tiles, so level 0 of the by-level order is
// the last tile.
template <bool CAUSAL>
__device__ __forceinline__ WorkItem query_item(int nqt) {
  WorkItem w = work_item<CAUSAL>(blockIdx.x, gridDim.x, nqt);
  if (CAUSAL) w.t = nqt - 1 - w.t;
  return w;
}

// Keys past the lane's limit in a partial tile: a value that cannot win the
// row extreme (the probabilities of these keys are zeroed in softmax16).
__device__ __forceinline__ void mask_tail16(f32x16 (&s)[2], int j0, int lim, float c2) {
  const int hh = (threadIdx.x & 63) >> 5;
  const float neutral = c2 >= 0.f ? -INFINITY : INFINITY;
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (j0 + 32 * sb + 8 * (r >> 2) + 4 * hh + (r & 3) > lim) s[sb][r] = neutral;
}

// Row max of the log2-scaled scores t = s * c2 over the tile (for c2 < 0 the
// max of t comes from the min of s); both lane halves get the row's value.
__device__ __forceinline__ float tile_max16(const f32x16 (&s)[2], float c2) {
  const float mt = c2 >= 0.f ? xhalf_max(frag2_max(s[0], s[1])) : xhalf_min(frag2_min(s[0], s[1]));
  return mt * c2;
}

// The reference max m (log2 domain) moves only when some row of the wave
// exceeds it by more than this many doublings; until then P = 2^(t - m) may
// reach 2^8, harmless in fp32 and in bf16/fp16 (same relative precision).
// The result is the same softmax: O = acc / l with acc and l built from the
// same reference.  A key that dominates its row may then keep a P in
// (1, 2^8] that is no power of two, and the 16-bit rounding of that P (up to
// 2^-8 relative for bf16) enters acc; the ping-pong kernel, which uses this
// threshold, therefore normalises O by the sum of the same rounded P (l[1]
// below), so the weights applied to V sum to one exactly and that rounding
// cancels between numerator and denominator, while the log-sum-exp uses the
// sum of the unrounded P (l[0]).  The pipelined kernel with its in-block key
// split at d = 64 (short rows) does the same.  Otherwise the pipelined kernel
// follows the exact running max (threshold 0: every P is at most 1 and the
// key that sets a row's max has P = 1 exactly) and normalises by l[0]; at
// d = 64 its VALU work sets its speed, and on long rows the rare extra
// rescales cost less than the rounded sum would.
constexpr float kRescaleThreshold = 8.0f;

// Move each row's reference to max(m, m_tile) and rescale its l and
// accumulator by 2^(m_old - m_new) (1 for rows whose reference stays).
template <int D>
__device__ __forceinline__ void rescale_to(float m_tile, float& m, f32x2& l,
                                           f32x16 (&acc)[Geo16<D>::DB]) {
  const float m_new = fmaxf(m, m_tile);
  const float alpha = fast_exp2(m - m_new);
  m = m_new;
  l *= alpha;
#pragma unroll
  for (int db = 0; db < Geo16<D>::DB; ++db) acc[db] *= alpha;
}

// Rescale when some row's tile max exceeds its reference by more than thr
// doublings: kRescaleThreshold with the rounded-sum normalisation, 0 (the
// exact running max) without it.
template <int D>
__device__ __forceinline__ void maybe_rescale(float m_tile, float& m, f32x2& l,
                                              f32x16 (&acc)[Geo16<D>::DB], float thr) {
  if (__builtin_amdgcn_ballot_w64(m_tile > m + thr) != 0)  // wave-uniform
    rescale_to<D>(m_tile, m, l, acc);
}

// Sum test, the cheaper alternative to the max test (used by the ping-pong
// kernel on every tile that needs no mask): P is first formed against the
// current reference m, without the tile's row max.  If every lane's sum of
// its 32 probabilities is at most 2^8, every P is at most 2^8 - the max
// test's bound - and the tile is done.  Otherwise the row max is taken, the
// rows are rescaled and P is formed again.  The rare path runs whenever the
// max test would (and also for some tiles whose max exceeds m by 3 to 8
// doublings).  The first tile always sets m from its row max.
constexpr float kSumLimit = 256.0f;

// P = 2^(s * c2 - m), packed to the element type (RNE) as the B operand of
// the P.V product.  Returns this lane's two row-sum contributions: [0] of the
// fp32 P (for the log-sum-exp, which depends on it directly) and [1] of the
// rounded P the product uses (for normalising O), the latter two packed
// values per v_dot2c against (1, 1).  PIN keeps each packing where the
// source puts it, right after its exponentials (an empty asm statement on
// the packed values), instead of letting the compiler sink it past the sum
// test's branch: in the ping-pong kernel's VALU phase that measured about
// 1 % faster at d = 128, in the pipelined kernel at d = 64 about 4 % slower.
template <class E, bool TAIL, bool RSUM = true, bool PIN = false>
__device__ __forceinline__ f32x2 softmax16(const f32x16 (&s)[2], float m, float c2,
                                           u32x4 (&pb)[2][2], int j0, int lim) {
  const int hh = (threadIdx.x & 63) >> 5;
  // Eight independent partial sums: a single running sum would be a chain
  // of 32 dependent adds, whose latency nothing hides when one wave of the
  // SIMD is in its softmax phase.
  // The first eight probabilities start the partial sums (no adds to zero).
  float part[8];
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = fast_exp2(fmaf(s[sb][r], c2, -m));
      if (TAIL && (j0 + 32 * sb + 8 * (r >> 2) + 4 * hh + (r & 3) > lim)) p[r] = 0.f;
      if (sb == 0 && r < 8)
        part[r] = p[r];
      else
        part[r & 7] += p[r];
    }
#pragma unroll
    for (int hq = 0; hq < 2; ++hq) {
      const int b0 = 8 * hq;
      pb[sb][hq] = (u32x4){E::pack2(p[b0 + 0], p[b0 + 1]), E::pack2(p[b0 + 2], p[b0 + 3]),
                           E::pack2(p[b0 + 4], p[b0 + 5]), E::pack2(p[b0 + 6], p[b0 + 7])};
      if (PIN) __asm__ volatile("" : "+v"(pb[sb][hq]));
    }
  }
  const float sum =
      ((part[0] + part[1]) + (part[2] + part[3])) + ((part[4] + part[5]) + (part[6] + part[7]));
  if (!RSUM) return (f32x2){sum, 0.f};
  // Sums of the rounded P: two chains of eight pair sums.
  float rp[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) rp[c] = E::sum2(pb[c][0][0], 0.f);
#pragma unroll
  for (int w = 1; w < 8; ++w)
#pragma unroll
    for (int c = 0; c < 2; ++c) rp[c] = E::sum2(pb[c][w >> 2][w & 3], rp[c]);
  return (f32x2){sum, rp[0] + rp[1]};
}

// O^T += V^T P^T, 16 keys per MFMA; V^T comes from transposing LDS reads:
// lane (p16, group) points at row key0 + p16/4, columns c0 + 4*(p16%4) .. +3,
// and receives column c0 + p16 of rows key0 .. key0+3.
template <class E, int D>
__device__ __forceinline__ void pv16(const lds_u8* vb, const u32x4 (&pb)[2][2],
                                     f32x16 (&acc)[Geo16<D>::DB]) {
  using G = Geo16<D>;
  const int lane = threadIdx.x & 63;
  const int hh = lane >> 5, p16 = lane & 15, colhalf = (lane >> 4) & 1;
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
    for (int hq = 0; hq < 2; ++hq) {
      const int r0 = 32 * sb + 16 * hq + 4 * hh + (p16 >> 2);
      const int r1 = r0 + 8;
      const int half8 = (p16 & 1) * 8;
#pragma unroll
      for (int db = 0; db < G::DB; ++db) {
        const int chunk = 4 * db + 2 * colhalf + ((p16 & 3) >> 1);
        const lds_u8* a0 = vb + r0 * G::ROWB + ((chunk ^ swz_v<D>(r0)) << 4) + half8;
        const lds_u8* a1 = vb + r1 * G::ROWB + ((chunk ^ swz_v<D>(r1)) << 4) + half8;
        const u32x2 lo = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(a0)));
        const u32x2 hi = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(a1)));
        const u32x4 a = (u32x4){lo[0], lo[1], hi[0], hi[1]};
        acc[db] = E::mfma(a, pb[sb][hq], acc[db]);
      }
    }
  }
}

// --- the kernel ---------------------------------------------------------------
//
// Software pipeline over key tiles.  Iteration t holds the scores S_t of tile
// t in registers and, in one straight-line block, turns S_t into P_t (VALU),
// computes S_{t+1} = K_{t+1} Q^T (MFMA, independent of P_t, so the two
// interleave) and accumulates P_t V_t (MFMA); then it takes the row max of
// S_{t+1} and, rarely, rescales.  K therefore runs one tile ahead of V:
// iteration t reads K_{t+1} and V_t while K_{t+2} and V_{t+1} stream into
// the other K and V buffers.
// KS2 = 2 (small grids): 8 waves, two per 32-row group.  Waves w and w + 4
// take the same rows and alternate key tiles (even tiles to w, odd tiles to
// w + 4), each with its own K/V buffers and online-softmax state; at the end
// the two states are merged through LDS, m = max(m0, m1), acc and l scaled by
// 2^(m_h - m), each half finalising and storing half of the output columns
// of its rows.  This puts two waves on every SIMD when the grid alone gives
// one.  Both halves run the same number of local tiles, so their barriers
// pair up; with an odd tile count the odd half's last local tile lies past
// the keys, is not loaded, and is fully masked.  Used without a causal mask
// or a split, for at least two key tiles.
// Register budget: at d = 64 without the key split the kernel is compiled for
// three waves per SIMD (at most 168 VGPRs; three blocks of four waves share a
// CU), which measured 2 % faster at N = 65536 than the build for two;
// otherwise for two waves per SIMD (up to 256 VGPRs).
template <class E, int D, bool CAUSAL, int KS2>
__global__ __launch_bounds__(kThreads * KS2)
__attribute__((amdgpu_waves_per_eu(D == 64 && KS2 == 1 ? 3 : 2)))
void attn_fwd_mfma16(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                     const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                     float* __restrict__ LSE, int N, int nqt, float c2, Layout L, Split sp) {
  using G = Geo16<D, 4>;
  constexpr int BM = 128;
  static_assert(KS2 == 1 || (KS2 == 2 && !CAUSAL), "the key split is for the plain forward");
  // Reference policy: with the key split at d = 64 (short rows, where the
  // exact max would rescale on most tiles) the lagging reference and O
  // divided by the rounded sum; otherwise the exact running max and O divided
  // by l (at d = 128 the key split has no registers left for the second sum).
  constexpr bool RSUM = KS2 == 2 && D == 64;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[4 * G::TILEB * KS2];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int rw = wave & 3, kh = wave >> 2;  // row group, key half
  const int li = lane & 31, hh = lane >> 5;
  lds_u8* const lsm = (lds_u8*)smem + kh * 4 * G::TILEB;
  lds_u8* const kbuf0 = lsm;
  lds_u8* const kbuf1 = lsm + G::TILEB;
  lds_u8* const vbuf0 = lsm + 2 * G::TILEB;
  lds_u8* const vbuf1 = lsm + 3 * G::TILEB;

  const WorkItem wi = query_item<CAUSAL>(nqt);
  const int bh = wi.bh, qt = wi.t;
  const uint16_t* const Qh = Q + L.base(L.q, bh);
  uint16_t* const Oh = O + L.base(L.o, bh);
  // this block's keys: rows kb0 .. kb0 + Nk - 1 of the head (all of them without a split)
  const int kb0 = sp.first_key(), Nk = sp.keys();
  const unsigned char* Kb =
      reinterpret_cast<const unsigned char*>(K + L.base(L.k, bh) + (long long)kb0 * L.k[2]);
  const unsigned char* Vb =
      reinterpret_cast<const unsigned char*>(V + L.base(L.v, bh) + (long long)kb0 * L.v[2]);

  const int T = key_tiles<CAUSAL>(Nk, qt * BM, BM, G::BN);
  // local tile i of this wave's half is global tile KS2 * i + kh; both halves run ntiles
  const int ntiles = (T + KS2 - 1) / KS2;
  auto J = [&](int i) __attribute__((always_inline)) { return (KS2 * i + kh) * G::BN; };
  const TileLoader<D, 4> loader(rw, (int)(L.k[2] * 2), (int)(L.v[2] * 2));
  if (J(0) < Nk) {
    loader.load_k(Kb, J(0), Nk, kbuf0);
    loader.load_v(Vb, J(0), Nk, vbuf0);
  }
  if (ntiles > 1 && J(1) < Nk) loader.load_k(Kb, J(1), Nk, kbuf1);

  // Q fragment, resident for the whole key loop: lane (li, hh) holds
  // d = 16 ks + 8 hh + [0, 8) of query row qrow.
  const int qrow = qt * BM + rw * 32 + li;
  const KeyLimit<CAUSAL> kl(Nk, qrow, qt * BM + rw * 32);
  u32x4 qf[G::KS];
  if (qrow < N) {
    const u32x4* qp = reinterpret_cast<const u32x4*>(Qh + (size_t)qrow * L.q[2] + 8 * hh);
#pragma unroll
    for (int ks = 0; ks < G::KS; ++ks) qf[ks] = qp[2 * ks];
  } else {
#pragma unroll
    for (int ks = 0; ks < G::KS; ++ks) qf[ks] = (u32x4){0u, 0u, 0u, 0u};
  }
  f32x16 acc[G::DB];
#pragma unroll
  for (int db = 0; db < G::DB; ++db) acc[db] = (f32x16){};
  f32x2 l = (f32x2){0.f, 0.f};  // row sums of the fp32 P and (with RSUM) of the rounded P

  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  block_barrier();

  f32x16 sA[2], sB[2];
  qk16<E, D>(kbuf0, qf, sA);
  if (kl.partial(J(0), G::BN)) mask_tail16(sA, J(0), kl.lane_lim, c2);
  float m = tile_max16(sA, c2);  // the first tile sets the reference exactly
  block_barrier();               // kbuf0 is free for K_2 only after every wave read K_0

  // This kernel keeps the max test: the sum test's branch would split the
  // block in which the compiler interleaves a tile's softmax with the next
  // tile's MFMAs (measured slower here).
  auto body = [&](int t, f32x16 (&cur)[2], f32x16 (&nxt)[2], const lds_u8* kb_next,
                  const lds_u8* vb_cur, lds_u8* kb_load, lds_u8* vb_load) {
    const int j1 = J(t + 1);
    if (t + 2 < ntiles && J(t + 2) < Nk) loader.load_k(Kb, J(t + 2), Nk, kb_load);
    if (j1 < Nk) loader.load_v(Vb, j1, Nk, vb_load);
    u32x4 pb[2][2];
    if (CAUSAL && kl.partial(J(t), G::BN))  // a diagonal tile (others are full)
      l += softmax16<E, true, RSUM>(cur, m, c2, pb, J(t), kl.lane_lim);
    else
      l += softmax16<E, false, RSUM>(cur, m, c2, pb, 0, 0);
    qk16<E, D>(kb_next, qf, nxt);
    pv16<E, D>(vb_cur, pb, acc);
    // Interleave: four VALU instructions (the softmax of this tile) after
    // each MFMA of the two products, instead of the compiler's clusters.
    // Measured against its own schedule (same box, bit-identical results):
    // B4 H8 N1024 d64 14.88 -> 14.42 us, B1 H8 N2048 d128 (key split)
    // 35.6 -> 33.7 us, B1 H8 N65536 d64 +0.7 %.
#pragma unroll
    for (int i = 0; i < 2 * G::KS + 4 * G::DB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // four VALU
    }
    if (kl.partial(j1, G::BN)) mask_tail16(nxt, j1, kl.lane_lim, c2);
    maybe_rescale<D>(tile_max16(nxt, c2), m, l, acc, RSUM ? kRescaleThreshold : 0.f);
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's loads landed
    block_barrier();                                     // ... and everyone's
  };
  auto last = [&](int t, const f32x16 (&cur)[2], const lds_u8* vb_cur) {
    u32x4 pb[2][2];
    const int j0 = J(t);
    // a key-split half's tile past the keys: its buffers were never loaded
    // (a zero P times unloaded LDS could still make NaN), so nothing to add
    if (KS2 == 2 && j0 >= Nk) return;
    if (kl.partial(j0, G::BN))
      l += softmax16<E, true, RSUM>(cur, m, c2, pb, j0, kl.lane_lim);
    else
      l += softmax16<E, false, RSUM>(cur, m, c2, pb, j0, 0);
    pv16<E, D>(vb_cur, pb, acc);
  };

  // Two iterations per trip so that every LDS address is a constant.
  int t = 0;
  for (; t + 2 < ntiles; t += 2) {
    body(t, sA, sB, kbuf1, vbuf0, kbuf0, vbuf1);
    body(t + 1, sB, sA, kbuf0, vbuf1, kbuf1, vbuf0);
  }
  if (t + 1 < ntiles) {
    body(t, sA, sB, kbuf1, vbuf0, kbuf0, vbuf1);
    last(t + 1, sB, vbuf1);
  } else {
    last(t, sA, vbuf0);
  }

  // Epilogue: O = acc / l (RNE to the element type; l[1], the rounded sum,
  // with the lagging reference), lse = (m + log2 l[0]) ln 2.
  if constexpr (KS2 == 2) {
    // Merge the two halves' states through LDS (the K/V buffers are free once
    // every wave is past its last P V product).  Half kh finalises column
    // blocks [kh HB, kh HB + HB) of its 32 rows: each wave hands its partner
    // (same rows, other half) its m, l and the partner's column blocks, and
    // both combine.  m = max of the two, each side scaled by 2^(m_side - m);
    // the sums of products come out the same in both halves (the two terms
    // commute), so the two halves agree on l and lse.  A half whose row saw
    // no key has l = 0 over the row and contributes nothing (its m may be
    // -inf); a NaN in either half's l reaches the output.
    constexpr int HB = G::DB / 2;
    constexpr int NX = 4 + 16 * HB;  // floats per lane: m, l[0], l[1], pad, the blocks
    typedef __attribute__((address_space(3))) float lds_f32;
    typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
    lds_f32* const xbase = (lds_f32*)(lds_u8*)smem;
    lds_f32* const mine = xbase + (rw * 2 + kh) * 64 * NX + lane * NX;
    const lds_f32* const theirs = xbase + (rw * 2 + (kh ^ 1)) * 64 * NX + lane * NX;
    auto give = [&](auto h0c) __attribute__((always_inline)) {
      constexpr int H0 = decltype(h0c)::value;
#pragma unroll
      for (int h = 0; h < HB; ++h)
#pragma unroll
        for (int r = 0; r < 16; r += 4)
          *(lds_f32x4*)(mine + 4 + 16 * h + r) =
              (f32x4){acc[H0 + h][r], acc[H0 + h][r + 1], acc[H0 + h][r + 2], acc[H0 + h][r + 3]};
    };
    block_barrier();
    *(lds_f32x4*)mine = (f32x4){m, l[0], l[1], 0.f};
    if (kh == 0) give(std::integral_constant<int, HB>{}); else give(std::integral_constant<int, 0>{});
    block_barrier();
    const f32x4 ml = *(const lds_f32x4*)theirs;
    const f32x2 lo = (f32x2){ml[1], ml[2]};
    const bool hs = xhalf_sum(l[0]) != 0.f, ho = xhalf_sum(lo[0]) != 0.f;  // NaN counts
    const float mn = hs && ho ? fmaxf(m, ml[0]) : (hs ? m : ml[0]);
    const float as = hs ? fast_exp2(m - mn) : 0.f, ao = ho ? fast_exp2(ml[0] - mn) : 0.f;
    l = (hs ? l * as : (f32x2){0.f, 0.f}) + (ho ? lo * ao : (f32x2){0.f, 0.f});
    m = mn;
    const float lt = xhalf_sum(l[0]);
    const float inv = 1.0f / (RSUM ? xhalf_sum(l[1]) : lt);
    const float lse = (m + log2f(lt)) * kLn2;
    // staging for this wave's 32 rows x HB blocks, past the exchange area
    static_assert((8 * 64 * NX) * 4 + 8 * 32 * HB * 64 <= 4 * G::TILEB * KS2,
                  "the merge and the output staging must fit");
    lds_u8* const area = (lds_u8*)smem + (8 * 64 * NX) * 4 + (rw * 2 + kh) * 32 * HB * 64;
    auto take = [&](auto h0c) __attribute__((always_inline)) {
      constexpr int H0 = decltype(h0c)::value;
#pragma unroll
      for (int h = 0; h < HB; ++h)
#pragma unroll
        for (int r = 0; r < 16; r += 4) {
          const f32x4 x = *(const lds_f32x4*)(theirs + 4 + 16 * h + r);
#pragma unroll
          for (int u = 0; u < 4; ++u)
            acc[H0 + h][r + u] = (hs ? acc[H0 + h][r + u] * as : 0.f) + (ho ? x[u] * ao : 0.f);
        }
      store_cols_lds<E, D, H0, HB>(area, Oh, kh == 0 ? LSE : nullptr, L, bh, N, qt * BM + rw * 32,
                                   acc, inv, lse);
    };
    if (kh == 0) take(std::integral_constant<int, 0>{}); else take(std::integral_constant<int, HB>{});
  } else {
    const float lt = xhalf_sum(l[0]);
    const float inv = 1.0f / (RSUM ? xhalf_sum(l[1]) : lt);
    const float lse = (m + log2f(lt)) * kLn2;
    if (sp.len) {
      if (qrow < N) store_row16<E, D>(Oh, LSE, sp, L, bh, gridDim.x / nqt, N, qrow, acc, inv, lse);
    } else {
      // Output staging in the two K buffers (every wave read its last K tile
      // before the last barrier it passed; only V is still read).
      static_assert(4 * 32 * 2 * D <= 2 * G::TILEB, "the output staging must fit");
      store_rows_lds<E, D>(kbuf0 + rw * 32 * 2 * D, Oh, LSE, L, bh, N, qt * BM + rw * 32, acc, inv,
                           lse);
    }
  }
}

// --- MFMA phase with lean registers ---------------------------------------
//
// acc += P V (from the V tile at LDS offset vbo) followed by S^T = K Q^T (from
// the K tile at kbo), for the ping-pong kernel.  LDS addresses: with the XOR
// swizzles above, the address of K fragment (sb, ks) is
// ((kq + kbo) ^ (ks << 5)) + sb * 32 * ROWB and that of V^T fragment
// (sb, hq, db, half) is ((vq + vbo) ^ (db << 6)) + (32 sb + 16 hq + 8 half) *
// ROWB, with kq, vq per-lane constants whose XORed bits are the swizzle bits
// (row parts are multiples of ROWB) and kbo, vbo multiples of the tile size,
// which leave those bits alone; so each fragment costs one v_xor and an
// immediate offset.  The LDS reads are scheduled a fixed LA MFMAs ahead of
// their use.
template <int D>
struct LdsLanes {
  uint32_t kq, vq;
  __device__ __forceinline__ LdsLanes() {
    const int lane = threadIdx.x & 63;
    const int li = lane & 31, hh = lane >> 5, p16 = lane & 15;
    constexpr int ROWB = D * 2;
    kq = (uint32_t)(li * ROWB + ((hh ^ swz_k<D>(li)) << 4));
    const int rowpart = 4 * hh + (p16 >> 2);
    const int cb = 2 * ((lane >> 4) & 1) + ((p16 & 3) >> 1);
    vq = (uint32_t)(rowpart * ROWB + 16 * cb + (p16 & 1) * 8 + ((swz_v<D>(rowpart) >> 2) << 6));
  }
};

// acc += P V over one 64-key V tile (LDS byte offset vbo).
template <class E, int D>
__device__ __forceinline__ void pv_tile(const lds_u8* lsm, uint32_t vq, uint32_t vbo,
                                        const u32x4 (&pb)[2][2], f32x16 (&acc)[Geo16<D>::DB]) {
  constexpr int ROWB = Geo16<D>::ROWB;
  const uint32_t vqb = vq + vbo;
#pragma unroll
  for (int db = 0; db < Geo16<D>::DB; ++db) {
    const lds_u8* va = lsm + (vqb ^ (uint32_t)(db << 6));
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int hq = 0; hq < 2; ++hq) {
        const lds_u8* a0 = va + (32 * sb + 16 * hq) * ROWB;
        const u32x2 lo = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(a0)));
        const u32x2 hi = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(a0 + 8 * ROWB)));
        acc[db] = E::mfma((u32x4){lo[0], lo[1], hi[0], hi[1]}, pb[sb][hq], acc[db]);
      }
  }
}

template <class E, int D>
__device__ __forceinline__ void mfma_phase(const lds_u8* lsm, uint32_t kbo, uint32_t vbo,
                                           LdsLanes<D> ln, bool with_pv,
                                           const u32x4 (&pb)[2][2],
                                           f32x16 (&acc)[Geo16<D>::DB],
                                           const u32x4 (&qf)[Geo16<D>::KS], f32x16 (&s)[2]) {
  using G = Geo16<D>;
  constexpr int ROWB = G::ROWB;
  // The MFMA phase runs at raised wave priority, so that when the other wave
  // of the SIMD (in its VALU phase) also has instructions ready, the MFMAs,
  // each of which keeps the matrix pipe busy for many cycles, issue first.
  __builtin_amdgcn_s_setprio(3);
  // The per-fragment addresses are left to the compiler, which hoists some of
  // them out of the key loop: forcing fresh copies each phase (so that every
  // XOR is formed inside the phase) measured about 1 % slower at d = 128.
  const uint32_t kq = ln.kq, vq = ln.vq;
  if (with_pv) pv_tile<E, D>(lsm, vq, vbo, pb, acc);
  const uint32_t kqb = kq + kbo;
  s[0] = (f32x16){};
  s[1] = (f32x16){};
#pragma unroll
  for (int ks = 0; ks < G::KS; ++ks) {
    const lds_u8* ka = lsm + (kqb ^ (uint32_t)(ks << 5));
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const u32x4 a = *(const lds_u32x4*)(ka + sb * 32 * ROWB);
      s[sb] = E::mfma(a, qf[ks], s[sb]);
    }
  }
  // Schedule: LDS reads run LA MFMAs ahead of the MFMA that consumes them.
  constexpr int LA = 4, NPV = 4 * G::DB, NQK = 2 * G::KS;
  constexpr int DSR = 0x100, MFMA = 0x008;
  if (with_pv) {
    __builtin_amdgcn_sched_group_barrier(DSR, 2 * LA, 0);
#pragma unroll
    for (int i = 0; i < NPV - LA; ++i) {
      __builtin_amdgcn_sched_group_barrier(MFMA, 1, 0);
      __builtin_amdgcn_sched_group_barrier(DSR, 2, 0);
    }
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      __builtin_amdgcn_sched_group_barrier(MFMA, 1, 0);
      __builtin_amdgcn_sched_group_barrier(DSR, 1, 0);
    }
  } else {
    __builtin_amdgcn_sched_group_barrier(DSR, LA, 0);
  }
#pragma unroll
  for (int i = 0; i < NQK - LA; ++i) {
    __builtin_amdgcn_sched_group_barrier(MFMA, 1, 0);
    __builtin_amdgcn_sched_group_barrier(DSR, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(MFMA, LA, 0);
  __builtin_amdgcn_s_setprio(0);
}

// S = K Q^T over one 64-key K tile (LDS byte offset kbo) alone: the rare
// path of the sum test forms S again rather than keeping it live.
template <class E, int D>
__device__ __forceinline__ void qk_tile(const lds_u8* lsm, uint32_t kbo, LdsLanes<D> ln,
                                        const u32x4 (&qf)[Geo16<D>::KS], f32x16 (&s)[2]) {
  using G = Geo16<D>;
  const uint32_t kqb = ln.kq + kbo;
  s[0] = (f32x16){};
  s[1] = (f32x16){};
#pragma unroll
  for (int ks = 0; ks < G::KS; ++ks) {
    const lds_u8* ka = lsm + (kqb ^ (uint32_t)(ks << 5));
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
      s[sb] = E::mfma(*(const lds_u32x4*)(ka + sb * 32 * G::ROWB), qf[ks], s[sb]);
  }
}

// Tile loads of the ping-pong kernel, issued by the four waves of one group.
// One buffer descriptor per tile and tensor: its base is the tile's first row
// and its size covers only the tile's rows below N, so the hardware range
// check zero-fills rows past the end of the sequence.  Load u of issuing wave
// w fills LDS block u * 4 + w (rows u * STEP_ROWS + r0, as in TileLoader); the
// per-lane source offsets are loop invariants.
template <int D>
struct PPLoader {
  using G = Geo16<D, 4>;
  static constexpr int NW = 4;
  static constexpr int LPW = G::LOADS_PER_WAVE;  // loads per wave per tensor and tile
  static constexpr int STEP_ROWS = NW * G::ROWS_PER_LOAD;  // rows between loads u, u+1
  uint32_t koff, voff;
  int krs, vrs;  // bytes between consecutive rows of K and of V in memory
  int wave;

  __device__ __forceinline__ PPLoader(int w, int k_row_bytes, int v_row_bytes)
      : krs(k_row_bytes), vrs(v_row_bytes), wave(w) {
    const int lane = threadIdx.x & 63;
    const int r0 = wave * G::ROWS_PER_LOAD + lane / G::CH;
    const int p = lane % G::CH;
    koff = (uint32_t)(r0 * krs + ((p ^ swz_k<D>(r0)) << 4));
    voff = (uint32_t)(r0 * vrs + ((p ^ swz_v<D>(r0)) << 4));
  }
  // Rows j0 .. j0+63 of X (row stride rs bytes) into the tile at LDS byte
  // address lds.  A tile that starts at or past row N gets a descriptor of
  // size 0: it reads as zeros and touches no memory.
  __device__ __forceinline__ void load(const unsigned char* Xb, uint32_t off, int rs, int j0,
                                       int N, uint32_t lds) const {
    const i32x4 rsrc = buffer_rsrc(Xb + (size_t)j0 * rs, j0 < N ? (N - j0) * rs : 0);
#pragma unroll
    for (int u = 0; u < LPW; ++u)
      lds_dma16(rsrc, off + (uint32_t)(u * STEP_ROWS * rs),
                lds + (uint32_t)((u * NW + wave) * G::LOADB));
  }
};


// --- ping-pong kernel ----------------------------------------------------------
//
// 8 waves = 256 query rows per block, in two groups of 4 waves; waves w and
// w + 4 run on the same SIMD.  Per key tile each wave has an MFMA phase
// (acc += P_{t-1} V_{t-1}, then S_t = K_t Q^T: 2 x 16 MFMAs) and a VALU phase
// (row max, rare rescale, P_t = 2^(t - m), row sum).  Execution proceeds in
// barrier-separated slots; group 1 runs one slot behind group 0, so in every
// slot one wave of each SIMD issues MFMAs while the other issues the VALU
// work that the MFMA pipe cannot do, instead of both competing for the same
// unit at the same time.
//
// Slot k (every wave passes the same barriers): group 0 runs the MFMA phase
// of tile k/2 at even k and its VALU phase at odd k; group 1 does the same one
// slot later.  Slot 2T is group 0's final P_{T-1} V_{T-1}, slot 2T + 1 group
// 1's.
//
// K and V tiles stream through four-deep LDS rings (tile t in ring slot
// t % 4).  Each group loads one tensor, right after its MFMA phase, where the
// wave's issue port has slack (the VALU phases are the longer ones):
//   * group 0, after the MFMA phase of tile t (slot 2t), loads V_{t+2}, which
//     overwrites V_{t-2}; it awaits V_t at the end of its VALU phase of tile
//     t (slot 2t + 1), in time for the MFMA phase of tile t + 1;
//   * group 1, after the MFMA phase of tile t (slot 2t + 1), loads K_{t+3},
//     which overwrites K_{t-1}, and awaits K_{t+1} right away, in time for
//     the MFMA phase of tile t + 1 at slot 2t + 2.
// The overwritten tiles were last read by the MFMA phases of tile t - 1
// (slots 2t - 2 and 2t - 1).  Each load has about four slots to arrive: the
// query blocks of a head stream the same tiles at about the same time, and
// the first of them to ask for a tile pays the full memory latency.  K_0..K_2
// and V_0, V_1 are loaded before the first slot.
constexpr int kPPThreads = 512;
constexpr int kRing = 4;

template <class E, int D, bool CAUSAL>
__global__ __launch_bounds__(kPPThreads) __attribute__((amdgpu_waves_per_eu(2)))
void attn_fwd_pp16(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                   const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                   float* __restrict__ LSE, int N, int nqt, float c2, Layout L, Split sp) {
  using G = Geo16<D, 8>;
  constexpr int BM = 256;
  constexpr uint32_t TB = G::TILEB;
  constexpr uint32_t VRING = kRing * TB;  // the V ring follows the K ring
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * kRing * G::TILEB];
  const lds_u8* const lsm = (const lds_u8*)smem;
  const uint32_t lbase = lds_addr(lsm);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = wave >> 2;
  const int li = lane & 31, hh = lane >> 5;

  const WorkItem wi = query_item<CAUSAL>(nqt);
  const int bh = wi.bh, qt = wi.t;
  const uint16_t* const Qh = Q + L.base(L.q, bh);
  uint16_t* const Oh = O + L.base(L.o, bh);
  // this block's keys: rows kb0 .. kb0 + Nk - 1 of the head (all of them without a split)
  const int kb0 = sp.first_key(), Nk = sp.keys();
  const unsigned char* Kb =
      reinterpret_cast<const unsigned char*>(K + L.base(L.k, bh) + (long long)kb0 * L.k[2]);
  const unsigned char* Vb =
      reinterpret_cast<const unsigned char*>(V + L.base(L.v, bh) + (long long)kb0 * L.v[2]);

  const int T = key_tiles<CAUSAL>(Nk, qt * BM, BM, G::BN);
  // Group 0 loads V tiles, group 1 K tiles; all values here are wave-uniform.
  const PPLoader<D> loader(wave & 3, (int)(L.k[2] * 2), (int)(L.v[2] * 2));
  constexpr int LPW = PPLoader<D>::LPW;
  const unsigned char* const Xb = grp == 0 ? Vb : Kb;
  const uint32_t xoff = grp == 0 ? loader.voff : loader.koff;
  const int xrs = grp == 0 ? loader.vrs : loader.krs;
  const uint32_t xring = lbase + (grp == 0 ? VRING : 0u);
  auto load_tile = [&](int j) __attribute__((always_inline)) {  // tile j of this group's tensor, into ring slot j % 4
    loader.load(Xb, xoff, xrs, j * G::BN, Nk, xring + (uint32_t)(j % kRing) * TB);
  };
  // Wait until at most the loads of tiles j+1 and j+2 (those that exist) are
  // still in flight, i.e. until tile j has landed (loads complete in order).
  auto wait_tile = [&](int j) __attribute__((always_inline)) {
    if (j + 2 < T)
      wait_vmcnt<2 * LPW>();
    else if (j + 1 < T)
      wait_vmcnt<LPW>();
    else
      wait_vmcnt<0>();
  };
  if (grp == 0) {
    load_tile(0);
    if (T > 1) load_tile(1);
  } else {
    load_tile(0);
    if (T > 1) load_tile(1);
    if (T > 2) load_tile(2);
  }

  const int qrow = qt * BM + wave * 32 + li;
  const KeyLimit<CAUSAL> kl(Nk, qrow, qt * BM + wave * 32);
  u32x4 qf[G::KS];
  if (qrow < N) {
    const u32x4* qp = reinterpret_cast<const u32x4*>(Qh + (size_t)qrow * L.q[2] + 8 * hh);
#pragma unroll
    for (int ks = 0; ks < G::KS; ++ks) qf[ks] = qp[2 * ks];
  } else {
#pragma unroll
    for (int ks = 0; ks < G::KS; ++ks) qf[ks] = (u32x4){0u, 0u, 0u, 0u};
  }
  f32x16 acc[G::DB];
#pragma unroll
  for (int db = 0; db < G::DB; ++db) acc[db] = (f32x16){};
  float m = -INFINITY;
  f32x2 l = (f32x2){0.f, 0.f};  // row sums of the fp32 P and of the rounded P
  f32x16 sc[2];
  u32x4 pb[2][2];
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int hq = 0; hq < 2; ++hq) pb[sb][hq] = (u32x4){0u, 0u, 0u, 0u};
  wait_vmcnt<0>();
  // The compiler cannot see the DMA loads (inline asm) and would otherwise
  // place its own waits for the Q loads at their first use, inside an MFMA
  // phase, counting only the loads it knows of: with tile loads in flight
  // those waits would stall on them.  Using Q here retires its loads in the
  // compiler's bookkeeping before any tile load is issued.
#pragma unroll
  for (int ks = 0; ks < G::KS; ++ks) __asm__ volatile("" ::"v"(qf[ks]));

  // --- phases -----------------------------------------------------------
  // MFMA phase of tile t: reads K_t from K ring slot t % 4 and, for t >= 1,
  // V_{t-1} from V ring slot (t - 1) % 4.
  const LdsLanes<D> ln;
  auto mfma_tile = [&](int t) __attribute__((always_inline)) {
    const uint32_t kbo = (uint32_t)(t % kRing) * TB;
    const uint32_t vbo = VRING + (uint32_t)((t + kRing - 1) % kRing) * TB;
    mfma_phase<E, D>(lsm, kbo, vbo, ln, t > 0, pb, acc, qf, sc);
  };
  // VALU phase of tile t.
  // The rare path forms S again from K_t, which stays in its ring slot until
  // both groups have finished the VALU phase of tile t.
  // Full tiles take the sum test; the causal kernel's diagonal tiles keep the
  // max test (its masking code leaves no registers for the second pass).
  auto valu_full = [&](int t) __attribute__((always_inline)) {
    f32x2 ps = softmax16<E, false, true, true>(sc, m, c2, pb, 0, 0);
    if (__builtin_amdgcn_ballot_w64(ps[0] > kSumLimit) != 0) {  // rare; wave-uniform
      qk_tile<E, D>(lsm, (uint32_t)(t % kRing) * TB, ln, qf, sc);
      rescale_to<D>(tile_max16(sc, c2), m, l, acc);
      ps = softmax16<E, false, true, true>(sc, m, c2, pb, 0, 0);
    }
    l += ps;
  };
  // The first tile sets the reference from its row max (m = -inf before).
  auto valu_first = [&]() __attribute__((always_inline)) {
    if (kl.partial(0, G::BN)) {
      mask_tail16(sc, 0, kl.lane_lim, c2);
      rescale_to<D>(tile_max16(sc, c2), m, l, acc);
      l += softmax16<E, true, true, true>(sc, m, c2, pb, 0, kl.lane_lim);
    } else {
      rescale_to<D>(tile_max16(sc, c2), m, l, acc);
      l += softmax16<E, false, true, true>(sc, m, c2, pb, 0, 0);
    }
  };
  // A tile that crosses the wave's causal diagonal (the max test).
  auto valu_diag = [&](int t) __attribute__((always_inline)) {
    const int j0 = t * G::BN;
    mask_tail16(sc, j0, kl.lane_lim, c2);
    maybe_rescale<D>(tile_max16(sc, c2), m, l, acc, kRescaleThreshold);
    l += softmax16<E, true, true, true>(sc, m, c2, pb, j0, kl.lane_lim);
  };
  auto valu_any = [&](int t) __attribute__((always_inline)) {
    const int j0 = t * G::BN;
    if (kl.partial(j0, G::BN)) {
      if (CAUSAL) {
        valu_diag(t);
        return;
      }
      f32x2 ps = softmax16<E, true, true, true>(sc, m, c2, pb, j0, kl.lane_lim);
      if (__builtin_amdgcn_ballot_w64(ps[0] > kSumLimit) != 0) {
        qk_tile<E, D>(lsm, (uint32_t)(t % kRing) * TB, ln, qf, sc);
        mask_tail16(sc, j0, kl.lane_lim, c2);
        rescale_to<D>(tile_max16(sc, c2), m, l, acc);
        ps = softmax16<E, true, true, true>(sc, m, c2, pb, j0, kl.lane_lim);
      }
      l += ps;
    } else {
      valu_full(t);
    }
  };
  // Tiles between the first and the last run in two stretches: 1 .. tmid-1,
  // which every row of the wave sees whole (the unmasked VALU phase, the
  // whole stretch without a causal mask), then tmid .. T-2, which with a
  // causal mask cross the wave's diagonal.  Keeping the diagonal tiles out
  // of the main loop keeps their masking code out of its register
  // allocation and schedule.  The stretches differ between waves, but every
  // wave runs T-2 iterations in all, so the barrier count is the same.
  const int tmid = CAUSAL ? min(T - 1, max(1, (kl.wave_lim + 1) / G::BN)) : T - 1;
  auto pv_last = [&]() __attribute__((always_inline)) {
    uint32_t vq = ln.vq;
    __asm__ volatile("" : "+v"(vq));
    pv_tile<E, D>(lsm, vq, VRING + (uint32_t)((T - 1) % kRing) * TB, pb, acc);
  };

  // --- the two schedules: 2T + 2 barriers each ----------------------------
  // One loop body per group over the full tiles 1 .. T-2; tile 0 and the
  // last tile (which may be partial) are peeled.
  if (grp == 0) {
    // slot 2t: MFMA phase of tile t, load V_{t+2}; slot 2t+1: VALU phase of
    // tile t, await V_t.
    block_barrier(); mfma_tile(0); if (2 < T) load_tile(2);
    block_barrier(); valu_first(); wait_tile(0);
    for (int t = 1; t < tmid; ++t) {
      block_barrier(); mfma_tile(t); if (t + 2 < T) load_tile(t + 2);
      block_barrier(); valu_full(t); wait_tile(t);
    }
    if (CAUSAL)
      for (int t = tmid; t < T - 1; ++t) {
        block_barrier(); mfma_tile(t); if (t + 2 < T) load_tile(t + 2);
        block_barrier(); valu_diag(t); wait_tile(t);
      }
    if (T > 1) {
      block_barrier(); mfma_tile(T - 1);
      block_barrier(); valu_any(T - 1); wait_tile(T - 1);
    }
    block_barrier(); pv_last();  // slot 2T
    block_barrier();             // slot 2T + 1
  } else {
    // one slot behind: slot 2t+1: MFMA phase of tile t, load K_{t+3}, await
    // K_{t+1}; slot 2t+2: VALU phase of tile t.
    block_barrier();  // slot 0
    block_barrier(); mfma_tile(0); if (3 < T) load_tile(3); wait_tile(1);
    block_barrier(); valu_first();
    for (int t = 1; t < tmid; ++t) {
      block_barrier(); mfma_tile(t); if (t + 3 < T) load_tile(t + 3); wait_tile(t + 1);
      block_barrier(); valu_full(t);
    }
    if (CAUSAL)
      for (int t = tmid; t < T - 1; ++t) {
        block_barrier(); mfma_tile(t); if (t + 3 < T) load_tile(t + 3); wait_tile(t + 1);
        block_barrier(); valu_diag(t);
      }
    if (T > 1) {
      block_barrier(); mfma_tile(T - 1); wait_tile(T);
      block_barrier(); valu_any(T - 1);
    }
    block_barrier(); pv_last();  // slot 2T + 1
  }

  const float lt = xhalf_sum(l[0]);
  const float inv = 1.0f / xhalf_sum(l[1]);
  const float lse = (m + log2f(lt)) * kLn2;
  if (sp.len) {
    if (qrow < N) store_row16<E, D>(Oh, LSE, sp, L, bh, gridDim.x / nqt, N, qrow, acc, inv, lse);
  } else {
    static_assert(kPPThreads / 64 * 32 * 2 * D <= kRing * G::TILEB,
                  "the output staging must fit in the K ring");
    // The K ring is free here: its last reader, the VALU phase of the last
    // tile (whose rare path may form S again from K), ended at this wave's
    // last barrier, and every tile load has landed.  Wave w takes bytes
    // w * 32 * 2D .. of it (8 waves x 8 KiB = the 4 K slots at d = 128).
    store_rows_lds<E, D>((lds_u8*)smem + wave * 32 * 2 * D, Oh, LSE, L, bh, N,
                         qt * BM + wave * 32, acc, inv, lse);
  }
}

// ---------------------------------------------------------------------------
// fp32 kernel: same structure on v_mfma_f32_32x32x2_f32, P kept in fp32.
// ---------------------------------------------------------------------------
template <int D>
struct Geo32 {
  static constexpr int BN = 32;
  static constexpr int ROWB = D * 4;
  static constexpr int CH = D / 4;             // 16-byte chunks per row
  static constexpr int TILEB = BN * ROWB;
  static constexpr int QV = D / 2;             // Q values per lane
  static constexpr int DB = D / 32;
  static constexpr int SMEM = 4 * TILEB;
};

// K rows are read 16 bytes at a time by 32 lanes of distinct rows; V rows are
// read 128 contiguous bytes per lane half, the two halves 4 rows apart.
template <int D> __device__ __forceinline__ int swz32_k(int row) { return row & 15; }
template <int D> __device__ __forceinline__ int swz32_v(int row) { return ((row >> 2) & 1) << 3; }

__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// KS > 1 (grids of a few blocks): the block's four waves split as RG = 4 / KS
// row groups of 32 rows times KS key groups; key group kh takes the tiles
// t = kh mod KS with its own double buffer, loaded by its own RG waves, and
// at the end groups 1 .. KS-1 hand their (m, l, acc) to group 0 through LDS,
// which merges them exactly as the per-tile rescale does.  Every group's
// first tile holds keys (at least 32 KS keys per head).  Without a causal
// mask.
template <int D, bool CAUSAL, int KS = 1>
__global__ __launch_bounds__(kThreads) void attn_fwd_mfma32(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int N, int nqt, float c2, Layout L, Split sp) {
  using G = Geo32<D>;
  static_assert(KS == 1 || !CAUSAL, "the key split is for the plain forward");
  constexpr int RG = 4 / KS, BM = 32 * RG;
  constexpr int GT = 64 * RG;                   // threads that load a key group's tiles
  constexpr int CPT = G::BN * G::CH / GT;       // 16-byte chunks per thread per tile
  __shared__ __attribute__((aligned(16))) unsigned char smem[G::SMEM * KS];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 31, hh = lane >> 5;
  const int rw = wave % RG, kh = wave / RG;     // row group, key group
  const int gt = rw * 64 + lane;                // thread index within the key group
  unsigned char* const lsm = smem + kh * G::SMEM;

  const WorkItem wi = query_item<CAUSAL>(nqt);
  const int bh = wi.bh, qt = wi.t;
  const float* Qh = Q + L.base(L.q, bh);
  // this block's keys: rows kb0 .. kb0 + Nk - 1 of the head (all of them without a split)
  const int kb0 = sp.first_key(), Nk = sp.keys();
  const float* Kh = K + L.base(L.k, bh) + (long long)kb0 * L.k[2];
  const float* Vh = V + L.base(L.v, bh) + (long long)kb0 * L.v[2];
  float* const Oh = O + L.base(L.o, bh);

  // Contraction index of K*Q^T: lane half hh covers d in [hh*D/2, (hh+1)*D/2),
  // one d per MFMA k-step.
  const int qrow = qt * BM + rw * 32 + li;
  const KeyLimit<CAUSAL> kl(Nk, qrow, qt * BM + rw * 32);
  float qf[G::QV];
  if (qrow < N) {
    const f32x4* qp = reinterpret_cast<const f32x4*>(Qh + (size_t)qrow * L.q[2] + hh * G::QV);
#pragma unroll
    for (int u = 0; u < G::QV / 4; ++u) {
      const f32x4 x = qp[u];
      qf[4 * u + 0] = x[0]; qf[4 * u + 1] = x[1]; qf[4 * u + 2] = x[2]; qf[4 * u + 3] = x[3];
    }
  } else {
#pragma unroll
    for (int u = 0; u < G::QV; ++u) qf[u] = 0.f;
  }

  f32x16 acc[G::DB];
#pragma unroll
  for (int db = 0; db < G::DB; ++db) acc[db] = (f32x16){};
  float m = -INFINITY, l = 0.f;

  // local tile t of this key group is global tile KS t + kh; all groups run ntiles
  const int ntiles = (key_tiles<CAUSAL>(Nk, qt * BM, BM, G::BN) + KS - 1) / KS;
  f32x4 kr[CPT], vr[CPT];
  auto gload = [&](int j0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int ci = gt + u * GT;
      const int row = ci / G::CH, c = ci % G::CH;
      if (j0 + row < Nk) {
        kr[u] = *reinterpret_cast<const f32x4*>(Kh + (size_t)(j0 + row) * L.k[2] + c * 4);
        vr[u] = *reinterpret_cast<const f32x4*>(Vh + (size_t)(j0 + row) * L.v[2] + c * 4);
      } else {
        kr[u] = (f32x4){0.f, 0.f, 0.f, 0.f};
        vr[u] = (f32x4){0.f, 0.f, 0.f, 0.f};
      }
    }
  };
  auto swrite = [&](unsigned char* kb, unsigned char* vb) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int ci = gt + u * GT;
      const int row = ci / G::CH, c = ci % G::CH;
      *reinterpret_cast<f32x4*>(kb + row * G::ROWB + ((c ^ swz32_k<D>(row)) << 4)) = kr[u];
      *reinterpret_cast<f32x4*>(vb + row * G::ROWB + ((c ^ swz32_v<D>(row)) << 4)) = vr[u];
    }
  };
  gload(kh * G::BN);
  swrite(lsm, lsm + G::TILEB);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int j0 = (KS * t + kh) * G::BN;
    const bool more = t + 1 < ntiles;
    if (more) gload(j0 + KS * G::BN);
    const unsigned char* kb = lsm + (t & 1) * 2 * G::TILEB;
    const unsigned char* vb = kb + G::TILEB;

    // S^T = K Q^T for 32 keys.
    f32x16 s = (f32x16){};
    {
      const int row = li;
      const unsigned char* rp = kb + row * G::ROWB;
      const int sw = swz32_k<D>(row);
#pragma unroll
      for (int u = 0; u < G::QV / 4; ++u) {
        const int c = hh * (G::QV / 4) + u;
        const f32x4 a = *reinterpret_cast<const f32x4*>(rp + ((c ^ sw) << 4));
        s = mfma_f32(a[0], qf[4 * u + 0], s);
        s = mfma_f32(a[1], qf[4 * u + 1], s);
        s = mfma_f32(a[2], qf[4 * u + 2], s);
        s = mfma_f32(a[3], qf[4 * u + 3], s);
      }
    }
    const bool tail = kl.partial(j0, G::BN);
    if (tail) {
      const float neutral = c2 >= 0.f ? -INFINITY : INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (j0 + 8 * (r >> 2) + 4 * hh + (r & 3) > kl.lane_lim) s[r] = neutral;
    }
    const float mt = c2 >= 0.f ? xhalf_max(frag_max(s)) : xhalf_min(frag_min(s));
    const float m_new = fmaxf(m, mt * c2);
    const float alpha = fast_exp2(m - m_new);
    m = m_new;
    float rs = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float p = fast_exp2(fmaf(s[r], c2, -m_new));
      if (tail && (j0 + 8 * (r >> 2) + 4 * hh + (r & 3) > kl.lane_lim)) p = 0.f;
      s[r] = p;
      rs += p;
    }
    l = l * alpha + rs;
#pragma unroll
    for (int db = 0; db < G::DB; ++db) acc[db] *= alpha;

    // O^T += V^T P^T: k-step r pairs P of key kr(hh) = 8(r/4) + 4hh + r%4
    // (B, lane half hh) with V row kr(hh), column 32 db + li (A).
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 8 * (r >> 2) + 4 * hh + (r & 3);
      const float* vrow = reinterpret_cast<const float*>(vb + row * G::ROWB);
#pragma unroll
      for (int db = 0; db < G::DB; ++db) {
        const int col = 32 * db + li;
        const int c = col >> 2;
        const float a = vrow[((c ^ swz32_v<D>(row)) << 2) + (col & 3)];
        acc[db] = mfma_f32(a, s[r], acc[db]);
      }
    }
    if (more) {
      unsigned char* nb = lsm + ((t + 1) & 1) * 2 * G::TILEB;
      swrite(nb, nb + G::TILEB);
    }
    __syncthreads();
  }

  if constexpr (KS > 1) {
    // groups 1 .. KS-1 write (acc, m, l) per lane; group 0 merges.  A group
    // whose row saw no key has l = 0 and adds nothing; a NaN l is kept.
    constexpr int NV = G::DB * 16 + 2;
    static_assert((KS - 1) * RG * 64 * NV * 4 <= G::SMEM * KS, "the merge area must fit");
    float* const xs = reinterpret_cast<float*>(smem);
    auto slot = [&](int g) __attribute__((always_inline)) {
      return xs + (size_t)(((g - 1) * RG + rw) * 64 + lane) * NV;
    };
    if (kh > 0) {
      float* const x = slot(kh);
#pragma unroll
      for (int db = 0; db < G::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) x[db * 16 + r] = acc[db][r];
      x[G::DB * 16] = m;
      x[G::DB * 16 + 1] = l;
    }
    __syncthreads();
    if (kh > 0) return;
    float mg[KS], lg[KS];
    bool hg[KS];
    mg[0] = m, lg[0] = l, hg[0] = xhalf_sum(l) != 0.f;
    float mn = hg[0] ? m : -INFINITY;
#pragma unroll
    for (int g = 1; g < KS; ++g) {
      mg[g] = slot(g)[G::DB * 16];
      lg[g] = slot(g)[G::DB * 16 + 1];
      hg[g] = xhalf_sum(lg[g]) != 0.f;
      if (hg[g]) mn = fmaxf(mn, mg[g]);
    }
    const float a0 = hg[0] ? fast_exp2(m - mn) : 0.f;
    l = hg[0] ? l * a0 : 0.f;
#pragma unroll
    for (int db = 0; db < G::DB; ++db) acc[db] = hg[0] ? acc[db] * a0 : (f32x16){};
#pragma unroll
    for (int g = 1; g < KS; ++g) {
      if (!hg[g]) continue;
      const float ag = fast_exp2(mg[g] - mn);
      const float* const x = slot(g);
      l += lg[g] * ag;
#pragma unroll
      for (int db = 0; db < G::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] += x[db * 16 + r] * ag;
    }
    m = mn;
  }

  const float lt = xhalf_sum(l);
  const float inv = 1.0f / lt;
  if (qrow < N) {
    float* op;
    if (sp.len) {
      const size_t r = ((size_t)blockIdx.y * (gridDim.x / nqt) + bh) * N + qrow;
      op = sp.opart + r * D;
      if (hh == 0) sp.lpart[r] = (m + log2f(lt)) * kLn2;
    } else {
      op = Oh + (size_t)qrow * L.o[2];
      if (LSE != nullptr && hh == 0) LSE[(size_t)bh * N + qrow] = (m + log2f(lt)) * kLn2;
    }
#pragma unroll
    for (int db = 0; db < G::DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = 32 * db + 8 * g + 4 * hh;
        *reinterpret_cast<f32x4*>(op + col) =
            (f32x4){acc[db][4 * g + 0] * inv, acc[db][4 * g + 1] * inv,
                    acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv};
      }
  }
}

// ---------------------------------------------------------------------------
// decode kernel: a few query rows against many keys
// ---------------------------------------------------------------------------
//
// With at most four query rows per head (generation: each new position scored
// against the whole cache of keys and values, which page 3 section 4 names as
// the memory-bandwidth-bound case of inference) an MFMA tile of 32 query rows
// would be almost all padding, and the time is that of reading K and V once.
// This kernel streams them with plain coalesced 16-byte loads and computes
// on the VALU:
//   * a group of LPR lanes holds one key (or value) row, each lane PPL
//     16-byte pieces of it; a wave covers G = 64 / LPR rows per load and keeps
//     U rows per group in flight (8 loads of 16 bytes per lane for K, 8 for
//     V);
//   * a score is the lane's partial dot product (v_dot2 for the 16-bit
//     types) summed over the group with DPP exchanges (xor 1, xor 2, then the
//     mirrors within 8 and within 16 lanes), which leaves the identical sum
//     in every lane of the group;
//   * each group runs the online softmax (page 1 section 4) over its rows
//     for each query: running max m, sum l and the lane's EPL columns of the
//     accumulator;
//   * at the end the 4 G group states of the block are merged through LDS
//     with the same exact rescaling as the split-KV merge, and wave 0 writes
//     the output rows (or, on the split-KV path, the fp32 partial results).
// The block takes the keys of its split (all keys without one) in steps of
// 4 waves x G x U rows; rows past the end are loaded from the last valid row
// and given probability 0.  Non-causal only.
// (A vector element is copied to a scalar before __builtin_bit_cast: the
// cast applied to a subscripted element of an ext_vector_type compiled to a
// read of element 0 for every subscript here.)
template <class T> struct DecElem;
template <> struct DecElem<Bf16T> {
  static constexpr int EP = 8;  // elements per 16 bytes
  static __device__ __forceinline__ float dot(u32x4 a, u32x4 b, float c) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32 ai = a[i], bi = b[i];
      c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, ai),
                                          __builtin_bit_cast(bf16x2, bi), c, false);
    }
    return c;
  }
  static __device__ __forceinline__ void widen(u32x4 x, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(x[i] << 16);
      f[2 * i + 1] = __uint_as_float(x[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ u32x4 narrow(const float* f) {
    return (u32x4){Bf16T::pack2(f[0], f[1]), Bf16T::pack2(f[2], f[3]), Bf16T::pack2(f[4], f[5]),
                   Bf16T::pack2(f[6], f[7])};
  }
};
template <> struct DecElem<F16T> {
  static constexpr int EP = 8;
  static __device__ __forceinline__ float dot(u32x4 a, u32x4 b, float c) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32 ai = a[i], bi = b[i];
      c = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, ai), __builtin_bit_cast(f16x2, bi), c,
                                 false);
    }
    return c;
  }
  static __device__ __forceinline__ void widen(u32x4 x, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32 xi = x[i];
      const f16x2 h = __builtin_bit_cast(f16x2, xi);
      f[2 * i] = (float)h[0];
      f[2 * i + 1] = (float)h[1];
    }
  }
  static __device__ __forceinline__ u32x4 narrow(const float* f) {
    return (u32x4){F16T::pack2(f[0], f[1]), F16T::pack2(f[2], f[3]), F16T::pack2(f[4], f[5]),
                   F16T::pack2(f[6], f[7])};
  }
};
struct F32T {};
template <> struct DecElem<F32T> {
  static constexpr int EP = 4;
  static __device__ __forceinline__ float dot(u32x4 a, u32x4 b, float c) {
#pragma unroll
    for (int i = 0; i < 4; ++i) c = fmaf(__uint_as_float(a[i]), __uint_as_float(b[i]), c);
    return c;
  }
  static __device__ __forceinline__ void widen(u32x4 x, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(x[i]);
  }
  static __device__ __forceinline__ u32x4 narrow(const float* f) {
    return (u32x4){__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                   __float_as_uint(f[3])};
  }
};

template <int ES, int D>
struct GeoDec {
  static constexpr int ROWB = D * ES;                       // bytes of a K or V row
  static constexpr int LPR = ROWB / 16 < 16 ? ROWB / 16 : 16;  // lanes per row
  static constexpr int PPL = ROWB / (16 * LPR);             // 16-byte pieces per lane
  static constexpr int EPL = PPL * 16 / ES;                 // elements per lane
  static constexpr int G = 64 / LPR;                        // rows per wave and load
  static constexpr int U = 8 / PPL;                         // rows per group in flight
  static constexpr int RB = 4 * G * U;                      // rows per block step
  static_assert(LPR == 8 || LPR == 16, "group sums cover 8 or 16 lanes");
};

// The value of another lane of the same row of 16, by a DPP pattern.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}

// Sum over aligned groups of LPR (8 or 16) lanes, the same value in each lane:
// every step adds a value and its exchange partner's, and a + b == b + a.
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp_f32<0xB1>(x);                            // quad_perm [1,0,3,2]: lane i ^ 1
  x += dpp_f32<0x4E>(x);                            // quad_perm [2,3,0,1]: lane i ^ 2
  x += dpp_f32<0x141>(x);                           // row_half_mirror: i <-> 7 - i
  if constexpr (LPR == 16) x += dpp_f32<0x140>(x);  // row_mirror: i <-> 15 - i
  return x;
}

template <class E, class T, int D, int NQ>
__global__ __launch_bounds__(kThreads) void attn_fwd_dec(const T* __restrict__ Q,
                                                         const T* __restrict__ K,
                                                         const T* __restrict__ V,
                                                         T* __restrict__ O,
                                                         float* __restrict__ LSE, int N, int nqt,
                                                         float c2, Layout L, Split sp) {
  using G = GeoDec<(int)sizeof(T), D>;
  using X = DecElem<E>;
  constexpr int LPR = G::LPR, PPL = G::PPL, EPL = G::EPL, GR = G::G, U = G::U;
  constexpr int NS = NQ * (EPL + 2);  // floats of one lane's state
  __shared__ float st[4 * 64 * NS];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int g = lane / LPR, j = lane % LPR;
  const int bh = blockIdx.x;
  (void)nqt;

  // the lane's pieces of the query rows (zero past N)
  u32x4 qf[NQ][PPL];
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi)
#pragma unroll
    for (int p = 0; p < PPL; ++p) {
      qf[qi][p] = (u32x4){0u, 0u, 0u, 0u};
      if (qi < N)
        qf[qi][p] = *reinterpret_cast<const u32x4*>(Q + L.base(L.q, bh) + (long long)qi * L.q[2] +
                                                    (j * PPL + p) * (16 / sizeof(T)));
    }

  const int kb0 = sp.first_key(), nkb = sp.keys();
  const unsigned char* const Kb = reinterpret_cast<const unsigned char*>(
      K + L.base(L.k, bh) + (long long)kb0 * L.k[2]) + j * PPL * 16;
  const unsigned char* const Vb = reinterpret_cast<const unsigned char*>(
      V + L.base(L.v, bh) + (long long)kb0 * L.v[2]) + j * PPL * 16;
  const int krs = (int)(L.k[2] * sizeof(T)), vrs = (int)(L.v[2] * sizeof(T));

  float m[NQ], l[NQ], acc[NQ][EPL];
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi) {
    m[qi] = -INFINITY;
    l[qi] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[qi][e] = 0.f;
  }

  for (int r0 = wave * GR * U; r0 < nkb; r0 += G::RB) {
    u32x4 kx[U][PPL], vx[U][PPL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = min(r0 + u * GR + g, nkb - 1);
#pragma unroll
      for (int p = 0; p < PPL; ++p) {
        kx[u][p] = *reinterpret_cast<const u32x4*>(Kb + r * krs + 16 * p);
        vx[u][p] = *reinterpret_cast<const u32x4*>(Vb + r * vrs + 16 * p);
      }
    }
    float pr[NQ][U];
#pragma unroll
    for (int qi = 0; qi < NQ; ++qi) {
      float s[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float a = 0.f;
#pragma unroll
        for (int p = 0; p < PPL; ++p) a = X::dot(qf[qi][p], kx[u][p], a);
        s[u] = r0 + u * GR + g < nkb ? group_sum<LPR>(a) * c2 : -INFINITY;
      }
      float mx = s[0];
#pragma unroll
      for (int u = 1; u < U; ++u) mx = fmaxf(mx, s[u]);
      const float mn = fmaxf(m[qi], mx);
      const float mr = mn == -INFINITY ? 0.f : mn;  // no finite score yet: all p are 0
      const float al = fast_exp2(m[qi] - mr);
      m[qi] = mn;
      float ps = 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        pr[qi][u] = fast_exp2(s[u] - mr);
        ps += pr[qi][u];
      }
      l[qi] = fmaf(l[qi], al, ps);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[qi][e] *= al;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float vf[EPL];
#pragma unroll
      for (int p = 0; p < PPL; ++p) X::widen(vx[u][p], vf + p * X::EP);
#pragma unroll
      for (int qi = 0; qi < NQ; ++qi)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[qi][e] = fmaf(pr[qi][u], vf[e], acc[qi][e]);
    }
  }

  // merge the 4 x GR group states of the block: state (w, g) of query qi
  // holds m, l (equal in its LPR lanes) and each lane's EPL columns
  float* const mine = st + (wave * 64 + lane) * NS;
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) mine[qi * (EPL + 2) + e] = acc[qi][e];
    mine[qi * (EPL + 2) + EPL] = m[qi];
    mine[qi * (EPL + 2) + EPL + 1] = l[qi];
  }
  __syncthreads();
  if (wave != 0) return;
  const int qi = lane / LPR;  // wave 0: query qi, column piece j
  if (qi >= NQ || qi >= N) return;
  float M = -INFINITY;
  for (int w = 0; w < 4; ++w)
    for (int gg = 0; gg < GR; ++gg)
      M = fmaxf(M, st[(w * 64 + gg * LPR + j) * NS + qi * (EPL + 2) + EPL]);
  const float Mr = M == -INFINITY ? 0.f : M;
  float lt = 0.f, o[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = 0.f;
  for (int w = 0; w < 4; ++w)
    for (int gg = 0; gg < GR; ++gg) {
      const float* const x = st + (w * 64 + gg * LPR + j) * NS + qi * (EPL + 2);
      const float wt = fast_exp2(x[EPL] - Mr);
      lt = fmaf(wt, x[EPL + 1], lt);
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] = fmaf(wt, x[e], o[e]);
    }
  const float inv = 1.0f / lt;
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] *= inv;
  const float lse = (M + log2f(lt)) * kLn2;
  if (sp.len) {
    const size_t r = ((size_t)blockIdx.y * gridDim.x + bh) * N + qi;
    float* const op = sp.opart + r * D + j * EPL;
#pragma unroll
    for (int e = 0; e < EPL; e += 4)
      *reinterpret_cast<f32x4*>(op + e) = (f32x4){o[e], o[e + 1], o[e + 2], o[e + 3]};
    if (j == 0) sp.lpart[r] = lse;
  } else {
    unsigned char* const op = reinterpret_cast<unsigned char*>(
        O + L.base(L.o, bh) + (long long)qi * L.o[2]) + j * PPL * 16;
#pragma unroll
    for (int p = 0; p < PPL; ++p)
      *reinterpret_cast<u32x4*>(op + 16 * p) = X::narrow(o + p * X::EP);
    if (LSE != nullptr && j == 0) LSE[(size_t)bh * N + qi] = lse;
  }
}

// ---------------------------------------------------------------------------
// split-KV merge
// ---------------------------------------------------------------------------
//
// Each split of a row's keys produced its own normalised output O_s and
// log-sum-exp lse_s.  They combine exactly as the per-block statistics of a
// long softmax row do (page 3 section 1.1: the maxima and sums of the blocks
// merge into the row's; section 5 stores lse for this purpose):
//   lse = ln sum_s exp(lse_s),   O = sum_s exp(lse_s - lse) O_s.
// One thread handles four consecutive columns of one row; the sum runs with
// the largest lse_s subtracted, as a softmax over the splits.
struct OutF32 {
  static __device__ __forceinline__ void store4(float* p, f32x4 v) {
    *reinterpret_cast<f32x4*>(p) = v;
  }
};
template <class E>
struct Out16 {
  static __device__ __forceinline__ void store4(uint16_t* p, f32x4 v) {
    *reinterpret_cast<u32x2*>(p) = (u32x2){E::pack2(v[0], v[1]), E::pack2(v[2], v[3])};
  }
};

constexpr int kMergeThreads = 256;

template <class OUT, class T, int D>
__global__ __launch_bounds__(kMergeThreads) void attn_merge(const float* __restrict__ opart,
                                                            const float* __restrict__ lpart,
                                                            T* __restrict__ O,
                                                            float* __restrict__ LSE, int N,
                                                            int nbh, int S, Layout L) {
  constexpr int TPR = D / 4;                // threads per row
  constexpr int RPB = kMergeThreads / TPR;  // rows per block
  const long long r = (long long)blockIdx.x * RPB + (int)threadIdx.x / TPR;  // of B*H*N rows
  const int c = 4 * ((int)threadIdx.x % TPR);
  const size_t plane = (size_t)nbh * N;
  if (r >= (long long)plane) return;
  // (both loops unrolled so that eight splits' loads are in flight at once:
  // with few rows the merge is a chain of memory latencies)
  float mx = -INFINITY;
#pragma unroll 8
  for (int sp = 0; sp < S; ++sp) mx = fmaxf(mx, lpart[sp * plane + r]);
  float sum = 0.f;
  f32x4 o = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
  for (int sp = 0; sp < S; ++sp) {
    const size_t rs = sp * plane + r;
    const float w = fast_exp2((lpart[rs] - mx) * kLog2e);
    sum += w;
    const f32x4 x = *reinterpret_cast<const f32x4*>(opart + rs * D + c);
    o[0] = fmaf(w, x[0], o[0]);
    o[1] = fmaf(w, x[1], o[1]);
    o[2] = fmaf(w, x[2], o[2]);
    o[3] = fmaf(w, x[3], o[3]);
  }
  const float inv = 1.0f / sum;
  o[0] *= inv, o[1] *= inv, o[2] *= inv, o[3] *= inv;
  const int bh = (int)(r / N), i = (int)(r - (long long)bh * N);
  OUT::store4(O + L.base(L.o, bh) + (long long)i * L.o[2] + c, o);
  if (LSE != nullptr && c == 0) LSE[r] = mx + log2f(sum) * kLn2;
}

// The merge of caller-supplied partial results (attn_fwd_merge): part s is an
// O_s in the element type and its lse_s, each a contiguous [B, H, N(, d)]
// tensor of its own; the same arithmetic as attn_merge.
struct MergeParts {
  const void* o[ATTN_MAX_SPLITS];
  const float* lse[ATTN_MAX_SPLITS];
};
struct InF32 {
  static __device__ __forceinline__ f32x4 load4(const float* p) {
    return *reinterpret_cast<const f32x4*>(p);
  }
};
struct InBf16 {
  static __device__ __forceinline__ f32x4 load4(const uint16_t* p) {
    const u32x2 x = *reinterpret_cast<const u32x2*>(p);
    return (f32x4){__uint_as_float(x[0] << 16), __uint_as_float(x[0] & 0xffff0000u),
                   __uint_as_float(x[1] << 16), __uint_as_float(x[1] & 0xffff0000u)};
  }
};
struct InF16 {
  static __device__ __forceinline__ f32x4 load4(const uint16_t* p) {
    const u32x2 x = *reinterpret_cast<const u32x2*>(p);
    const u32 x0 = x[0], x1 = x[1];
    const f16x2 a = __builtin_bit_cast(f16x2, x0), b = __builtin_bit_cast(f16x2, x1);
    return (f32x4){(float)a[0], (float)a[1], (float)b[0], (float)b[1]};
  }
};

template <class OUT, class IN, class T, int D>
__global__ __launch_bounds__(kMergeThreads) void attn_merge_parts(MergeParts P, int S,
                                                                  T* __restrict__ O,
                                                                  float* __restrict__ LSE,
                                                                  long long rows) {
  constexpr int TPR = D / 4, RPB = kMergeThreads / TPR;
  const long long r = (long long)blockIdx.x * RPB + (int)threadIdx.x / TPR;  // of B*H*N rows
  const int c = 4 * ((int)threadIdx.x % TPR);
  if (r >= rows) return;
  float mx = -INFINITY;
#pragma unroll 8
  for (int sp = 0; sp < S; ++sp) mx = fmaxf(mx, P.lse[sp][r]);
  float sum = 0.f;
  f32x4 o = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
  for (int sp = 0; sp < S; ++sp) {
    const float w = fast_exp2((P.lse[sp][r] - mx) * kLog2e);
    sum += w;
    const f32x4 x = IN::load4(static_cast<const T*>(P.o[sp]) + r * D + c);
    o[0] = fmaf(w, x[0], o[0]);
    o[1] = fmaf(w, x[1], o[1]);
    o[2] = fmaf(w, x[2], o[2]);
    o[3] = fmaf(w, x[3], o[3]);
  }
  const float inv = 1.0f / sum;
  o[0] *= inv, o[1] *= inv, o[2] *= inv, o[3] *= inv;
  OUT::store4(O + r * D + c, o);
  if (LSE != nullptr && c == 0) LSE[r] = mx + log2f(sum) * kLn2;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return na > 0 && nb > 0 && x < y + nb && y < x + na;
}

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

// Everything a launch needs besides the kernel choice.
struct Launch {
  hipStream_t stream;
  const void *q, *k, *v;
  void* o;
  float* lse;
  int64_t bh, N, nk, d;  // heads, query rows, key rows, head dimension
  float c2;
  Layout L;
  Split sp;    // sp.len == 0: no split
  int splits;  // grid y (1 without a split)
};

template <class T>
int launch(void (*kernel)(const T*, const T*, const T*, T*, float*, int, int, float, Layout,
                          Split),
           int64_t nblocks, int threads, int nqt, const Launch& a) {
  hipLaunchKernelGGL(kernel, dim3((unsigned)nblocks, (unsigned)a.splits), dim3(threads), 0,
                     a.stream, static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                     static_cast<const T*>(a.v), static_cast<T*>(a.o), a.lse, (int)a.N, nqt,
                     a.c2, a.L, a.sp);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

constexpr int kNumCUs = 256;  // MI355X

// Kernel choice for the 16-bit types: at d = 128 the 8-wave ping-pong kernel
// (256 query rows per block) when it still gives every CU a block and the
// queries fill more than one 128-row block, else the 4-wave pipelined kernel
// (128 rows per block, up to two blocks per CU).  With at most 128 query rows
// a 256-row block would be half padding or more: a split-KV call of 8 or 16
// rows against 65536 keys (B1 H32) measured 184 us with the pipelined kernel
// against 231 us with the ping-pong kernel.  At d = 64, where the softmax
// work per tile is as large as the MFMA work, the pipelined kernel with up to
// three blocks per CU wins on large grids (workload B1 H8 N65536: 2-8 %),
// but while the grid gives each CU one or two 256-row blocks (two to four
// 128-row ones) the ping-pong kernel's 8 waves per block measured 3-10 %
// faster (B1 H32 N2048: 41.0 against 45.0 us; B1 H16 N4096: 78.2 against
// 84.0; B1 H64 N1024: 23.3 against 25.1), so there it runs at d = 64 too.
// With a causal mask at d = 128 the ping-pong kernel wins from N = 2048 on
// (B2 H16 N4096: 134.6 against 155.6 us; B1 H32 N16384: 1879 against 2162;
// B1 H16 N4096, one block per CU: 95.0 against 98.8), the pipelined kernel
// up to N = 1024 (B1 H256 N1024: 109.7 against 112.1), where the diagonal
// tiles are a large share of the work; at d = 64 the pipelined kernel is
// 4-15 % faster on every causal shape tried.  The environment variable
// ATTN_FWD_KERNEL=pingpong|pipelined forces one (for tests and sweeps).
bool use_pingpong(int64_t blocks256, int64_t N, int64_t d, bool causal) {
  const char* env = getenv("ATTN_FWD_KERNEL");
  if (env != nullptr && strcmp(env, "pingpong") == 0) return true;
  if (env != nullptr && (strcmp(env, "pipelined") == 0 || strcmp(env, "pipelined2") == 0))
    return false;
  if (N <= 128 || blocks256 < kNumCUs) return false;
  if (causal) return d == 128 && N >= 2048;
  return d == 128 || blocks256 <= 2 * kNumCUs;
}

// The pipelined kernel's in-block key split: when the grid of 128-row blocks
// gives at most one block per CU (one wave per SIMD), without a causal mask,
// outside the split-KV path (its epilogue writes the final O only, not the
// fp32 partial results a split-KV call merges, even when that call ends up
// with a single split) and with at least two key tiles (nk > 64).
// ATTN_FWD_KERNEL=pipelined turns it off, =pipelined2 forces it where it
// applies (tests and sweeps).
bool use_key_split(int64_t blocks128, int64_t nk, bool causal, bool splitkv) {
  if (causal || splitkv || nk <= 64) return false;
  const char* env = getenv("ATTN_FWD_KERNEL");
  if (env != nullptr && strcmp(env, "pipelined2") == 0) return true;
  if (env != nullptr && strcmp(env, "pipelined") == 0) return false;
  return blocks128 <= kNumCUs;
}

// The decode kernel: at most four query rows per head, without a causal mask.
// ATTN_FWD_KERNEL=pingpong|pipelined|pipelined2 force an MFMA kernel instead
// (=decode, or no setting, leaves this choice).
bool use_decode(int64_t N, bool causal) {
  if (causal || N > 4) return false;
  const char* env = getenv("ATTN_FWD_KERNEL");
  return env == nullptr || (strcmp(env, "pingpong") != 0 && strcmp(env, "pipelined") != 0 &&
                            strcmp(env, "pipelined2") != 0);
}

template <class E, class T>
int launch_dec(const Launch& a) {
  auto kern = a.d == 128 ? (a.N == 1   ? attn_fwd_dec<E, T, 128, 1>
                            : a.N == 2 ? attn_fwd_dec<E, T, 128, 2>
                                       : attn_fwd_dec<E, T, 128, 4>)
                         : (a.N == 1   ? attn_fwd_dec<E, T, 64, 1>
                            : a.N == 2 ? attn_fwd_dec<E, T, 64, 2>
                                       : attn_fwd_dec<E, T, 64, 4>);
  return launch<T>(kern, a.bh, kThreads, 1, a);
}

template <class E, class T, bool C>
int launch16(const Launch& a) {
  if (use_decode(a.N, C)) return launch_dec<E, T>(a);
  if (use_pingpong(a.bh * ((a.N + 255) / 256) * a.splits, a.N, a.d, C)) {
    const int64_t nqt = (a.N + 255) / 256;
    auto kern = a.d == 128 ? attn_fwd_pp16<E, 128, C> : attn_fwd_pp16<E, 64, C>;
    return launch<T>(kern, a.bh * nqt, kPPThreads, (int)nqt, a);
  }
  const int64_t nqt = (a.N + 127) / 128;
  if (use_key_split(a.bh * nqt, a.nk, C, a.sp.len != 0)) {
    auto kern = a.d == 128 ? attn_fwd_mfma16<E, 128, false, 2> : attn_fwd_mfma16<E, 64, false, 2>;
    return launch<T>(kern, a.bh * nqt, 2 * kThreads, (int)nqt, a);
  }
  auto kern = a.d == 128 ? attn_fwd_mfma16<E, 128, C, 1> : attn_fwd_mfma16<E, 64, C, 1>;
  return launch<T>(kern, a.bh * nqt, kThreads, (int)nqt, a);
}

template <bool C>
int launch32(const Launch& a) {
  if (use_decode(a.N, C)) return launch_dec<F32T, float>(a);
  const int64_t nqt = (a.N + 127) / 128;
  // Few blocks (at most a quarter of the CUs): split each block's keys over
  // its waves (4 groups of 32-key tiles at d = 64, 2 at d = 128, where the
  // LDS holds two groups' buffers) and use more, shorter blocks.  Every
  // group's first tile must hold keys (nk >= 32 groups); not on the split-KV
  // path, whose blocks may hold a single key.
  if (!C && a.sp.len == 0 && a.bh * nqt <= kNumCUs / 4) {
    if (a.d == 64 && a.nk >= 4 * 32) {
      const int64_t n = (a.N + 31) / 32;
      return launch<float>(attn_fwd_mfma32<64, false, 4>, a.bh * n, kThreads, (int)n, a);
    }
    if (a.d == 128 && a.nk >= 2 * 32) {
      const int64_t n = (a.N + 63) / 64;
      return launch<float>(attn_fwd_mfma32<128, false, 2>, a.bh * n, kThreads, (int)n, a);
    }
  }
  auto kern = a.d == 128 ? attn_fwd_mfma32<128, C> : attn_fwd_mfma32<64, C>;
  return launch<float>(kern, a.bh * nqt, kThreads, (int)nqt, a);
}

template <class OUT, class T>
int launch_merge(const Launch& a) {
  const int64_t rows = a.bh * a.N;
  const int tpr = (int)a.d / 4, rpb = kMergeThreads / tpr;
  auto kern = a.d == 128 ? attn_merge<OUT, T, 128> : attn_merge<OUT, T, 64>;
  hipLaunchKernelGGL(kern, dim3((unsigned)((rows + rpb - 1) / rpb)), dim3(kMergeThreads), 0,
                     a.stream, a.sp.opart, a.sp.lpart, static_cast<T*>(a.o), a.lse, (int)a.N,
                     (int)a.bh, a.splits, a.L);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

// Byte ranges of a strided [B, H, N, d] tensor: the lowest and one past the
// highest byte any element occupies (strides are non-negative).
void span_of(const void* p, const int64_t (&st)[3], int64_t B, int64_t H, int64_t N, int64_t d,
             size_t esize, uintptr_t* lo, uintptr_t* hi) {
  const uintptr_t base = reinterpret_cast<uintptr_t>(p);
  const uint64_t last = (uint64_t)(B - 1) * st[0] + (uint64_t)(H - 1) * st[1] +
                        (uint64_t)(N - 1) * st[2] + (uint64_t)(d - 1);
  *lo = base;
  *hi = base + (last + 1) * esize;
}

bool ranges_overlap(uintptr_t a0, uintptr_t a1, uintptr_t b0, uintptr_t b1) {
  return a0 < b1 && b0 < a1;
}

// Rows of one tensor never share bytes: either every (b, h, n) row has its
// own d-element slot under the stride order, which holds when the strides,
// sorted, each cover the extent of the dimensions below them.
bool rows_disjoint(const int64_t (&st)[3], int64_t B, int64_t H, int64_t N, int64_t d) {
  int64_t dims[3][2] = {{st[0], B}, {st[1], H}, {st[2], N}};
  // sort by stride (three elements)
  for (int i = 0; i < 3; ++i)
    for (int j = i + 1; j < 3; ++j)
      if (dims[j][0] < dims[i][0]) {
        int64_t t0 = dims[i][0], t1 = dims[i][1];
        dims[i][0] = dims[j][0], dims[i][1] = dims[j][1];
        dims[j][0] = t0, dims[j][1] = t1;
      }
  int64_t extent = d;  // elements covered by one step of the next dimension
  for (int i = 0; i < 3; ++i) {
    if (dims[i][1] <= 1) continue;  // a dimension of size 1 never steps
    if (dims[i][0] < extent) return false;
    extent = dims[i][0] * dims[i][1];
  }
  return true;
}

// Keys per split (a multiple of the 64-key tile) and the number of non-empty
// splits for a requested split count.
void split_plan(int64_t N, int requested, int64_t* len, int* splits) {
  const int64_t tiles = (N + 63) / 64;
  const int64_t per = (tiles + requested - 1) / requested;
  *len = per * 64;
  *splits = (int)((tiles + per - 1) / per);
}

}  // namespace

// The workspace of attn_fwd_splitkv_static: fp32 partial outputs and
// log-sum-exps between the split-KV kernel and the merge, in a library-owned
// device array (each device that runs the library holds its own copy until
// the process ends).  In host code `scratch` names a host-side stand-in, not
// device memory: only the address hipGetSymbolAddress returns for the
// current device may be handed to kernels.
static __device__ __align__(256) unsigned char scratch[ATTN_STATIC_WORKSPACE_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

// The current device's address of `scratch`, looked up once per device (with
// that device current) and kept.
int static_workspace(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return ATTN_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ATTN_OK;
}

// The plain path (splits == 0), or the split-KV path with its workspace: the
// caller's (ws, ws_bytes), or with static_ws the library's own array.
int run_fwd(const attn_fwd_args_t& a, int splits = 0, void* ws = nullptr, size_t ws_bytes = 0,
            bool static_ws = false) {
  // --- validation: no HIP call before this block has passed -------------
  const int64_t B = a.B, H = a.H, N = a.N, d = a.d;
  const int64_t Nk = a.Nk == 0 ? N : a.Nk;  // key rows per head (0: as many as queries)
  if (B < 0 || H < 0 || N < 0 || Nk < 0 || d < 0) return ATTN_ERR_SHAPE;
  if (a.dtype != ATTN_DTYPE_F32 && a.dtype != ATTN_DTYPE_F16 && a.dtype != ATTN_DTYPE_BF16)
    return ATTN_ERR_DTYPE;
  if (d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
  if (!isfinite(a.scale)) return ATTN_ERR_SCALE;
  if ((a.flags & ~ATTN_CAUSAL) != 0) return ATTN_ERR_FLAGS;
  if (splits != 0 && (splits < 1 || splits > ATTN_MAX_SPLITS)) return ATTN_ERR_SPLITS;
  if (splits != 0 && (a.flags & ATTN_CAUSAL) != 0) return ATTN_ERR_FLAGS;
  if (Nk != N && (a.flags & ATTN_CAUSAL) != 0) return ATTN_ERR_FLAGS;
  int64_t bh = 0, bhn = 0, elems = 0, kelems = 0;
  if (!mul_ok(B, H, &bh) || !mul_ok(bh, N, &bhn) || !mul_ok(bhn, d, &elems) ||
      !mul_ok(bh, Nk, &kelems) || !mul_ok(kelems, d, &kelems))
    return ATTN_ERR_SHAPE;
  if (bhn == 0) return ATTN_OK;  // empty: nothing to launch
  if (N > ATTN_MAX_N || Nk > ATTN_MAX_N) return ATTN_ERR_SHAPE;
  if (a.q == nullptr || a.k == nullptr || a.v == nullptr || a.o == nullptr)
    return ATTN_ERR_NULLPTR;
  const size_t esize = a.dtype == ATTN_DTYPE_F32 ? 4 : 2;
  if (elems > INT64_MAX / (int64_t)esize || kelems > INT64_MAX / (int64_t)esize)
    return ATTN_ERR_SHAPE;
  int64_t nblocks = 0;  // the largest grid: 128 query rows per block
  if (!mul_ok(bh, (N + 127) / 128, &nblocks) || nblocks > INT32_MAX) return ATTN_ERR_SHAPE;
  if (H > INT32_MAX) return ATTN_ERR_SHAPE;

  // strides: all zero means contiguous [B, H, rows, d]; q and o have N rows
  // per head, k and v Nk
  int64_t st[4][3];
  const int64_t* given[4] = {a.q_stride, a.k_stride, a.v_stride, a.o_stride};
  const int64_t rows[4] = {N, Nk, Nk, N};
  for (int t = 0; t < 4; ++t) {
    const int64_t* g = given[t];
    const int64_t R = rows[t];
    if (g[0] == 0 && g[1] == 0 && g[2] == 0) {
      st[t][0] = H * R * d, st[t][1] = R * d, st[t][2] = d;
    } else {
      for (int i = 0; i < 3; ++i) {
        if (g[i] < 0 || g[i] % 8 != 0 || g[i] > INT64_MAX / 4) return ATTN_ERR_LAYOUT;
        st[t][i] = g[i];
      }
      if (st[t][2] < d) return ATTN_ERR_LAYOUT;  // rows of one head overlap
      // the whole tensor must be addressable: sum of (dim - 1) * stride
      int64_t x = 0, y = 0, z = 0;
      if (!mul_ok(B - 1, st[t][0], &x) || !mul_ok(H - 1, st[t][1], &y) ||
          !mul_ok(R - 1, st[t][2], &z) || x > INT64_MAX / 4 - y - z - d)
        return ATTN_ERR_LAYOUT;
    }
    // the kernels address a head's rows with 32-bit byte offsets
    int64_t head_bytes = 0;
    if (!mul_ok(R, st[t][2], &head_bytes) || !mul_ok(head_bytes, (int64_t)esize, &head_bytes) ||
        head_bytes >= ((int64_t)1 << 31))
      return ATTN_ERR_SHAPE;
  }
  if (!rows_disjoint(st[3], B, H, N, d)) return ATTN_ERR_LAYOUT;

  auto misaligned = [](const void* p, uintptr_t al) {
    return (reinterpret_cast<uintptr_t>(p) & (al - 1)) != 0;
  };
  if (misaligned(a.q, 16) || misaligned(a.k, 16) || misaligned(a.v, 16) ||
      misaligned(a.o, 16) || (a.lse != nullptr && misaligned(a.lse, 4)))
    return ATTN_ERR_ALIGN;
  uintptr_t r[4][2];
  const void* ptrs[4] = {a.q, a.k, a.v, a.o};
  for (int t = 0; t < 4; ++t)
    span_of(ptrs[t], st[t], B, H, rows[t], d, esize, &r[t][0], &r[t][1]);
  for (int t = 0; t < 3; ++t)
    if (ranges_overlap(r[3][0], r[3][1], r[t][0], r[t][1])) return ATTN_ERR_ALIAS;
  if (a.lse != nullptr) {
    const uintptr_t l0 = reinterpret_cast<uintptr_t>(a.lse), l1 = l0 + (size_t)bhn * 4;
    for (int t = 0; t < 4; ++t)
      if (ranges_overlap(l0, l1, r[t][0], r[t][1])) return ATTN_ERR_ALIAS;
  }
  int64_t split_len = 0;
  int nsplit = 1;
  if (splits != 0) {
    split_plan(Nk, splits, &split_len, &nsplit);
    int64_t need = 0;
    if (!mul_ok(bhn, (d + 1) * 4, &need) || !mul_ok(need, nsplit, &need)) return ATTN_ERR_SHAPE;
    if (static_ws) {
      // the size limit is checked before the first HIP call of this path
      if ((uint64_t)need > ATTN_STATIC_WORKSPACE_BYTES) return ATTN_ERR_STATIC_LIMIT;
      const int rc = static_workspace(&ws);
      if (rc != ATTN_OK) return rc;
      ws_bytes = ATTN_STATIC_WORKSPACE_BYTES;
    }
    if (ws == nullptr) return ATTN_ERR_NULLPTR;
    if (misaligned(ws, 16)) return ATTN_ERR_ALIGN;
    if (ws_bytes < (uint64_t)need) return ATTN_ERR_WORKSPACE;
    const uintptr_t w0 = reinterpret_cast<uintptr_t>(ws), w1 = w0 + (size_t)need;
    for (int t = 0; t < 4; ++t)
      if (ranges_overlap(w0, w1, r[t][0], r[t][1])) return ATTN_ERR_ALIAS;
    if (a.lse != nullptr) {
      const uintptr_t l0 = reinterpret_cast<uintptr_t>(a.lse), l1 = l0 + (size_t)bhn * 4;
      if (ranges_overlap(w0, w1, l0, l1)) return ATTN_ERR_ALIAS;
    }
  }

  // --- launch -------------------------------------------------------------
  Launch x;
  x.stream = reinterpret_cast<hipStream_t>(a.stream);
  x.q = a.q, x.k = a.k, x.v = a.v, x.o = a.o, x.lse = a.lse;
  x.bh = bh, x.N = N, x.nk = Nk, x.d = d;
  x.c2 = a.scale * kLog2e;
  x.L.H = (int)H;
  for (int i = 0; i < 3; ++i) {
    x.L.q[i] = st[0][i], x.L.k[i] = st[1][i], x.L.v[i] = st[2][i], x.L.o[i] = st[3][i];
  }
  x.splits = nsplit;
  x.sp.len = (int)split_len;
  x.sp.nk = (int)Nk;
  x.sp.opart = splits ? static_cast<float*>(ws) : nullptr;
  x.sp.lpart = splits ? static_cast<float*>(ws) + (size_t)nsplit * bhn * d : nullptr;
  const bool causal = (a.flags & ATTN_CAUSAL) != 0;
  int rc;
  if (a.dtype == ATTN_DTYPE_BF16)
    rc = causal ? launch16<Bf16T, uint16_t, true>(x) : launch16<Bf16T, uint16_t, false>(x);
  else if (a.dtype == ATTN_DTYPE_F16)
    rc = causal ? launch16<F16T, uint16_t, true>(x) : launch16<F16T, uint16_t, false>(x);
  else
    rc = causal ? launch32<true>(x) : launch32<false>(x);
  if (rc != ATTN_OK || !splits) return rc;
  if (a.dtype == ATTN_DTYPE_BF16) return launch_merge<Out16<Bf16T>, uint16_t>(x);
  if (a.dtype == ATTN_DTYPE_F16) return launch_merge<Out16<F16T>, uint16_t>(x);
  return launch_merge<OutF32, float>(x);
}

}  // namespace

extern "C" int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                        int64_t B, int64_t H, int64_t N, int64_t d, float scale, int dtype,
                        void* stream) {
  attn_fwd_args_t a;
  memset(&a, 0, sizeof(a));
  a.q = q, a.k = k, a.v = v, a.o = o, a.lse = lse;
  a.B = B, a.H = H, a.N = N, a.d = d;
  a.Nk = N;
  a.scale = scale;
  a.dtype = dtype;
  a.stream = stream;
  return run_fwd(a);
}

extern "C" int attn_fwd_ex(const attn_fwd_args_t* args) {
  if (args == nullptr) return ATTN_ERR_NULLPTR;
  return run_fwd(*args);
}

extern "C" size_t attn_fwd_splitkv_workspace_ex(int64_t B, int64_t H, int64_t N, int64_t Nk,
                                                int64_t d, int splits) {
  if (Nk == 0) Nk = N;
  if (B < 0 || H < 0 || N < 0 || Nk < 0 || (d != 64 && d != 128) || splits < 1 ||
      splits > ATTN_MAX_SPLITS)
    return 0;
  int64_t bh = 0, bhn = 0, per = 0;
  if (!mul_ok(B, H, &bh) || !mul_ok(bh, N, &bhn) || !mul_ok(bhn, (d + 1) * 4, &per)) return 0;
  if (bhn == 0) return 0;
  int64_t len = 0;
  int nsplit = 1;
  split_plan(Nk, splits, &len, &nsplit);
  int64_t total = 0;
  if (!mul_ok(per, nsplit, &total)) return 0;
  return (size_t)total;
}

extern "C" size_t attn_fwd_splitkv_workspace(int64_t B, int64_t H, int64_t N, int64_t d,
                                             int splits) {
  return attn_fwd_splitkv_workspace_ex(B, H, N, N, d, splits);
}

extern "C" int attn_fwd_splitkv(const attn_fwd_args_t* args, int splits, void* workspace,
                                size_t workspace_bytes) {
  if (args == nullptr) return ATTN_ERR_NULLPTR;
  if (splits < 1 || splits > ATTN_MAX_SPLITS) return ATTN_ERR_SPLITS;
  return run_fwd(*args, splits, workspace, workspace_bytes);
}

extern "C" int attn_fwd_splitkv_static(const attn_fwd_args_t* args, int splits) {
  if (args == nullptr) return ATTN_ERR_NULLPTR;
  if (splits < 1 || splits > ATTN_MAX_SPLITS) return ATTN_ERR_SPLITS;
  return run_fwd(*args, splits, nullptr, 0, true);
}

extern "C" int attn_fwd_merge(const void* const* o_parts, const float* const* lse_parts,
                              int nparts, void* o, float* lse, int64_t B, int64_t H, int64_t N,
                              int64_t d, int dtype, void* stream) {
  // --- validation: no HIP call before this block has passed -------------
  if (B < 0 || H < 0 || N < 0 || d < 0) return ATTN_ERR_SHAPE;
  if (dtype != ATTN_DTYPE_F32 && dtype != ATTN_DTYPE_F16 && dtype != ATTN_DTYPE_BF16)
    return ATTN_ERR_DTYPE;
  if (d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
  if (nparts < 1 || nparts > ATTN_MAX_SPLITS) return ATTN_ERR_SPLITS;
  int64_t bh = 0, rows = 0, elems = 0;
  if (!mul_ok(B, H, &bh) || !mul_ok(bh, N, &rows) || !mul_ok(rows, d, &elems) ||
      elems > INT64_MAX / 4)
    return ATTN_ERR_SHAPE;
  if (rows == 0) return ATTN_OK;
  if (o_parts == nullptr || lse_parts == nullptr || o == nullptr) return ATTN_ERR_NULLPTR;
  const size_t esize = dtype == ATTN_DTYPE_F32 ? 4 : 2;
  const size_t ob = (size_t)elems * esize, lb = (size_t)rows * 4;
  auto misaligned = [](const void* p, uintptr_t al) {
    return (reinterpret_cast<uintptr_t>(p) & (al - 1)) != 0;
  };
  if (misaligned(o, 16) || (lse != nullptr && misaligned(lse, 4))) return ATTN_ERR_ALIGN;
  MergeParts P;
  for (int s = 0; s < nparts; ++s) {
    if (o_parts[s] == nullptr || lse_parts[s] == nullptr) return ATTN_ERR_NULLPTR;
    if (misaligned(o_parts[s], 16) || misaligned(lse_parts[s], 4)) return ATTN_ERR_ALIGN;
    // outputs must not overlap any input
    if (overlaps(o, ob, o_parts[s], ob) || overlaps(o, ob, lse_parts[s], lb))
      return ATTN_ERR_ALIAS;
    if (lse != nullptr && (overlaps(lse, lb, o_parts[s], ob) || overlaps(lse, lb, lse_parts[s], lb)))
      return ATTN_ERR_ALIAS;
    P.o[s] = o_parts[s];
    P.lse[s] = lse_parts[s];
  }
  if (lse != nullptr && overlaps(o, ob, lse, lb)) return ATTN_ERR_ALIAS;
  for (int s = nparts; s < ATTN_MAX_SPLITS; ++s) P.o[s] = nullptr, P.lse[s] = nullptr;

  // --- launch -------------------------------------------------------------
  const int tpr = (int)d / 4, rpb = kMergeThreads / tpr;
  const int64_t nblocks = (rows + rpb - 1) / rpb;
  if (nblocks > INT32_MAX) return ATTN_ERR_SHAPE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)nblocks), block(kMergeThreads);
  if (dtype == ATTN_DTYPE_BF16) {
    auto k = d == 128 ? attn_merge_parts<Out16<Bf16T>, InBf16, uint16_t, 128>
                      : attn_merge_parts<Out16<Bf16T>, InBf16, uint16_t, 64>;
    hipLaunchKernelGGL(k, grid, block, 0, st, P, nparts, static_cast<uint16_t*>(o), lse,
                       (long long)rows);
  } else if (dtype == ATTN_DTYPE_F16) {
    auto k = d == 128 ? attn_merge_parts<Out16<F16T>, InF16, uint16_t, 128>
                      : attn_merge_parts<Out16<F16T>, InF16, uint16_t, 64>;
    hipLaunchKernelGGL(k, grid, block, 0, st, P, nparts, static_cast<uint16_t*>(o), lse,
                       (long long)rows);
  } else {
    auto k = d == 128 ? attn_merge_parts<OutF32, InF32, float, 128>
                      : attn_merge_parts<OutF32, InF32, float, 64>;
    hipLaunchKernelGGL(k, grid, block, 0, st, P, nparts, static_cast<float*>(o), lse,
                       (long long)rows);
  }
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

extern "C" const char* attn_strerror(int code) {
  switch (code) {
    case ATTN_OK: return "success";
    case ATTN_ERR_NULLPTR: return "q, k, v or o is NULL";
    case ATTN_ERR_SHAPE: return "invalid shape: negative size, overflow, N or Nk > ATTN_MAX_N or grid too large";
    case ATTN_ERR_HEAD_DIM: return "unsupported head dimension (need 64 or 128)";
    case ATTN_ERR_DTYPE: return "unknown dtype";
    case ATTN_ERR_SCALE: return "scale is not finite";
    case ATTN_ERR_ALIGN: return "q/k/v/o must be 16-byte aligned and lse 4-byte aligned";
    case ATTN_ERR_ALIAS: return "an output overlaps an input (or lse overlaps o)";
    case ATTN_ERR_HIP: return "HIP kernel launch failed";
    case ATTN_ERR_FLAGS: return "unknown flag bits, or causal with the split-KV path or with Nk != N";
    case ATTN_ERR_SPLITS: return "split count out of range (1 .. ATTN_MAX_SPLITS)";
    case ATTN_ERR_WORKSPACE: return "workspace smaller than attn_fwd_splitkv_workspace()";
    case ATTN_ERR_LAYOUT: return "invalid strides: negative, not a multiple of 8 elements, or overlapping output rows";
    case ATTN_ERR_STATIC_LIMIT: return "the split-KV partial results exceed the library's static workspace (ATTN_STATIC_WORKSPACE_BYTES)";
    default: return "unknown error code";
  }
}

extern "C" int attn_version(void) { return 210; }
