// attn_bwd.hip - attention backward for AMD MI355X (gfx950): dQ, dK, dV of
// O = softmax(scale * Q K^T) V, from the forward's saved O and log-sum-exp.
//
// The gradients are those of the plain definition by the chain rule (the
// backward that page 3 "OpenAI Triton from introduction to model practice",
// section 6, calls from its autograd wrapper, which saves q, k, v, o and lse):
//   P  = exp(s - lse)            s = scale * q.k, recomputed tile by tile
//   dV = P^T dO,  dP = dO V^T,  D = rowsum(dO * O),  dS = P * (dP - D),
//   dQ = scale * dS K,  dK = scale * dS^T Q.
// Like the forward, nothing of size N x N reaches device memory: each block
// recomputes its tiles of s and P from Q, K and the stored lse.
//
// Two kernels (for bf16/fp16; fp32 has its own pair, dq32 and dkdv32, below):
//   * dq:     one block = 128 query rows (4 waves); it first forms per query
//             row the pair (lse log2 e, D = rowsum(dO * O)) and stores it in
//             the workspace for dkdv, then loops over key tiles and
//             accumulates dQ^T = K^T dS^T in registers (the forward's
//             layout: lane l owns query row l % 32 of its wave);
//   * dkdv:   one block = 256 keys (8 waves; 128 keys and 4 waves when that
//             leaves CUs without a block); it loops over query tiles and
//             accumulates dK^T = Q^T dS and dV^T = dO^T P (the transposed
//             layout: lane l owns key l % 32 of its wave).
// Each gradient row is owned by exactly one lane pair, so there are no
// atomics and the results are deterministic.
//
// MFMA shapes and fragments (v_mfma_f32_32x32x16_{bf16,f16}): the A operand
// of lane l holds row l % 32, contraction slots 8 (l / 32) .. +7; B holds
// column l % 32 of the same slots; C holds column l % 32 and rows
// 8 (r / 4) + 4 (l / 32) + r % 4.  Any consistent assignment of contraction
// indices to (half, slot) is valid, so a C fragment in register order is
// directly the B operand of the next product, and the matching A operand is
// read from a row-major LDS tile with the transposing ds_read_b64_tr_b16.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "attn_bwd.h"
#include "attn_common.h"

namespace {

// LDS swizzle of the backward's tiles: physical 16-byte chunk = logical chunk
// ^ swz_b(row).  Each tile is read two ways - as A-operand rows (16-byte
// reads by 16 lanes of 16 consecutive rows) and transposed
// (ds_read_b64_tr_b16: per 32 lanes, 4 consecutive rows x 4 consecutive
// chunks) - and swz_b keeps both free of LDS bank conflicts (64 banks of 4
// bytes): over each aligned group of 16 rows it permutes the chunk positions,
// and the 4 rows of each aligned group of 4 get distinct values in the chunk
// bits above the 4 that a transposed read spans (for d = 64, where two rows
// share the bank range, distinct for rows of the same parity).
template <int D> __device__ __forceinline__ int swz_b(int row);
template <> __device__ __forceinline__ int swz_b<128>(int row) {
  return ((row & 3) << 2) | ((row >> 2) & 3);
}
template <> __device__ __forceinline__ int swz_b<64>(int row) {
  return (((row >> 1) & 1) << 2) ^ ((row >> 2) & 1) ^ (((row >> 3) & 1) << 1);
}

// Per-lane parts of the fragment addresses in a [rows, D] LDS tile whose
// rows are dense (2D bytes) with 16-byte chunks XOR-swizzled by swz_b.
// swz_b depends on row bits 0-3 only, and the loop indices only set
// chunk-index bits that the lane's own chunk bits XOR with, so the read of
// row block r0 (a multiple of 16) at k-step ks (column block db) is at
//   r0 * 2D + (lane offset ^ (ks << 5))      ( ^ (db << 6) )
// with the row block in the instruction's immediate offset: a handful of
// per-lane registers instead of one per distinct read.
template <int D>
struct FragOff {
  static constexpr int ROWB = D * 2;
  uint32_t row;       // A operand rows: row l % 32 of the block, chunk l / 32
  uint32_t tra, trb;  // transposed reads: rows 4 (l / 32) + (l % 16) / 4 and that + 8
  __device__ __forceinline__ FragOff() {
    const int lane = threadIdx.x & 63;
    const int li = lane & 31, hh = lane >> 5, p16 = lane & 15, colhalf = (lane >> 4) & 1;
    row = (uint32_t)(li * ROWB + ((hh ^ swz_b<D>(li)) << 4));
    const int ra = 4 * hh + (p16 >> 2), rb = ra + 8;
    const int c0 = 2 * colhalf + ((p16 & 3) >> 1);  // chunk within column block 0
    const int half8 = (p16 & 1) * 8;
    tra = (uint32_t)(ra * ROWB + ((c0 ^ swz_b<D>(ra)) << 4) + half8);
    trb = (uint32_t)(rb * ROWB + ((c0 ^ swz_b<D>(rb)) << 4) + half8);
  }
};

// One tile of a [N, D] tensor in LDS (layout above).
template <int D>
struct Tile {
  static constexpr int ROWB = D * 2;
  const lds_u8* base;
  // A operand: 8 elements of row r0 + l % 32, contraction slots
  // d = 16 ks + 8 (l / 32) .. +7.
  __device__ __forceinline__ u32x4 row_op(const FragOff<D>& f, int r0, int ks) const {
    return *(const lds_u32x4*)(base + r0 * ROWB + (f.row ^ (uint32_t)(ks << 5)));
  }
  // A operand of a transposed product: column 32 db + l % 32 of rows
  // r0 + 8 (t / 4) + 4 hh + t % 4, t = 0..7 (the C-fragment row order of
  // rows r0 .. r0 + 15 in the lane's half).
  __device__ __forceinline__ u32x4 tr_op(const FragOff<D>& f, int r0, int db) const {
    const lds_u8* a0 = base + r0 * ROWB + (f.tra ^ (uint32_t)(db << 6));
    const lds_u8* a1 = base + r0 * ROWB + (f.trb ^ (uint32_t)(db << 6));
    const u32x2 lo =
        __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(a0)));
    const u32x2 hi =
        __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(a1)));
    return (u32x4){lo[0], lo[1], hi[0], hi[1]};
  }
};

// 8 consecutive elements of row `row` (the B operand of a product with a
// resident row): d = 16 ks + 8 hh .. +7, for ks = 0 .. D/16 - 1.
template <int D>
__device__ __forceinline__ void load_row_frag(const uint16_t* __restrict__ X, int row, int N,
                                              u32x4 (&f)[D / 16]) {
  const int hh = (threadIdx.x & 63) >> 5;
  if (row < N) {
    const u32x4* p = reinterpret_cast<const u32x4*>(X + (size_t)row * D + 8 * hh);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) f[ks] = p[2 * ks];
  } else {
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) f[ks] = (u32x4){0u, 0u, 0u, 0u};
  }
}

// Store of one gradient row owned by the lane (C fragments of X^T in
// register order: columns 32 db + 8 g + 4 hh .. +3), times `mul`, rounded to
// the element type.
template <class E, int D>
__device__ __forceinline__ void store_grad_row(uint16_t* __restrict__ X, int row,
                                               const f32x16 (&acc)[D / 32], float mul) {
  const int hh = (threadIdx.x & 63) >> 5;
  uint16_t* p = X + (size_t)row * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const u32x2 w = (u32x2){E::pack2(acc[db][4 * g + 0] * mul, acc[db][4 * g + 1] * mul),
                              E::pack2(acc[db][4 * g + 2] * mul, acc[db][4 * g + 3] * mul)};
      *reinterpret_cast<u32x2*>(p + 32 * db + 8 * g + 4 * hh) = w;
    }
}

// Pack a 32 x 32 block of fp32 values in C-fragment order (two 16-row halves
// hq) as two B operands, rounding to nearest even.
template <class E>
__device__ __forceinline__ void pack_frag(const f32x16& x, u32x4 (&pb)[2]) {
#pragma unroll
  for (int hq = 0; hq < 2; ++hq) {
    const int b0 = 8 * hq;
    pb[hq] = (u32x4){E::pack2(x[b0 + 0], x[b0 + 1]), E::pack2(x[b0 + 2], x[b0 + 3]),
                     E::pack2(x[b0 + 4], x[b0 + 5]), E::pack2(x[b0 + 6], x[b0 + 7])};
  }
}

constexpr int kBN = 64;  // rows per streamed tile (keys in dq, queries in dkdv)

constexpr int kBM = 128; // rows owned per block (queries in dq, keys in dkdv)

// --- D = rowsum(dO * O) ------------------------------------------------------
// Eight elements (one 16-byte chunk) of a row, widened to fp32 exactly.
template <class E>
struct Widen;
template <>
struct Widen<Bf16T> {
  static __device__ __forceinline__ void get(u32x4 x, float (&f)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(x[i] << 16);
      f[2 * i + 1] = __uint_as_float(x[i] & 0xffff0000u);
    }
  }
};
template <>
struct Widen<F16T> {
  static __device__ __forceinline__ void get(u32x4 x, float (&f)[8]) {
    const f16x8 h = __builtin_bit_cast(f16x8, x);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = (float)h[i];
  }
};

// Loads of ROWS rows of a [N, D] tensor (rows 2D bytes apart in memory) into
// a dense LDS tile in the swz_b layout, by NW waves: 16-byte direct
// global->LDS loads, one buffer descriptor per tile whose range ends at row
// N, so rows past N read as zero.
template <int D, int ROWS, int NW>
struct RowLoader {
  static constexpr int ROWB = 2 * D, CH = D / 8;
  static constexpr int RPL = 1024 / ROWB;     // rows per wave-wide 16-byte load
  static constexpr int STEP = NW * RPL;       // rows between one wave's loads
  static constexpr int LOADS = ROWS / STEP;   // loads per wave and tile
  static_assert(STEP % 16 == 0 && LOADS >= 1 && ROWS % STEP == 0,
                "the swizzle bits must not depend on the load");
  uint32_t off;  // this lane's byte offset from the tile's first row
  int wave;      // index among the NW loading waves (uniform)
  __device__ __forceinline__ explicit RowLoader(int w) : wave(w) {
    const int lane = threadIdx.x & 63;
    const int r0 = wave * RPL + lane / CH, p = lane % CH;
    off = (uint32_t)(r0 * ROWB + ((p ^ swz_b<D>(r0)) << 4));
  }
  // Rows q0 .. q0 + ROWS - 1 (q0 < N).
  __device__ __forceinline__ void load(const unsigned char* Xb, int q0, int N,
                                       lds_u8* dst) const {
    const i32x4 rsrc = buffer_rsrc(Xb + (size_t)q0 * ROWB, (N - q0) * ROWB);
#pragma unroll
    for (int u = 0; u < LOADS; ++u)
      lds_dma16(rsrc, off + (uint32_t)(u * STEP * ROWB),
                lds_addr(dst + (u * NW + wave) * 1024));
  }
};

// --- dQ ------------------------------------------------------------------------
//
// Block: 4 waves, query rows qt*128 + 32 w + (l % 32).  Per 64-key tile (K_j,
// V_j double-buffered in LDS through direct loads):
//   S^T = K Q^T and dP^T = V dO^T  (A from K / V rows, B = resident Q / dO),
//   P = 2^(S c2 - lse log2 e), dS = P (dP - D) per element (lane = query),
//   dQ^T += K^T dS^T               (A from K transposed, B = dS packed).
template <class E, int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void attn_bwd_dq(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                 const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                 const uint16_t* __restrict__ O, const float* __restrict__ LSE,
                 float2* __restrict__ stats, uint16_t* __restrict__ dQ, int N, int nqt,
                 float c2, float scale) {
  using G = Geo16<D, 4>;
  constexpr int TB = G::TILEB, KS = D / 16, DB = D / 32;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[4 * TB];
  lds_u8* const lsm = (lds_u8*)smem;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 31, hh = lane >> 5;

  // causal: the last query tile of a head visits the most key tiles
  WorkItem wi = work_item<CAUSAL>(blockIdx.x, gridDim.x, nqt);
  if (CAUSAL) wi.t = nqt - 1 - wi.t;
  const int bh = wi.bh, qt = wi.t;
  const size_t hoff = (size_t)bh * N * D;
  const unsigned char* Kb = reinterpret_cast<const unsigned char*>(K + hoff);
  const unsigned char* Vb = reinterpret_cast<const unsigned char*>(V + hoff);
  const int q0 = qt * kBM;
  const int T = ((CAUSAL ? min(N, q0 + kBM) : N) + kBN - 1) / kBN;

  const RowLoader<D, kBN, 4> loader(__builtin_amdgcn_readfirstlane(wave));
  auto load = [&](int t, int buf) __attribute__((always_inline)) {
    loader.load(Kb, t * kBN, N, lsm + (2 * buf) * TB);
    loader.load(Vb, t * kBN, N, lsm + (2 * buf + 1) * TB);
  };
  load(0, 0);

  const int qrow = q0 + wave * 32 + li;
  u32x4 qf[KS], df[KS], of[KS];
  load_row_frag<D>(Q + hoff, qrow, N, qf);
  load_row_frag<D>(dO + hoff, qrow, N, df);
  load_row_frag<D>(O + hoff, qrow, N, of);
  const float lse2 = qrow < N ? LSE[(size_t)bh * N + qrow] * kLog2e : INFINITY;
  const int lim = CAUSAL ? min(N - 1, qrow) : N - 1;         // last key this row sees
  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = (f32x16){};
  wait_vmcnt<0>();
  // D = rowsum(dO * O) of the row, from the two lane halves' d ranges (rows
  // past N have zero fragments, D = 0); stored with lse log2 e for the dK/dV
  // kernel, which runs after this one.
  float dpart = 0.f;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    float a[8], b[8];
    Widen<E>::get(of[ks], a);
    Widen<E>::get(df[ks], b);
#pragma unroll
    for (int i = 0; i < 8; ++i) dpart = fmaf(a[i], b[i], dpart);
  }
  const float dl = xhalf_sum(dpart);
  if (hh == 0 && qrow < N) stats[(size_t)bh * N + qrow] = make_float2(lse2, dl);
  // The compiler cannot see the DMA loads (inline asm); using the row
  // fragments here retires their loads in its bookkeeping, so that it places
  // no wait of its own inside the loop, where tile loads are in flight.
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) __asm__ volatile("" ::"v"(qf[ks]), "v"(df[ks]));
  __asm__ volatile("" ::"v"(lse2), "v"(dl));
  __syncthreads();

  FragOff<D> fo;
  // A operand of MFMA i of the S / dP products of half sb: even i the K row
  // fragment of k-step i / 2 (into S), odd i the V row fragment (into dP).
  auto sdp_a = [&](const Tile<D>& kt, const Tile<D>& vt, int sb, int i)
      __attribute__((always_inline)) -> u32x4 {
    return (i & 1) ? vt.row_op(fo, 32 * sb, i >> 1) : kt.row_op(fo, 32 * sb, i >> 1);
  };
  // One element r of dS = P (dP - D), from S and dP.  In a masked tile, key
  // 32 sb + 8 (r / 4) + 4 hh + r % 4 of the tile is visible to the lane's row
  // if 32 sb + 8 (r / 4) + r % 4 <= xlim = lim - j0 - 4 hh (one compare with
  // a constant).
  // The value passes through an empty asm statement, which pins its
  // computation to the step that asks for it (the compiler would otherwise
  // sink it to the packing that consumes it).
  auto ds_elem = [&](int xlim, int sb, int r, bool masked, float sv, float dpv)
      __attribute__((always_inline)) -> float {
    float p = fast_exp2(fmaf(sv, c2, -lse2));
    if (masked && 32 * sb + 8 * (r >> 2) + (r & 3) > xlim) p = 0.f;
    float x = p * (dpv - dl);
    __asm__ volatile("" : "+v"(x));
    return x;
  };
  // One tile.  Its two 32-key halves are staggered so that the softmax
  // arithmetic of one half issues between the MFMAs of the other half's
  // products, in this order (each step a straight run of instructions):
  //   1. S0 = K0 Q^T, dP0 = V0 dO^T                       16 MFMAs (d = 128)
  //   2. S1, dP1, and element i of dS0 after MFMA i        16 MFMAs + dS0
  //   3. dQ^T += K0^T dS0^T, elements 2i, 2i+1 of dS1     8 MFMAs + dS1
  //   4. dQ^T += K1^T dS1^T                                8 MFMAs
  // masked: some keys of the tile lie past a row's limit (tail or diagonal).
  constexpr int NS = 2 * KS;  // MFMAs of S and dP per half
  // Step 1 (needs no mask).
  auto step1 = [&](const Tile<D>& kt, const Tile<D>& vt, f32x16& s0, f32x16& dp0)
      __attribute__((always_inline)) {
    s0 = (f32x16){};
    dp0 = (f32x16){};
    __builtin_amdgcn_s_setprio(2);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (i & 1)
        dp0 = E::mfma(sdp_a(kt, vt, 0, i), df[i >> 1], dp0);
      else
        s0 = E::mfma(sdp_a(kt, vt, 0, i), qf[i >> 1], s0);
    }
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
  };
  // Steps 2-4.
  auto steps234 = [&](const Tile<D>& kt, const Tile<D>& vt, int j0, bool masked, f32x16& s0,
                      const f32x16& dp0) __attribute__((always_inline)) {
    f32x16 s1 = (f32x16){}, dp1 = (f32x16){};
    int xlim = lim - j0 - 4 * hh;
    __asm__ volatile("" : "+v"(xlim));  // kept whole: no per-element offsets hoisted
    // 2.  The operand of MFMA i + 2 is read before MFMA i issues; dS
    // replaces S in place.
    u32x4 a[NS];
    a[0] = sdp_a(kt, vt, 1, 0);
    a[1] = sdp_a(kt, vt, 1, 1);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (i + 2 < NS) a[i + 2] = sdp_a(kt, vt, 1, i + 2);
      if (i & 1)
        dp1 = E::mfma(a[i], df[i >> 1], dp1);
      else
        s1 = E::mfma(a[i], qf[i >> 1], s1);
#pragma unroll
      for (int r = i * 16 / NS; r < (i + 1) * 16 / NS; ++r)
        s0[r] = ds_elem(xlim, 0, r, masked, s0[r], dp0[r]);
      __builtin_amdgcn_sched_barrier(0);
    }
    u32x4 pb0[2], pb1[2];
    pack_frag<E>(s0, pb0);
    __builtin_amdgcn_sched_barrier(0);
    // 3.
    constexpr int NQ = 2 * DB;  // MFMAs of dQ per half
    u32x4 b[NQ];
    b[0] = kt.tr_op(fo, 0, 0);
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int db = i >> 1, hq = i & 1;
      if (i + 1 < NQ) b[i + 1] = kt.tr_op(fo, 16 * ((i + 1) & 1), (i + 1) >> 1);
      acc[db] = E::mfma(b[i], pb0[hq], acc[db]);
#pragma unroll
      for (int r = i * 16 / NQ; r < (i + 1) * 16 / NQ; ++r)
        s1[r] = ds_elem(xlim, 1, r, masked, s1[r], dp1[r]);
      __builtin_amdgcn_sched_barrier(0);
    }
    pack_frag<E>(s1, pb1);
    __builtin_amdgcn_sched_barrier(0);
    // 4.
    __builtin_amdgcn_s_setprio(2);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int hq = 0; hq < 2; ++hq)
        acc[db] = E::mfma(kt.tr_op(fo, 32 + 16 * hq, db), pb1[hq], acc[db]);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto run_tile = [&](int t, bool masked) __attribute__((always_inline)) {
    const int buf = t & 1;
    if (t + 1 < T) load(t + 1, buf ^ 1);
    const Tile<D> kt{lsm + (2 * buf) * TB}, vt{lsm + (2 * buf + 1) * TB};
    // Fresh copies of the lane offsets each tile, so that the per-fragment
    // XORs are formed where they are used instead of being hoisted out of
    // the loop into a register each.
    __asm__ volatile("" : "+v"(fo.row), "+v"(fo.tra), "+v"(fo.trb));
    f32x16 s0, dp0;
    step1(kt, vt, s0, dp0);
    steps234(kt, vt, t * kBN, masked, s0, dp0);
    wait_vmcnt<0>();
    __syncthreads();
  };
  // Tiles below TF are visible in full to every row of the block; the rest
  // (the sequence tail, the causal diagonal) take the mask.
  const int TF = min(T, ((CAUSAL ? min(N - 1, q0) : N - 1) + 1) / kBN);
  int t = 0;
  for (; t < TF; ++t) run_tile(t, false);
  for (; t < T; ++t) run_tile(t, true);
  if (qrow < N) store_grad_row<E, D>(dQ + hoff, qrow, acc, scale);
}

// --- dK, dV ------------------------------------------------------------------
//
// Block: KW = 8 waves (4 on grids too small to give every CU a block of 8),
// keys kt*32KW + 32 w + (l % 32).  K rows stay in registers
// (the B operand of S); the block's V rows are staged once in LDS and read
// back as the B operand of dP, which keeps a wave at no more than 256 VGPRs
// (two waves per SIMD, one block per CU): the resident state is K (D/4
// VGPRs) and the fp32 dK, dV accumulators (D/2 each).  Per 64-query tile
// (Q_i, dO_i double-buffered in LDS, with lse and D of those queries):
//   S = Q K^T and dP = dO V^T      (A from Q / dO rows),
//   P = 2^(S c2 - lse log2 e), dS = P (dP - D) per element (lane = key),
//   dV^T += dO^T P, dK^T += Q^T dS (A from dO / Q transposed, B = P / dS).
constexpr int kKW = 8;             // waves of a dK/dV block (4 on small grids)

template <class E, int D, bool CAUSAL, int KW = kKW>
__global__ __launch_bounds__(64 * KW) __attribute__((amdgpu_waves_per_eu(2)))
void attn_bwd_dkdv(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                   const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                   const float2* __restrict__ stats,
                   uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int N, int nkt,
                   float c2, float scale) {
  constexpr int kBK = 32 * KW;  // keys per block
  using G = Geo16<D, KW>;
  constexpr int TB = G::TILEB, KS = D / 16, DB = D / 32;
  constexpr int VT = kBK / kBN;  // V tiles of the block
  // two buffers of (Q tile, dO tile), the block's V rows, then two buffers
  // of (lse * log2 e, D)
  __shared__ __attribute__((aligned(1024))) unsigned char smem[(4 + VT) * TB + 2 * 2 * kBN * 4];
  lds_u8* const lsm = (lds_u8*)smem;
  float* const stat = reinterpret_cast<float*>(smem + (4 + VT) * TB);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 31, hh = lane >> 5;

  // causal: the first key tile of a head is seen by the most query tiles
  const WorkItem wi = work_item<CAUSAL>(blockIdx.x, gridDim.x, nkt);
  const int bh = wi.bh, kt = wi.t;
  const size_t hoff = (size_t)bh * N * D;
  const unsigned char* Qb = reinterpret_cast<const unsigned char*>(Q + hoff);
  const unsigned char* dOb = reinterpret_cast<const unsigned char*>(dO + hoff);
  const int k0 = kt * kBK;
  // causal: queries before the block's first key see none of its keys
  const int t0 = CAUSAL ? k0 / kBN : 0;
  const int T = (N + kBN - 1) / kBN;

  const RowLoader<D, kBN, KW> loader(__builtin_amdgcn_readfirstlane(wave));
  auto load = [&](int t, int buf) __attribute__((always_inline)) {
    loader.load(Qb, t * kBN, N, lsm + (2 * buf) * TB);
    loader.load(dOb, t * kBN, N, lsm + (2 * buf + 1) * TB);
  };
  // The block's V rows (tiles past N are left unwritten: they only feed
  // the gradients of keys past N, which are not stored).
  const Tile<D> vt{lsm + 4 * TB};
  {
    const unsigned char* Vb = reinterpret_cast<const unsigned char*>(V + hoff);
#pragma unroll
    for (int u = 0; u < VT; ++u)
      if (k0 + u * kBN < N) loader.load(Vb, k0 + u * kBN, N, lsm + (4 + u) * TB);
  }
  // lse (log2 domain; +inf past N, so P = 0) and D of the tile's queries:
  // thread i < 128 fetches one value into a register early in an iteration
  // and stores it to LDS at its end, once the iteration's compute is issued.
  // Whether a thread fetches lse (wave 0) or D (wave 1) is wave-uniform
  // (kBN = 64 threads each), and so is its out-of-range default: both are
  // formed in scalars, so that the default takes no vector register across
  // the key loop (at d = 128 every vector register is taken, and a per-lane
  // default was spilled to scratch and reloaded in every iteration).
  const int swave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const float sdefault = swave == 0 ? INFINITY : 0.f;
  static_assert(kBN == 64, "one wave per statistic");
  const int slane = (int)(threadIdx.x & (kBN - 1));
  // past the end the lane reads the last row (in bounds); the value is
  // replaced by the default when it is stored, after it has arrived
  auto fetch_stat = [&](int t) __attribute__((always_inline)) -> float {
    if (swave >= 2) return sdefault;
    const int q = min(t * kBN + slane, N - 1);
    return reinterpret_cast<const float*>(stats)[2 * ((size_t)bh * N + q) + swave];
  };
  auto store_stat = [&](float x, int t, int buf) __attribute__((always_inline)) {
    if (threadIdx.x < 2 * kBN)
      stat[buf * 2 * kBN + threadIdx.x] = t * kBN + slane < N ? x : sdefault;
  };
  load(t0, 0);
  store_stat(fetch_stat(t0), t0, 0);

  const int key = k0 + wave * 32 + li;
  u32x4 kf[KS];
  load_row_frag<D>(K + hoff, key, N, kf);
  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dk[db] = (f32x16){};
    dv[db] = (f32x16){};
  }
  // causal: tiles starting before the wave's last key hold queries that some
  // of its keys do not see (queries past N have lse = +inf, hence P = 0)
  const int kmax = k0 + wave * 32 + 31;
  wait_vmcnt<0>();
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) __asm__ volatile("" ::"v"(kf[ks]));
  __syncthreads();

  const FragOff<D> fo;
  for (int t = t0; t < T; ++t) {
    const int buf = (t - t0) & 1;
    const bool more = t + 1 < T;
    float nxt = 0.f;
    if (more) {
      nxt = fetch_stat(t + 1);
      load(t + 1, buf ^ 1);
    }
    const Tile<D> qt_{lsm + (2 * buf) * TB}, dot{lsm + (2 * buf + 1) * TB};
    const float* st = stat + buf * 2 * kBN;
    const int i0 = t * kBN;
    const bool partial = CAUSAL && i0 < kmax;
    // one 32-query half of the tile at a time (fewer live registers)
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      f32x16 s = (f32x16){}, dp = (f32x16){};
      __builtin_amdgcn_s_setprio(2);  // MFMA section (see attn_bwd_dq)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s = E::mfma(qt_.row_op(fo, 32 * sb, ks), kf[ks], s);
        dp = E::mfma(dot.row_op(fo, 32 * sb, ks), vt.row_op(fo, 32 * wave, ks), dp);
      }
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
      // P and dS in place of S and dP
      // the lane's offset into the statistics, formed again each half from
      // the thread index rather than kept live (or spilled) across the loop
      int hh4 = (int)(threadIdx.x >> 3) & 4;
      __asm__ volatile("" : "+v"(hh4));
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // queries 32 sb + 8 g + 4 hh .. +3 of the tile: their lse and D
        const int qi = 32 * sb + 8 * g + hh4;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(st + qi);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(st + kBN + qi);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          float pv = fast_exp2(fmaf(s[r], c2, -l4[e]));
          if (partial && key > i0 + qi + e) pv = 0.f;
          s[r] = pv;
          dp[r] = pv * (dp[r] - d4[e]);
        }
      }
      u32x4 pb[2], dsb[2];
      pack_frag<E>(s, pb);
      pack_frag<E>(dp, dsb);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(2);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int hq = 0; hq < 2; ++hq) {
          dv[db] = E::mfma(dot.tr_op(fo, 32 * sb + 16 * hq, db), pb[hq], dv[db]);
          dk[db] = E::mfma(qt_.tr_op(fo, 32 * sb + 16 * hq, db), dsb[hq], dk[db]);
        }
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
    }
    if (more) store_stat(nxt, t + 1, buf ^ 1);
    wait_vmcnt<0>();
    __syncthreads();
  }
  if (key < N) {
    store_grad_row<E, D>(dK + hoff, key, dk, scale);
    store_grad_row<E, D>(dV + hoff, key, dv, 1.0f);
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
namespace {

bool mul_ok_b(int64_t a, int64_t b, int64_t* out) {
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

// ---------------------------------------------------------------------------
// fp32 backward
// ---------------------------------------------------------------------------
//
// The same two passes for fp32 inputs, on the VALU with LDS tiles (fp32 has no
// rounding of P or dS to mirror, and no faster matrix path: the fp32 MFMA
// peak equals the packed fp32 VALU peak).  Tiles of 32 rows; a block of 256
// threads.  In dq32 thread t owns query row i = t / 8 of the block and, for
// the 32x32 tiles of S and dP, the keys j = t % 8 + 8u (u < 4); for dQ the
// columns 4 (t % 8 + 8w) .. +3 (w < D / 32).  dkdv32 is the same with keys and
// queries exchanged.  Strided row and column assignments keep the threads of
// a wave on distinct LDS banks; rows are padded by 4 floats for the same
// reason.
constexpr int kT32 = 32;  // rows per tile in the fp32 backward

template <int D>
struct Tile32 {
  static constexpr int LD = D + 4;  // padded row of an LDS tile, in floats
};

// Rows r0 .. r0 + 31 of a [rows, D] fp32 tensor (rows >= n read as zero) into
// an LDS tile, 16 bytes per thread and step.
template <int D>
__device__ __forceinline__ void load_tile32(float* __restrict__ dst, const float* __restrict__ src,
                                            int r0, int n) {
  constexpr int C4 = D / 4;
  for (int e = threadIdx.x; e < kT32 * C4; e += 256) {
    const int r = e / C4, c = (e - r * C4) * 4;
    f32x4 x = (f32x4){0.f, 0.f, 0.f, 0.f};
    if (r0 + r < n) x = *reinterpret_cast<const f32x4*>(src + (size_t)(r0 + r) * D + c);
    *reinterpret_cast<f32x4*>(dst + r * Tile32<D>::LD + c) = x;
  }
}

// Four dot products of LDS row a with LDS rows b + 8u * LD (u < 4), over D.
template <int D>
__device__ __forceinline__ void dot4x(const float* a, const float* b, float (&s)[4]) {
  constexpr int LD = Tile32<D>::LD;
#pragma unroll
  for (int u = 0; u < 4; ++u) s[u] = 0.f;
#pragma unroll 4
  for (int c = 0; c < D; c += 4) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(a + c);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const f32x4 y = *reinterpret_cast<const f32x4*>(b + 8 * u * LD + c);
      s[u] = fmaf(x[0], y[0], s[u]);
      s[u] = fmaf(x[1], y[1], s[u]);
      s[u] = fmaf(x[2], y[2], s[u]);
      s[u] = fmaf(x[3], y[3], s[u]);
    }
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void attn_bwd_dq32(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ dO, const float* __restrict__ O, const float* __restrict__ LSE,
    float2* __restrict__ stats, float* __restrict__ dQ, int N, int nqt, float c2, float scale) {
  constexpr int LD = Tile32<D>::LD, W = D / 32;
  __shared__ __attribute__((aligned(16))) float qs[kT32 * LD], gs[kT32 * LD];
  __shared__ __attribute__((aligned(16))) float ks[kT32 * LD], vs[kT32 * LD];
  __shared__ float ds[kT32][kT32 + 1];
  __shared__ float2 st[kT32];
  const int bh = blockIdx.x / nqt, q0 = (blockIdx.x - bh * nqt) * kT32;
  const size_t base = (size_t)bh * N * D;
  const int t = threadIdx.x, i = t >> 3, jg = t & 7;
  load_tile32<D>(qs, Q + base, q0, N);
  load_tile32<D>(gs, dO + base, q0, N);
  // per query row: (lse log2 e, D = sum_c dO O), 8 threads per row
  {
    float dd = 0.f;
    if (q0 + i < N) {
      const float* orow = O + base + (size_t)(q0 + i) * D;
      const float* grow = dO + base + (size_t)(q0 + i) * D;
      for (int c = jg * 4; c < D; c += 32) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(orow + c);
        const f32x4 b = *reinterpret_cast<const f32x4*>(grow + c);
        dd = fmaf(a[0], b[0], fmaf(a[1], b[1], fmaf(a[2], b[2], fmaf(a[3], b[3], dd))));
      }
    }
    dd += __shfl_xor(dd, 1);
    dd += __shfl_xor(dd, 2);
    dd += __shfl_xor(dd, 4);
    if (jg == 0) {
      const float2 x = q0 + i < N ? make_float2(LSE[(size_t)bh * N + q0 + i] * kLog2e, dd)
                                  : make_float2(INFINITY, 0.f);
      st[i] = x;
      if (q0 + i < N) stats[(size_t)bh * N + q0 + i] = x;
    }
  }
  float acc[W][4];
#pragma unroll
  for (int w = 0; w < W; ++w)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[w][e] = 0.f;
  const int kend = CAUSAL ? min(N, q0 + kT32) : N;
  for (int j0 = 0; j0 < kend; j0 += kT32) {
    __syncthreads();  // previous tile's K, V and dS fully read
    load_tile32<D>(ks, K + base, j0, N);
    load_tile32<D>(vs, V + base, j0, N);
    __syncthreads();
    float s[4], dp[4];
    dot4x<D>(qs + i * LD, ks + jg * LD, s);
    dot4x<D>(gs + i * LD, vs + jg * LD, dp);
    const float2 x = st[i];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = j0 + jg + 8 * u;
      const bool live = j < N && q0 + i < N && (!CAUSAL || j <= q0 + i);
      const float p = live ? fast_exp2(s[u] * c2 - x.x) : 0.f;
      ds[i][jg + 8 * u] = p * (dp[u] - x.y);
    }
    __syncthreads();
    for (int j = 0; j < kT32; ++j) {
      const float dsv = ds[i][j];
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const f32x4 kv = *reinterpret_cast<const f32x4*>(ks + j * LD + 4 * (jg + 8 * w));
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[w][e] = fmaf(dsv, kv[e], acc[w][e]);
      }
    }
  }
  if (q0 + i < N) {
    float* const out = dQ + base + (size_t)(q0 + i) * D;
#pragma unroll
    for (int w = 0; w < W; ++w)
      *reinterpret_cast<f32x4*>(out + 4 * (jg + 8 * w)) =
          (f32x4){acc[w][0] * scale, acc[w][1] * scale, acc[w][2] * scale, acc[w][3] * scale};
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void attn_bwd_dkdv32(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ dO, const float2* __restrict__ stats, float* __restrict__ dK,
    float* __restrict__ dV, int N, int nkt, float c2, float scale) {
  constexpr int LD = Tile32<D>::LD, W = D / 32;
  __shared__ __attribute__((aligned(16))) float ks[kT32 * LD], vs[kT32 * LD];
  __shared__ __attribute__((aligned(16))) float qs[kT32 * LD], gs[kT32 * LD];
  __shared__ float ps[kT32][kT32 + 1], ds[kT32][kT32 + 1];
  __shared__ float2 st[kT32];
  const int bh = blockIdx.x / nkt, k0 = (blockIdx.x - bh * nkt) * kT32;
  const size_t base = (size_t)bh * N * D;
  const int t = threadIdx.x, j = t >> 3, ig = t & 7;  // key j of the block
  load_tile32<D>(ks, K + base, k0, N);
  load_tile32<D>(vs, V + base, k0, N);
  float dk[W][4], dv[W][4];
#pragma unroll
  for (int w = 0; w < W; ++w)
#pragma unroll
    for (int e = 0; e < 4; ++e) dk[w][e] = dv[w][e] = 0.f;
  // causal: query rows before k0 see none of these keys
  for (int i0 = CAUSAL ? k0 : 0; i0 < N; i0 += kT32) {
    __syncthreads();  // previous tile's Q, dO, P and dS fully read
    load_tile32<D>(qs, Q + base, i0, N);
    load_tile32<D>(gs, dO + base, i0, N);
    if (t < kT32) st[t] = i0 + t < N ? stats[(size_t)bh * N + i0 + t] : make_float2(INFINITY, 0.f);
    __syncthreads();
    float s[4], dp[4];
    dot4x<D>(ks + j * LD, qs + ig * LD, s);   // s[u] = S[query ig + 8u][key j]
    dot4x<D>(vs + j * LD, gs + ig * LD, dp);  // dP likewise
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int qi = ig + 8 * u;
      const float2 x = st[qi];
      const bool live = i0 + qi < N && k0 + j < N && (!CAUSAL || k0 + j <= i0 + qi);
      const float p = live ? fast_exp2(s[u] * c2 - x.x) : 0.f;
      ps[qi][j] = p;
      ds[qi][j] = p * (dp[u] - x.y);
    }
    __syncthreads();
    for (int qi = 0; qi < kT32; ++qi) {
      const float p = ps[qi][j], d = ds[qi][j];
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const f32x4 g = *reinterpret_cast<const f32x4*>(gs + qi * LD + 4 * (ig + 8 * w));
        const f32x4 q = *reinterpret_cast<const f32x4*>(qs + qi * LD + 4 * (ig + 8 * w));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dv[w][e] = fmaf(p, g[e], dv[w][e]);
          dk[w][e] = fmaf(d, q[e], dk[w][e]);
        }
      }
    }
  }
  if (k0 + j < N) {
    float* const ok = dK + base + (size_t)(k0 + j) * D;
    float* const ov = dV + base + (size_t)(k0 + j) * D;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      *reinterpret_cast<f32x4*>(ok + 4 * (ig + 8 * w)) =
          (f32x4){dk[w][0] * scale, dk[w][1] * scale, dk[w][2] * scale, dk[w][3] * scale};
      *reinterpret_cast<f32x4*>(ov + 4 * (ig + 8 * w)) =
          (f32x4){dv[w][0], dv[w][1], dv[w][2], dv[w][3]};
    }
  }
}

bool overlap_b(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return na > 0 && nb > 0 && x < y + nb && y < x + na;
}

template <class E, int D, bool C>
int launch_bwd(const attn_bwd_args_t& a, float2* stats, int64_t bh) {
  hipStream_t s = reinterpret_cast<hipStream_t>(a.stream);
  const float c2 = a.scale * kLog2e;
  const int64_t nt = (a.N + kBM - 1) / kBM;
  const uint16_t *q = static_cast<const uint16_t*>(a.q), *k = static_cast<const uint16_t*>(a.k),
                 *v = static_cast<const uint16_t*>(a.v),
                 *dout = static_cast<const uint16_t*>(a.dout);
  hipLaunchKernelGGL((attn_bwd_dq<E, D, C>), dim3((unsigned)(bh * nt)), dim3(256), 0, s, q, k, v,
                     dout, static_cast<const uint16_t*>(a.o), a.lse, stats,
                     static_cast<uint16_t*>(a.dq), (int)a.N, (int)nt, c2, a.scale);
  if (hipGetLastError() != hipSuccess) return ATTN_ERR_HIP;
  // dK, dV: blocks of 8 waves (256 keys) when that gives every CU a block,
  // else of 4 waves (128 keys), twice the blocks
  const int64_t nkt8 = (a.N + 32 * kKW - 1) / (32 * kKW);
  if (bh * nkt8 >= 256) {
    hipLaunchKernelGGL((attn_bwd_dkdv<E, D, C, kKW>), dim3((unsigned)(bh * nkt8)),
                       dim3(64 * kKW), 0, s, q, k, v, dout, stats,
                       static_cast<uint16_t*>(a.dk), static_cast<uint16_t*>(a.dv), (int)a.N,
                       (int)nkt8, c2, a.scale);
  } else {
    const int64_t nkt4 = (a.N + 127) / 128;
    hipLaunchKernelGGL((attn_bwd_dkdv<E, D, C, 4>), dim3((unsigned)(bh * nkt4)), dim3(256), 0,
                       s, q, k, v, dout, stats, static_cast<uint16_t*>(a.dk),
                       static_cast<uint16_t*>(a.dv), (int)a.N, (int)nkt4, c2, a.scale);
  }
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

template <class E>
int launch_bwd_e(const attn_bwd_args_t& a, float2* stats, int64_t bh) {
  const bool c = (a.flags & ATTN_CAUSAL) != 0;
  if (a.d == 128) return c ? launch_bwd<E, 128, true>(a, stats, bh)
                           : launch_bwd<E, 128, false>(a, stats, bh);
  return c ? launch_bwd<E, 64, true>(a, stats, bh) : launch_bwd<E, 64, false>(a, stats, bh);
}

template <int D, bool C>
int launch_bwd32(const attn_bwd_args_t& a, float2* stats, int64_t bh) {
  hipStream_t s = reinterpret_cast<hipStream_t>(a.stream);
  const float c2 = a.scale * kLog2e;
  const int64_t nt = (a.N + kT32 - 1) / kT32;
  const float *q = static_cast<const float*>(a.q), *k = static_cast<const float*>(a.k),
              *v = static_cast<const float*>(a.v), *dout = static_cast<const float*>(a.dout);
  hipLaunchKernelGGL((attn_bwd_dq32<D, C>), dim3((unsigned)(bh * nt)), dim3(256), 0, s, q, k, v,
                     dout, static_cast<const float*>(a.o), a.lse, stats,
                     static_cast<float*>(a.dq), (int)a.N, (int)nt, c2, a.scale);
  if (hipGetLastError() != hipSuccess) return ATTN_ERR_HIP;
  hipLaunchKernelGGL((attn_bwd_dkdv32<D, C>), dim3((unsigned)(bh * nt)), dim3(256), 0, s, q, k,
                     v, dout, stats, static_cast<float*>(a.dk), static_cast<float*>(a.dv),
                     (int)a.N, (int)nt, c2, a.scale);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int launch_bwd_f32(const attn_bwd_args_t& a, float2* stats, int64_t bh) {
  const bool c = (a.flags & ATTN_CAUSAL) != 0;
  if (a.d == 128) return c ? launch_bwd32<128, true>(a, stats, bh)
                           : launch_bwd32<128, false>(a, stats, bh);
  return c ? launch_bwd32<64, true>(a, stats, bh) : launch_bwd32<64, false>(a, stats, bh);
}

}  // namespace

extern "C" size_t attn_bwd_workspace(int64_t B, int64_t H, int64_t N, int64_t d) {
  if (B < 0 || H < 0 || N < 0 || (d != 64 && d != 128)) return 0;
  int64_t bh = 0, bhn = 0;
  if (!mul_ok_b(B, H, &bh) || !mul_ok_b(bh, N, &bhn) || bhn > INT64_MAX / 8) return 0;
  return (size_t)bhn * 8;
}

extern "C" int attn_bwd(const attn_bwd_args_t* args, void* ws, size_t ws_bytes) {
  // --- validation: no HIP call before this block has passed -------------
  if (args == nullptr) return ATTN_ERR_NULLPTR;
  const attn_bwd_args_t& a = *args;
  const int64_t B = a.B, H = a.H, N = a.N, d = a.d;
  if (B < 0 || H < 0 || N < 0 || d < 0) return ATTN_ERR_SHAPE;
  if (a.dtype != ATTN_DTYPE_F16 && a.dtype != ATTN_DTYPE_BF16 && a.dtype != ATTN_DTYPE_F32)
    return ATTN_ERR_DTYPE;
  if (d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
  if (!isfinite(a.scale)) return ATTN_ERR_SCALE;
  if ((a.flags & ~ATTN_CAUSAL) != 0) return ATTN_ERR_FLAGS;
  const int64_t esize = a.dtype == ATTN_DTYPE_F32 ? 4 : 2;
  int64_t bh = 0, bhn = 0, elems = 0;
  if (!mul_ok_b(B, H, &bh) || !mul_ok_b(bh, N, &bhn) || !mul_ok_b(bhn, d, &elems) ||
      elems > INT64_MAX / esize)
    return ATTN_ERR_SHAPE;
  if (bhn == 0) return ATTN_OK;
  if (N > ATTN_MAX_N || N * d * esize >= ((int64_t)1 << 31)) return ATTN_ERR_SHAPE;
  // the largest grid: 32-row tiles (fp32), 128-row blocks otherwise
  if (bh * ((N + kT32 - 1) / kT32) > INT32_MAX || bhn > INT32_MAX) return ATTN_ERR_SHAPE;
  const void* ptrs[9] = {a.q, a.k, a.v, a.o, a.dout, a.lse, a.dq, a.dk, a.dv};
  for (const void* p : ptrs)
    if (p == nullptr) return ATTN_ERR_NULLPTR;
  if (ws == nullptr) return ATTN_ERR_NULLPTR;
  for (int i = 0; i < 9; ++i)
    if ((reinterpret_cast<uintptr_t>(ptrs[i]) & (i == 5 ? 3u : 15u)) != 0) return ATTN_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(ws) & 15u) != 0) return ATTN_ERR_ALIGN;
  const size_t tb = (size_t)elems * esize, lb = (size_t)bhn * 4, wb = (size_t)bhn * 8;
  if (ws_bytes < wb) return ATTN_ERR_WORKSPACE;
  const size_t sizes[9] = {tb, tb, tb, tb, tb, lb, tb, tb, tb};
  // outputs (dq, dk, dv) and the workspace must not overlap anything else
  for (int i = 6; i < 9; ++i)
    for (int j = 0; j < 9; ++j)
      if (j != i && overlap_b(ptrs[i], sizes[i], ptrs[j], sizes[j])) return ATTN_ERR_ALIAS;
  for (int j = 0; j < 9; ++j)
    if (overlap_b(ws, wb, ptrs[j], sizes[j])) return ATTN_ERR_ALIAS;

  // --- launch -------------------------------------------------------------
  float2* stats = static_cast<float2*>(ws);
  if (a.dtype == ATTN_DTYPE_BF16) return launch_bwd_e<Bf16T>(a, stats, bh);
  if (a.dtype == ATTN_DTYPE_F16) return launch_bwd_e<F16T>(a, stats, bh);
  return launch_bwd_f32(a, stats, bh);
}
