// attn_common.h - device-side building blocks shared by the attention
// forward and backward kernels for gfx950 (internal to the library; not part
// of its C ABI): vector types, the bf16/fp16 MFMA element traits, cross-lane
// and reduction helpers, the LDS tile geometry and swizzles, and the direct
// global-to-LDS tile loader.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace {

typedef unsigned int u32;
typedef u32 u32x2 __attribute__((ext_vector_type(2)));
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kXcds = 8;      // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr int kThreads = 256; // 4 wave64s per block

// ---------------------------------------------------------------------------
// element traits for the 16-bit paths
// ---------------------------------------------------------------------------
struct Bf16T {
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // Two fp32 -> two bf16, round to nearest even (v_cvt_pk_bf16_f32).
  static __device__ __forceinline__ u32 pack2(float lo, float hi) {
    return __builtin_bit_cast(u32, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
  }
  // acc + the two bf16 values packed in w, in fp32 (v_dot2c_f32_bf16 with 1, 1).
  static __device__ __forceinline__ float sum2(u32 w, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w),
                                           (bf16x2){(__bf16)1.0f, (__bf16)1.0f}, acc, false);
  }
};

struct F16T {
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  // Two fp32 -> two fp16, round to nearest even.
  static __device__ __forceinline__ u32 pack2(float lo, float hi) {
    return __builtin_bit_cast(u32, __builtin_convertvector((f32x2){lo, hi}, f16x2));
  }
  // acc + the two fp16 values packed in w, in fp32 (v_dot2c_f32_f16 with 1, 1).
  static __device__ __forceinline__ float sum2(u32 w, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w),
                                  (f16x2){(_Float16)1.0f, (_Float16)1.0f}, acc, false);
  }
};

// ---------------------------------------------------------------------------
// shared helpers
// ---------------------------------------------------------------------------

// Map the hardware block index to a logical tile so that each XCD (own L2)
// receives one contiguous range of tiles: consecutive tiles are query blocks
// of the same head, which read the same K/V.  Bijective for any count.
__device__ __forceinline__ int xcd_remap(int b, int nb) {
  const int q = nb / kXcds, r = nb % kXcds;
  const int x = b % kXcds, i = b / kXcds;
  return x * q + (x < r ? x : r) + i;
}

// Work item (head bh, tile t) of block b in a grid of nbh heads x nt tiles.
// Equal-length tiles: the xcd_remap order (a head's tiles contiguous on one
// XCD).  Tiles whose length grows or shrinks with t (causal attention):
// level by level over all heads, so that every head's longest tiles start
// before any shorter one (longest-processing-time order keeps the CUs evenly
// loaded to the end of the grid); level 0 is t = 0 and the caller maps it to
// its longest tile.  The hardware deals blocks round-robin over the XCDs, so
// when nbh is a multiple of 8 a head's blocks all land on XCD bh % 8 and
// still share its L2.
struct WorkItem {
  int bh, t;
};
template <bool BY_LEVEL>
__device__ __forceinline__ WorkItem work_item(int b, int nb, int nt) {
  if (BY_LEVEL) {
    const int nbh = nb / nt;
    return {b % nbh, b / nbh};
  }
  const int tile = xcd_remap(b, nb);
  return {tile / nt, tile - (tile / nt) * nt};
}

// Value held by lane l ^ 32, combined with the lane's own by op.
__device__ __forceinline__ float xhalf_max(float x) {
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  float r;
  __asm__("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(__uint_as_float(s[0])), "v"(__uint_as_float(s[1])));
  return r;
}
__device__ __forceinline__ float xhalf_min(float x) {
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  float r;
  __asm__("v_min_f32 %0, %1, %2" : "=v"(r) : "v"(__uint_as_float(s[0])), "v"(__uint_as_float(s[1])));
  return r;
}
__device__ __forceinline__ float xhalf_sum(float x) {
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroup barrier that is also a hard scheduling fence: no instruction
// (MFMA, VALU, LDS read or DMA load) may be moved across it by the compiler.
// The buffer-reuse protocol of the kernels relies on loads staying on their
// side of a barrier, and the ping-pong schedule relies on phases staying in
// their slots.
__device__ __forceinline__ void block_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  __builtin_amdgcn_sched_barrier(0);
}

// v_max3_f32 / v_min3_f32 on values that come straight from MFMA or VALU
// arithmetic (never signalling NaNs), so no canonicalising moves are needed.
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  __asm__("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float min3f(float a, float b, float c) {
  float r;
  __asm__("v_min3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Row extreme over two 16-value fragments (32 values).
__device__ __forceinline__ float frag2_max(const f32x16& s, const f32x16& t) {
  float a = max3f(s[0], s[1], s[2]), b = max3f(s[3], s[4], s[5]);
  float c = max3f(s[6], s[7], s[8]), d = max3f(s[9], s[10], s[11]);
  float e = max3f(s[12], s[13], s[14]), f = max3f(s[15], t[0], t[1]);
  float g = max3f(t[2], t[3], t[4]), h = max3f(t[5], t[6], t[7]);
  float i = max3f(t[8], t[9], t[10]), j = max3f(t[11], t[12], t[13]);
  float k = max3f(a, b, c), m = max3f(d, e, f), n = max3f(g, h, i);
  return max3f(max3f(k, m, n), j, fmaxf(t[14], t[15]));
}
__device__ __forceinline__ float frag2_min(const f32x16& s, const f32x16& t) {
  float a = min3f(s[0], s[1], s[2]), b = min3f(s[3], s[4], s[5]);
  float c = min3f(s[6], s[7], s[8]), d = min3f(s[9], s[10], s[11]);
  float e = min3f(s[12], s[13], s[14]), f = min3f(s[15], t[0], t[1]);
  float g = min3f(t[2], t[3], t[4]), h = min3f(t[5], t[6], t[7]);
  float i = min3f(t[8], t[9], t[10]), j = min3f(t[11], t[12], t[13]);
  float k = min3f(a, b, c), m = min3f(d, e, f), n = min3f(g, h, i);
  return min3f(min3f(k, m, n), j, fminf(t[14], t[15]));
}
__device__ __forceinline__ float frag_max(const f32x16& s) { return frag2_max(s, s); }
__device__ __forceinline__ float frag_min(const f32x16& s) { return frag2_min(s, s); }

// ---------------------------------------------------------------------------
// bf16 / fp16 kernel
// ---------------------------------------------------------------------------
template <int D, int NWAVES = 4>
struct Geo16 {
  static constexpr int BN = 64;                // keys per LDS tile
  static constexpr int ROWB = D * 2;           // bytes per K/V row
  static constexpr int CH = D / 8;             // 16-byte chunks per row
  static constexpr int TILEB = BN * ROWB;      // bytes of one K or V tile
  static constexpr int KS = D / 16;            // k-steps of K*Q^T
  static constexpr int DB = D / 32;            // 32-wide column blocks of O
  static constexpr int LOADB = 64 * 16;        // bytes one wave-wide 16-byte load moves
  static constexpr int ROWS_PER_LOAD = LOADB / ROWB;
  static constexpr int LOADS_PER_WAVE = TILEB / LOADB / NWAVES;
  static_assert(LOADS_PER_WAVE >= 1, "every wave loads at least one block");
};

// LDS swizzles: physical 16-byte chunk = logical chunk ^ f(row).
//  K is read as 16-byte row fragments by 32 lanes of distinct rows: XOR the
//  chunk with the row so that consecutive rows hit distinct banks.
//  V is read by ds_read_b64_tr_b16 as 8 rows x 64 bytes per wave: XOR bits 2-3
//  of the chunk so that the 8 rows spread over the whole bank range.
template <int D> __device__ __forceinline__ int swz_k(int row);
template <> __device__ __forceinline__ int swz_k<128>(int row) { return row & 15; }
template <> __device__ __forceinline__ int swz_k<64>(int row) { return (row & 7) ^ ((row >> 3) & 1); }
template <int D> __device__ __forceinline__ int swz_v(int row);
template <> __device__ __forceinline__ int swz_v<128>(int row) { return (row & 3) << 2; }
template <> __device__ __forceinline__ int swz_v<64>(int row) { return ((row >> 1) & 1) << 2; }

typedef __attribute__((address_space(1))) void gmem_void;
typedef __attribute__((address_space(3))) void lds_void;

// Stream one K tile and one V tile (keys j0 .. j0+63) straight from global
// memory into LDS with 16-byte direct loads (buffer_load_dwordx4 ... lds):
// lane i of a wave-wide load fills bytes [16 i, 16 i + 16) of a 1 KiB LDS
// block, so the swizzle is applied on the source side, by choosing which
// chunk each lane fetches.  Every row of a tile is a contiguous 2*d-byte run
// of K or V, read whole by CH consecutive lanes (coalesced).
//
// With NWAVES issuing waves, load u of issuing wave w fills block
// u * NWAVES + w, i.e. rows u * STEP_ROWS + r0 with r0 = w * ROWS_PER_LOAD +
// lane / CH and STEP_ROWS a multiple of 16.  The swizzle
// bits of those rows do not depend on u, so each lane's byte offset within
// the 16/32-row group is a loop invariant.  Each load gets a buffer
// descriptor whose base is the group's first row and whose size covers only
// rows < N: the hardware range check returns zeros for rows past the end of
// the sequence (their scores are masked, and zero V rows add nothing), so no
// load ever touches memory outside the head.
constexpr int kBufferWord3 = 0x00020000;  // raw buffer, 32-bit data format

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer descriptor: base, stride 0, size in bytes (the range check), word 3.
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, int bytes) {
  const unsigned long long a = reinterpret_cast<unsigned long long>(base);
  return (i32x4){(int)(unsigned)a, (int)((unsigned)(a >> 32) & 0xffffu), bytes, kBufferWord3};
}

typedef __attribute__((address_space(3))) unsigned char lds_u8;

// LDS byte offset of an LDS pointer (a compile-time constant plus offsets
// when the pointer derives from a __shared__ array).
__device__ __forceinline__ uint32_t lds_addr(const lds_u8* p) {
  return (uint32_t)(uintptr_t)(p);
}

// One wave-wide 16-byte-per-lane load into LDS at lds (uniform) + 16 * lane.
// Written as inline asm on purpose: the compiler cannot tell which LDS bytes
// a DMA load writes, and for the builtin it waits for every outstanding load
// before the next LDS read of ANY buffer, which would expose the full load
// latency once per tile.  Here completion is awaited explicitly
// (s_waitcnt vmcnt(0)) before the barrier that publishes a tile, and no
// buffer is read while a load into it is in flight.  M0 holds the LDS base;
// nothing else in these kernels uses M0.
__device__ __forceinline__ void lds_dma16(i32x4 rsrc, uint32_t voff, uint32_t lds) {
  __asm__ volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                   :
                   : "v"(voff), "s"(rsrc), "s"(lds)
                   : "memory");
}

template <int D, int NWAVES>
struct TileLoader {
  using G = Geo16<D, NWAVES>;
  static constexpr int NW = NWAVES;
  static constexpr int STEP_ROWS = NW * G::ROWS_PER_LOAD;  // rows between loads u, u+1
  static_assert(STEP_ROWS % 16 == 0, "swizzle bits must not depend on u");
  uint32_t koff, voff;  // this lane's byte offset from the group's first row
  int krs, vrs;         // bytes between consecutive rows of K and of V in memory
  int wave;             // index of the issuing wave among the NWAVES, uniform

  __device__ __forceinline__ TileLoader(int w, int k_row_bytes, int v_row_bytes)
      : krs(k_row_bytes), vrs(v_row_bytes), wave(w) {
    const int lane = threadIdx.x & 63;
    const int r0 = wave * G::ROWS_PER_LOAD + lane / G::CH;
    const int p = lane % G::CH;
    koff = (uint32_t)(r0 * krs + ((p ^ swz_k<D>(r0)) << 4));
    voff = (uint32_t)(r0 * vrs + ((p ^ swz_v<D>(r0)) << 4));
  }

  // Rows j0 .. j0+63 (j0 < N) of one tensor (K or V, with its lane offset and
  // row stride rs in bytes) -> xb, stored densely (ROWB bytes per row) in LDS.
  // One descriptor per tile, from row j0 to row N; load u adds its rows to
  // the per-lane offset, which is what the hardware range check applies to.
  __device__ __forceinline__ void load(const unsigned char* Xb, uint32_t off, int rs, int j0,
                                       int N, lds_u8* xb) const {
    const i32x4 rsrc = buffer_rsrc(Xb + (size_t)j0 * rs, (N - j0) * rs);  // N*rs < 2^31
#pragma unroll
    for (int u = 0; u < G::LOADS_PER_WAVE; ++u) {
      const int blk = u * NW + wave;
      lds_dma16(rsrc, off + (uint32_t)(u * STEP_ROWS * rs), lds_addr(xb + blk * G::LOADB));
    }
  }
  __device__ __forceinline__ void load_k(const unsigned char* Kb, int j0, int N,
                                         lds_u8* kb) const {
    load(Kb, koff, krs, j0, N, kb);
  }
  __device__ __forceinline__ void load_v(const unsigned char* Vb, int j0, int N,
                                         lds_u8* vb) const {
    load(Vb, voff, vrs, j0, N, vb);
  }
};

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

}  // namespace
