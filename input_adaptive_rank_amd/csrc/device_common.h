// Device-side building blocks for the gfx950 DyRA kernels: bf16 conversion,
// MFMA wrappers, the swizzled LDS tile layout, and the XCD-aware tile order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef double f64x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf2f(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16, round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

// Token segments of a forward: uniform runs of `seg` rows when off is null,
// else rows [off[b], off[b + 1]) of a device offsets array (off[0] = 0,
// off[B] = n, every segment at least one row).  Passed by value.
struct SegMap {
  const int32_t* off;
  int64_t seg, B, n;
  // The offsets are read through the constant address space: with a
  // wave-uniform index that is a scalar load, counted by lgkmcnt, so a wave
  // that looks up a segment never waits for its own outstanding vector
  // stores (vmcnt); they are never written while a kernel runs.
  __device__ __forceinline__ int64_t at(int64_t i) const {
    return (int64_t)reinterpret_cast<const __attribute__((address_space(4))) int32_t*>(
        reinterpret_cast<uintptr_t>(off))[i];
  }
  __device__ __forceinline__ int64_t lo(int64_t b) const { return off ? at(b) : b * seg; }
  __device__ __forceinline__ int64_t hi(int64_t b) const {
    return off ? at(b + 1) : ((b + 1) * seg < n ? (b + 1) * seg : n);
  }
  // the segment holding `row` (0 <= row < n)
  __device__ __forceinline__ int64_t of(int64_t row) const {
    if (!off) return row / seg;
    int64_t a = 0, z = B;   // off[a] <= row < off[z]
    while (z - a > 1) {
      const int64_t mid = (a + z) >> 1;
      if (at(mid) <= row) a = mid;
      else z = mid;
    }
    return a;
  }
};

// Element traits.  A 16-byte chunk holds KPC elements; one "k-substep" of the
// MMA covers two chunks (lanes 0-31 read chunk 2s, lanes 32-63 chunk 2s+1).
template <typename T> struct TT;

template <> struct TT<bf16_t> {
  static constexpr int KPC = 8;
  static constexpr int ESZ = 2;
  // 32x32 block += (lane rows of a) x (lane rows of b)^T over 16 k values.
  __device__ static __forceinline__ void mma(f32x16& acc, const uint4& a, const uint4& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
  }
  __device__ static __forceinline__ float to_f(bf16_t v) { return bf2f(v); }
  __device__ static __forceinline__ bf16_t from_f(float v) { return f2bf(v); }
};

template <> struct TT<float> {
  static constexpr int KPC = 4;
  static constexpr int ESZ = 4;
  // four 32x32x2 fp32 MFMAs, element e of each lane's chunk in the e-th one.
  __device__ static __forceinline__ void mma(f32x16& acc, const uint4& a, const uint4& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
  }
  __device__ static __forceinline__ float to_f(float v) { return v; }
  __device__ static __forceinline__ float from_f(float v) { return v; }
};

// Operand tiles in LDS: one row = 128 bytes = 8 chunks of 16 bytes.  The LDS
// serves a 16-byte-per-lane read 16 lanes at a time from a 256-byte bank
// window (two rows), so the chunk index is XOR-swizzled with row / 2: 16
// consecutive rows reading the same logical chunk then cover all 16 slots of
// the window (row parity picks the half, row / 2 the slot).
__device__ __forceinline__ int lds_off(int row, int chunk) { return row * 128 + (((chunk ^ (row >> 1)) & 7) << 4); }

// Output staging tiles: rows of CPR 16-byte chunks (CPR a multiple of 8).
// The epilogue writes 8 bytes per lane with lanes l = 0..31 on rows l, so the
// swizzle spreads consecutive rows over the 256-byte bank window: with CPR a
// multiple of 16 every row starts at the same window offset and the chunk is
// XORed with row % 16 (16 slots, 2-way at 64 lanes); otherwise rows alternate
// window halves and the low three bits are XORed with row / 2.
template <int CPR>
__device__ __forceinline__ int stage_chunk(int row, int chunk) {
  static_assert(CPR % 8 == 0, "staging rows are whole 128-byte groups");
  if constexpr (CPR % 16 == 0) return chunk ^ (row & 15);
  else return (chunk & ~7) | ((chunk ^ (row >> 1)) & 7);
}

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2).  Renumber so that consecutive tile ids run on the same XCD and share
// operand rows in its L2.
__device__ __forceinline__ int xcd_tile_id(int bid, int nwg) {
  const int full = nwg & ~7;
  if (bid >= full) return bid;
  const int per = full >> 3;
  return (bid & 7) * per + (bid >> 3);
}

__device__ __forceinline__ uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

// 16x16 block += A(16 x 32) * B(32 x 16): lane (i, g) holds A[i][8g .. 8g+7],
// lane (j, g) holds B[8g .. 8g+7][j]; D[i][j] at lane j + 16 (i / 4), reg i % 4.
__device__ __forceinline__ void mma16(f32x4& acc, const uint4& a, const uint4& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                acc, 0, 0, 0);
}

// 8 x 8 transpose of 16-bit elements held in registers: in[e] holds row e
// (8 elements), out[c] receives column c (element e = in[e][c]).
__device__ __forceinline__ void transpose8x8_b16(const uint4 (&in)[8], uint4 (&out)[8]) {
  uint32_t w[8][4];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    w[e][0] = in[e].x;
    w[e][1] = in[e].y;
    w[e][2] = in[e].z;
    w[e][3] = in[e].w;
  }
  uint32_t o[8][4];
#pragma unroll
  for (int p = 0; p < 4; ++p)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      // low halves of rows 2m, 2m+1 -> column 2p; high halves -> column 2p+1
      o[2 * p][m] = __builtin_amdgcn_perm(w[2 * m + 1][p], w[2 * m][p], 0x05040100u);
      o[2 * p + 1][m] = __builtin_amdgcn_perm(w[2 * m + 1][p], w[2 * m][p], 0x07060302u);
    }
#pragma unroll
  for (int c = 0; c < 8; ++c) out[c] = make_uint4(o[c][0], o[c][1], o[c][2], o[c][3]);
}
