// MFMA GEMM engine for gfx950: C[BM x BN] tile += sum over phases of
// A_phase[BM x K_phase] * B_phase[BN x K_phase]^T, every operand contiguous
// along its reduction axis ("TN" layout).  A phase sequence lets one tile
// accumulate products with different operands (e.g. T V + L R_b for several
// segments b) through one software pipeline:
//   global -> registers (tile t+1)  ||  LDS -> MFMA (tile t)  -> LDS (t+1)
// with double-buffered, XOR-swizzled LDS stages and one barrier per k-tile.
// The MFMA is issued with the operands swapped so each lane ends up holding
// four consecutive output columns of one output row; the epilogue stages the
// tile through LDS and writes 16-byte coalesced rows.
#pragma once

#include "device_common.h"

// One K-contiguous operand of a phase: tile rows [row0, row0 + tile) of a
// row-major matrix; rows outside [row_lo, row_hi) and bytes at or beyond
// kbytes along k read as zero.  kbytes is a multiple of 16.
struct OpK {
  const char* ptr;   // byte address of (row 0, k 0)
  int64_t ld;        // bytes between rows
  int64_t row0, row_lo, row_hi;
  int64_t kbytes;
};

struct Phase {
  OpK a, b;
};

template <typename T, int BM_, int BN_, int NWM_, int NWN_>
struct GemmCfg {
  typedef T elem;
  static constexpr int BM = BM_, BN = BN_, NWM = NWM_, NWN = NWN_;
  static constexpr int NT = NWM * NWN * 64;
  static constexpr int WM = BM / NWM, WN = BN / NWN;
  static constexpr int FM = WM / 32, FN = WN / 32;
  static constexpr int ACH = BM * 8 / NT, BCH = BN * 8 / NT;
  static constexpr int STAGE = (BM + BN) * 128;
  static constexpr int LDS_OPS = 2 * STAGE;
  static constexpr int CPR = BN * TT<T>::ESZ / 16;
  static constexpr int LDS_OUT = BM * CPR * 16;
  static constexpr int LDS = LDS_OPS > LDS_OUT ? LDS_OPS : LDS_OUT;
  // single-stage pipeline (gemm_mainloop1): one operand stage
  static constexpr int LDS1 = STAGE > LDS_OUT ? STAGE : LDS_OUT;
  static_assert(ACH * NT == BM * 8, "A tile chunks must divide over the threads");
  static_assert(BCH * NT == BN * 8, "B tile chunks must divide over the threads");
  static_assert(FM * 32 == WM && FN * 32 == WN, "wave tile must be a multiple of 32x32");
  static_assert(CPR % 8 == 0, "output row must be a multiple of 128 bytes");
};

template <class C>
struct TileRegs {
  uint4 a[C::ACH];
  uint4 b[C::BCH];
};

// Operand loads are raw buffer loads relative to the tile's first row: a
// chunk outside the operand (row mask or k extent) gets an out-of-range
// offset and reads as zero, so the loads are branch-free and the compiler can
// keep several k-tiles in flight.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const OpK& o) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(o.ptr + o.row0 * o.ld), (short)0, 0x7fffffff,
                                           0x00020000);
}

__device__ __forceinline__ uint4 load_opk(const OpK& o, __amdgpu_buffer_rsrc_t rs, int row, int kb) {
  const int64_t grow = o.row0 + row;
  const bool ok = grow >= o.row_lo && grow < o.row_hi && kb < o.kbytes;
  const int off = ok ? (int)(row * o.ld) + kb : (int)0x80000000u;
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
}

template <class C>
__device__ __forceinline__ void load_tile(const Phase& ph, int kt, TileRegs<C>& r, int tid) {
  const int kb = kt * 128;
  const __amdgpu_buffer_rsrc_t ra = tile_rsrc(ph.a), rb = tile_rsrc(ph.b);
#pragma unroll
  for (int i = 0; i < C::ACH; ++i) {
    const int c = tid + i * C::NT;
    r.a[i] = load_opk(ph.a, ra, c >> 3, kb + (c & 7) * 16);
  }
#pragma unroll
  for (int i = 0; i < C::BCH; ++i) {
    const int c = tid + i * C::NT;
    r.b[i] = load_opk(ph.b, rb, c >> 3, kb + (c & 7) * 16);
  }
}

template <class C>
__device__ __forceinline__ void store_tile(char* stage, const TileRegs<C>& r, int tid) {
#pragma unroll
  for (int i = 0; i < C::ACH; ++i) {
    const int c = tid + i * C::NT;
    *reinterpret_cast<uint4*>(stage + lds_off(c >> 3, c & 7)) = r.a[i];
  }
  char* bs = stage + C::BM * 128;
#pragma unroll
  for (int i = 0; i < C::BCH; ++i) {
    const int c = tid + i * C::NT;
    *reinterpret_cast<uint4*>(bs + lds_off(c >> 3, c & 7)) = r.b[i];
  }
}

// acc[fm][fn] (a 32x32 block, transposed in the lanes) += A_blk * B_blk^T over
// one 128-byte k-tile held in `stage`.
template <class C>
__device__ __forceinline__ void compute_tile(const char* stage, f32x16 (&acc)[C::FM][C::FN], int lane,
                                             int wm, int wn) {
  typedef typename C::elem T;
  const char* as = stage;
  const char* bs = stage + C::BM * 128;
  const int l = lane & 31, g = lane >> 5;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    uint4 af[C::FM], bfr[C::FN];
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm) {
      const int row = wm * C::WM + fm * 32 + l;
      af[fm] = *reinterpret_cast<const uint4*>(as + lds_off(row, 2 * ks + g));
    }
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) {
      const int row = wn * C::WN + fn * 32 + l;
      bfr[fn] = *reinterpret_cast<const uint4*>(bs + lds_off(row, 2 * ks + g));
    }
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn) TT<T>::mma(acc[fm][fn], bfr[fn], af[fm]);
  }
}

// Runs the software pipeline over `total` k-tiles.  src(t, ph, kt) resolves
// flat k-tile t to its phase operands and the k-tile index inside the phase
// (uniform scalar arithmetic, no state carried between iterations).
template <class C, class Src>
__device__ __forceinline__ void gemm_mainloop(const Src& src, int total, char* lds,
                                              f32x16 (&acc)[C::FM][C::FN]) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w / C::NWN, wn = w % C::NWN;
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[fm][fn][v] = 0.f;
  if (total <= 0) return;
  TileRegs<C> r;
  {
    Phase ph;
    int kt;
    src(0, ph, kt);
    load_tile<C>(ph, kt, r, tid);
  }
  store_tile<C>(lds, r, tid);
  __syncthreads();
  for (int t = 0; t < total; ++t) {
    const bool more = t + 1 < total;
    if (more) {
      Phase ph;
      int kt;
      src(t + 1, ph, kt);
      load_tile<C>(ph, kt, r, tid);
    }
    compute_tile<C>(lds + (t & 1) * C::STAGE, acc, lane, wm, wn);
    if (more) {
      store_tile<C>(lds + ((t + 1) & 1) * C::STAGE, r, tid);
      __syncthreads();
    }
  }
}

// Single-stage variant: registers prefetch k-tile t + 1 while t is computed
// from the one LDS stage (two barriers per k-tile).  Half the operand LDS of
// gemm_mainloop, so twice as many workgroups fit on a CU; with short
// reductions (a few k-tiles per output tile) the extra resident workgroups,
// whose epilogues overlap each other's k-loops, outweigh the second barrier.
template <class C, class Src>
__device__ __forceinline__ void gemm_mainloop1(const Src& src, int total, char* lds,
                                               f32x16 (&acc)[C::FM][C::FN]) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w / C::NWN, wn = w % C::NWN;
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[fm][fn][v] = 0.f;
  if (total <= 0) return;
  TileRegs<C> r;
  {
    Phase ph;
    int kt;
    src(0, ph, kt);
    load_tile<C>(ph, kt, r, tid);
  }
  for (int t = 0; t < total; ++t) {
    store_tile<C>(lds, r, tid);
    __syncthreads();
    if (t + 1 < total) {
      Phase ph;
      int kt;
      src(t + 1, ph, kt);
      load_tile<C>(ph, kt, r, tid);
    }
    compute_tile<C>(lds, acc, lane, wm, wn);
    __syncthreads();
  }
}

// One k-tile of both operands straight from memory into an LDS stage
// (buffer loads with the LDS as destination; no registers), in the
// store_tile layout: wave w fills 8-row blocks w, w + NW, ..., lane L of a
// block the 16-byte slot L % 8 of row L / 8, which lds_off assigns to chunk
// (L % 8) ^ ((row / 2) % 8).  Chunks outside the operand read as zero.
template <class C>
__device__ __forceinline__ void dma_tile(const Phase& ph, int kt, char* stage, int lane, int w) {
  typedef __attribute__((address_space(3))) void lds_void;
  constexpr int NW = C::NT / 64;
  const int kb = kt * 128;
  auto one = [&](const OpK& o, char* base, int nblk) {
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(o);
#pragma unroll
    for (int j = 0; j < nblk; ++j) {
      const int blk = w + j * NW;
      const int row = blk * 8 + (lane >> 3);
      const int chunk = (lane & 7) ^ ((row >> 1) & 7);
      const int64_t grow = o.row0 + row;
      const int kk = kb + chunk * 16;
      const bool ok = grow >= o.row_lo && grow < o.row_hi && kk < o.kbytes;
      const int off = ok ? (int)(row * o.ld) + kk : (int)0x80000000u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(base + blk * 1024), 16, off, 0, 0, 0);
    }
  };
  one(ph.a, stage, C::ACH);
  one(ph.b, stage + C::BM * 128, C::BCH);
}

// Single stage fed by dma_tile: no operand registers at all (so more
// workgroups fit on a CU); the load latency of a k-tile is hidden by the
// other resident workgroups rather than inside this one.
template <class C, class Src>
__device__ __forceinline__ void gemm_mainloop1_dma(const Src& src, int total, char* lds,
                                                   f32x16 (&acc)[C::FM][C::FN]) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w / C::NWN, wn = w % C::NWN;
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[fm][fn][v] = 0.f;
  for (int t = 0; t < total; ++t) {
    Phase ph;
    int kt;
    src(t, ph, kt);
    dma_tile<C>(ph, kt, lds, lane, w);
    __syncthreads();   // waits for this wave's loads; then every wave's have landed
    compute_tile<C>(lds, acc, lane, wm, wn);
    __syncthreads();   // every wave is done reading before the next k-tile lands
  }
}

__device__ __forceinline__ int ktiles(int64_t kbytes) { return (int)((kbytes + 127) >> 7); }

// Writes acc (+ bias[col] when bias != nullptr; bias points at the tile's
// first column and holds bias_n valid entries) into the LDS staging tile as T.
template <class C>
__device__ __forceinline__ void stage_out(char* lds, const f32x16 (&acc)[C::FM][C::FN],
                                          const typename C::elem* bias, int bias_n) {
  typedef typename C::elem T;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w / C::NWN, wn = w % C::NWN;
  const int l = lane & 31, g = lane >> 5;
  __syncthreads();
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm) {
    const int row = wm * C::WM + fm * 32 + l;
    char* rowp = lds + row * (C::CPR * 16);
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = wn * C::WN + fn * 32 + 8 * q + 4 * g;
        float v0 = acc[fm][fn][4 * q + 0], v1 = acc[fm][fn][4 * q + 1];
        float v2 = acc[fm][fn][4 * q + 2], v3 = acc[fm][fn][4 * q + 3];
        if (bias != nullptr && col < bias_n) {
          T b4[4];
          if constexpr (TT<T>::ESZ == 2) *reinterpret_cast<uint2*>(b4) = *reinterpret_cast<const uint2*>(bias + col);
          else *reinterpret_cast<float4*>(b4) = *reinterpret_cast<const float4*>(bias + col);
          v0 += TT<T>::to_f(b4[0]);
          v1 += TT<T>::to_f(b4[1]);
          v2 += TT<T>::to_f(b4[2]);
          v3 += TT<T>::to_f(b4[3]);
        }
        if constexpr (TT<T>::ESZ == 2) {
          uint2 pk;
          pk.x = (uint32_t)f2bf(v0) | ((uint32_t)f2bf(v1) << 16);
          pk.y = (uint32_t)f2bf(v2) | ((uint32_t)f2bf(v3) << 16);
          const int chunk = col >> 3;
          *reinterpret_cast<uint2*>(rowp + stage_chunk<C::CPR>(row, chunk) * 16 + (col & 4) * 2) = pk;
        } else {
          const int chunk = col >> 2;
          *reinterpret_cast<float4*>(rowp + stage_chunk<C::CPR>(row, chunk) * 16) = make_float4(v0, v1, v2, v3);
        }
      }
    }
  }
  __syncthreads();
}

// Copies the staged tile to global rows: dst = byte address of the tile's
// (0, 0) element, ldb = bytes between rows; rows >= rows_valid and bytes >=
// colbytes_valid are not written.
// STREAM: the destination is a final output nobody reads back soon; its
// lines are stored non-temporally so they do not evict the operands that the
// other workgroups of the XCD are still reading from L2.  Every wave store
// covers whole 128-byte lines, which the non-temporal path needs to stay
// efficient.
template <class C, bool STREAM = false>
__device__ __forceinline__ void copy_out(const char* lds, char* dst, int64_t ldb, int rows_valid,
                                         int64_t colbytes_valid) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  for (int c = threadIdx.x; c < C::BM * C::CPR; c += C::NT) {
    const int row = c / C::CPR, ch = c % C::CPR;
    if (row < rows_valid && (int64_t)ch * 16 < colbytes_valid) {
      const uint4 v = *reinterpret_cast<const uint4*>(lds + row * (C::CPR * 16) + stage_chunk<C::CPR>(row, ch) * 16);
      char* p = dst + row * ldb + ch * 16;
      if constexpr (STREAM) __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4*>(p));
      else *reinterpret_cast<uint4*>(p) = v;
    }
  }
}

// Reads element (row, col) of the staged tile.
template <class C>
__device__ __forceinline__ typename C::elem staged_elem(const char* lds, int row, int col) {
  typedef typename C::elem T;
  const int byte = col * TT<T>::ESZ;
  return *reinterpret_cast<const T*>(lds + row * (C::CPR * 16) + stage_chunk<C::CPR>(row, byte >> 4) * 16 + (byte & 15));
}
