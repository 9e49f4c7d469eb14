// DyRA layer forward on gfx950: kernels and the C-ABI entry points that
// launch them.
//
// Per segment b (rows [b s, (b+1) s) of X), following the one-step ALS
// correction of the DyRA pages (nanless.github.io digest: residual-product
// objective, its cheap ordering, and the one-iteration form
// XW ~ X W_hat + L1 R1; paperlayer.ai 2.2 and 2.4):
//   S1  [T | L] = X [U | P]           one MFMA pass over X (T = X U_f, L = X P)
//   S3  M_b = L_b^T X_b, G_b = L_b^T L_b   split-N MFMA reductions over tokens
//   S4  Ginv_b = (G_b + lambda_b I)^-1     symmetric sweep (AUTO, every r; fp32,
//                                          fp64 where a pivot needs it), or the
//                                          Cholesky route / Newton-Schulz
//       M'_b = Ginv_b M_b
//   S5  R_b = M'_b W_res               one GEMM over all segments (R^T stored)
//   S6  Y_b = T_b V + L_b R_b + bias    one fused GEMM, K = k + r, with a
//                                       per-segment second operand; L R is
//                                       never written to memory
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <atomic>
#include <mutex>
#include <type_traits>

#include "../../include/dyra.h"
#include "device_common.h"
#include "gemm_engine.h"
#include "lds_dma.h"
#include "spec.h"

using namespace dyra_spec_util;

namespace {

__host__ __device__ __forceinline__ int64_t imin64(int64_t a, int64_t b) { return a < b ? a : b; }
__host__ __device__ __forceinline__ int64_t imax64(int64_t a, int64_t b) { return a > b ? a : b; }

// ===========================================================================
// generic single-phase GEMM: C[M x N] = A[M x K] B[N x K]^T (+ bias[N])
// ===========================================================================

// ONE_STAGE / WPE: as for the fused output GEMM (single operand stage, at
// least WPE waves per SIMD worth of registers).
template <class C, bool ONE_STAGE = false, int WPE = 1, bool DMA = false>
__global__ __launch_bounds__(C::NT, WPE) void gemm_tn_kernel(const char* A, int64_t lda, const char* B,
                                                        int64_t ldb, char* Cg, int64_t ldc, int64_t M,
                                                        int64_t N, int64_t K,
                                                        const typename C::elem* bias, int tiles_n,
                                                        int64_t sA, int64_t sB, int64_t sC, int tiles_per_batch) {
  typedef typename C::elem T;
  __shared__ __attribute__((aligned(16))) char lds[ONE_STAGE ? C::LDS1 : C::LDS];
  // batch z: A += z sA, B += z sB, C += z sC (byte strides)
  const int z = blockIdx.x / tiles_per_batch;
  const int t = xcd_tile_id(blockIdx.x % tiles_per_batch, tiles_per_batch);
  A += z * sA;
  B += z * sB;
  Cg += z * sC;
  const int64_t m0 = (int64_t)(t / tiles_n) * C::BM, n0 = (int64_t)(t % tiles_n) * C::BN;
  const int64_t kb = K * TT<T>::ESZ;
  auto src = [=](int tt, Phase& ph, int& kt) {
    ph.a = OpK{A, lda, m0, 0, M, kb};
    ph.b = OpK{B, ldb, n0, 0, N, kb};
    kt = tt;
  };
  f32x16 acc[C::FM][C::FN];
  if constexpr (DMA) gemm_mainloop1_dma<C>(src, ktiles(kb), lds, acc);
  else if constexpr (ONE_STAGE) gemm_mainloop1<C>(src, ktiles(kb), lds, acc);
  else gemm_mainloop<C>(src, ktiles(kb), lds, acc);
  stage_out<C>(lds, acc, bias ? bias + n0 : nullptr, (int)(N - n0));
  copy_out<C>(lds, Cg + m0 * ldc + n0 * TT<T>::ESZ, ldc, (int)imin64(C::BM, M - m0),
              (N - n0) * TT<T>::ESZ);
}

// Slice z of a split-K C = A B^T (bf16 operands, 128 x 128 tiles, single
// operand stage as above): the fp32 sums over K elements
// [z kslice, z kslice + kslice) into P + z M N (row pitch N, N % 4 == 0),
// straight from the accumulators.
template <class C>
__global__ __launch_bounds__(C::NT, 4) void gemm_tn_splitk_kernel(const char* A, int64_t lda, const char* B,
                                                                  int64_t ldb, float* P, int64_t M, int64_t N,
                                                                  int64_t K, int64_t kslice, int tiles_n,
                                                                  int tiles) {
  static_assert(TT<typename C::elem>::ESZ == 2, "bf16 operands");
  __shared__ __attribute__((aligned(16))) char lds[C::LDS1];
  const int z = blockIdx.x / tiles;
  const int t = xcd_tile_id(blockIdx.x % tiles, tiles);
  const int64_t m0 = (int64_t)(t / tiles_n) * C::BM, n0 = (int64_t)(t % tiles_n) * C::BN;
  const int64_t k0 = z * kslice, kb = imin64(kslice, K - k0) * 2;
  A += k0 * 2;
  B += k0 * 2;
  auto src = [=](int tt, Phase& ph, int& kt) {
    ph.a = OpK{A, lda, m0, 0, M, kb};
    ph.b = OpK{B, ldb, n0, 0, N, kb};
    kt = tt;
  };
  f32x16 acc[C::FM][C::FN];
  gemm_mainloop1_dma<C>(src, ktiles(kb), lds, acc);
  // accumulator (fm, fn) element 4 q + e: row wm WM + 32 fm + lane % 32,
  // column wn WN + 32 fn + 8 q + 4 (lane / 32) + e
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w / C::NWN, wn = w % C::NWN, l = lane & 31, g = lane >> 5;
  float* Pz = P + z * M * N;
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm) {
    const int64_t row = m0 + wm * C::WM + fm * 32 + l;
    if (row >= M) continue;
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t col = n0 + wn * C::WN + fn * 32 + 8 * q + 4 * g;
        if (col < N)
          *reinterpret_cast<float4*>(Pz + row * N + col) =
              make_float4(acc[fm][fn][4 * q], acc[fm][fn][4 * q + 1], acc[fm][fn][4 * q + 2], acc[fm][fn][4 * q + 3]);
      }
  }
}

// out[i] = bf16(sum over z < slices of P[z MN + i]), eight elements per
// thread (MN % 8 == 0).
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ P, bf16_t* __restrict__ out,
                                                            int64_t MN, int slices) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i >= MN) return;
  float4 a = *reinterpret_cast<const float4*>(P + i), b = *reinterpret_cast<const float4*>(P + i + 4);
  for (int z = 1; z < slices; ++z) {
    const float4 u = *reinterpret_cast<const float4*>(P + z * MN + i);
    const float4 v = *reinterpret_cast<const float4*>(P + z * MN + i + 4);
    a.x += u.x;
    a.y += u.y;
    a.z += u.z;
    a.w += u.w;
    b.x += v.x;
    b.y += v.y;
    b.z += v.z;
    b.w += v.w;
  }
  uint4 pk;
  pk.x = (uint32_t)f2bf(a.x) | ((uint32_t)f2bf(a.y) << 16);
  pk.y = (uint32_t)f2bf(a.z) | ((uint32_t)f2bf(a.w) << 16);
  pk.z = (uint32_t)f2bf(b.x) | ((uint32_t)f2bf(b.y) << 16);
  pk.w = (uint32_t)f2bf(b.z) | ((uint32_t)f2bf(b.w) << 16);
  *reinterpret_cast<uint4*>(out + i) = pk;
}

// L = bf16(sum over z < slices of P[z][t][p]) for SRL_T tokens per workgroup
// (r <= 128): rows into L (pitch ldo) for t < n, and L^T (pitch ldt) through
// an LDS transpose for t < ldt, tokens past n as zeros.
constexpr int SRL_T = 16;
__global__ __launch_bounds__(256) void splitk_reduce_lt_kernel(const float* __restrict__ P, int slices, int64_t n,
                                                               int r, bf16_t* __restrict__ L, int64_t ldo,
                                                               bf16_t* __restrict__ Lt, int64_t ldt) {
  __shared__ __attribute__((aligned(16))) bf16_t tr[128][SRL_T + 8];
  const int64_t t0 = (int64_t)blockIdx.x * SRL_T;
  const int ru = r / 8;
  for (int q = threadIdx.x; q < SRL_T * ru; q += 256) {
    const int tl = q / ru, p0 = (q - tl * ru) * 8;
    const int64_t t = t0 + tl;
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (t < n) {
#pragma unroll 4
      for (int z = 0; z < slices; ++z) {
        const float* src = P + ((int64_t)z * n + t) * r + p0;
        const float4 a = *reinterpret_cast<const float4*>(src), b = *reinterpret_cast<const float4*>(src + 4);
        v[0] += a.x;
        v[1] += a.y;
        v[2] += a.z;
        v[3] += a.w;
        v[4] += b.x;
        v[5] += b.y;
        v[6] += b.z;
        v[7] += b.w;
      }
    }
    bf16_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      h[e] = f2bf(v[e]);
      tr[p0 + e][tl] = h[e];
    }
    if (t < n) *reinterpret_cast<uint4*>(L + t * ldo + p0) = *reinterpret_cast<const uint4*>(h);
  }
  __syncthreads();
  // L^T rows p: SRL_T tokens in runs of 16 bytes
  for (int q = threadIdx.x; q < r * (SRL_T / 8); q += 256) {
    const int p = q / (SRL_T / 8), u = q % (SRL_T / 8);
    if (t0 + u * 8 < ldt)
      *reinterpret_cast<uint4*>(Lt + (int64_t)p * ldt + t0 + u * 8) = *reinterpret_cast<const uint4*>(&tr[p][u * 8]);
  }
}

// ===========================================================================
// S1 (low-rank): [T | L] = X [U_f | P], plus L^T (token-contiguous) for S3
// ===========================================================================

// TL: output rows of pitch ldo elements (columns [0, k) = T, [k, k + r) = L).
template <class C, bool ONE_STAGE = false, int WPE = 1, bool DMA = false>
__global__ __launch_bounds__(C::NT, WPE) void s1_lowrank_kernel(const typename C::elem* X,
                                                           const typename C::elem* UPt,
                                                           typename C::elem* TL, typename C::elem* Lt,
                                                           int64_t n, int64_t c1, int k, int r,
                                                           int64_t ldt, int tiles_n, int64_t ldo) {
  typedef typename C::elem T;
  constexpr int E = TT<T>::ESZ, KPC = TT<T>::KPC;
  __shared__ __attribute__((aligned(16))) char lds[ONE_STAGE ? C::LDS1 : C::LDS];
  const int t = xcd_tile_id(blockIdx.x, gridDim.x);
  const int64_t m0 = (int64_t)(t / tiles_n) * C::BM, n0 = (int64_t)(t % tiles_n) * C::BN;
  const int64_t N = k + r;
  auto src = [=](int t, Phase& ph, int& kt) {
    ph.a = OpK{reinterpret_cast<const char*>(X), c1 * E, m0, 0, n, c1 * E};
    ph.b = OpK{reinterpret_cast<const char*>(UPt), c1 * E, n0, 0, N, c1 * E};
    kt = t;
  };
  f32x16 acc[C::FM][C::FN];
  if constexpr (DMA) gemm_mainloop1_dma<C>(src, ktiles(c1 * E), lds, acc);
  else if constexpr (ONE_STAGE) gemm_mainloop1<C>(src, ktiles(c1 * E), lds, acc);
  else gemm_mainloop<C>(src, ktiles(c1 * E), lds, acc);
  stage_out<C>(lds, acc, nullptr, 0);
  copy_out<C>(lds, reinterpret_cast<char*>(TL) + (m0 * ldo + n0) * E, ldo * E,
              (int)imin64(C::BM, n - m0), (N - n0) * E);
  // L columns of this tile, written transposed: Lt[j - k][m0 + rows]
  const int64_t j0 = imax64(n0, k), j1 = imin64(n0 + C::BN, N);
  if (j0 < j1) {
    const int ncol = (int)(j1 - j0);
    const int groups = C::BM / KPC;
    for (int c = threadIdx.x; c < ncol * groups; c += C::NT) {
      const int jl = (int)(j0 - n0) + c / groups, rg = c % groups;
      const int64_t row = m0 + (int64_t)rg * KPC;
      if (row >= ldt) continue;
      T v[KPC];
#pragma unroll
      for (int e = 0; e < KPC; ++e) v[e] = staged_elem<C>(lds, rg * KPC + e, jl);
      *reinterpret_cast<uint4*>(Lt + (n0 + jl - k) * ldt + row) = *reinterpret_cast<const uint4*>(v);
    }
  }
}

// Tokens of an 8-token run (t0 ..) outside [lo, hi) set to zero.
template <typename T>
__device__ __forceinline__ uint4 mask_tokens(uint4 v, int64_t t0, int64_t lo, int64_t hi) {
  constexpr int KPC = TT<T>::KPC;
  if (t0 >= lo && t0 + KPC <= hi) return v;
  if (t0 + KPC <= lo || t0 >= hi) return zero4();
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < KPC; ++e) {
    const int64_t tt = t0 + e;
    if (tt < lo || tt >= hi) {
      if constexpr (KPC == 8) w[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
      else w[e] = 0u;
    }
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// ---------------------------------------------------------------------------
// S1 (bf16, k + r = 320): [T | L] = X [U | P] and L^T, one 160 x 320 tile
// per workgroup (a single round of row blocks on 256 CUs; X is read once).
// Eight symmetric waves (two per SIMD) each compute 80 x 80 of the tile as
// 5 x 5 blocks of 16x16x32 MFMAs (5 + 5 fragments per 25 MFMAs), fed with
// LDS-DMA loads three 32-wide k-tiles ahead by every wave: a 4-slot ring of
// UPt k-tiles and a 3-region ring of X k-tile pairs (whole 128-byte lines).  Nothing is stored before the last k-tile, so a
// wave's wait for its part of a slot is a plain vmcnt count.  The barrier
// that publishes k-tile t + 1 comes before the MFMAs of k-tile t (whose
// fragments are already in registers), so the next fragments are read while
// they run.  The epilogue stages the tile in the ring and writes whole rows
// of [T | L] and whole token runs of L^T.  With Gp (r = 32 or 64, segments of
// at least 160 tokens) it also leaves the tile's Gram partials
// L_t^T L_t, one per segment the tile meets (slot 0: the segment of its first
// row, slot 1: the next one), at Gp[(tile * 2 + slot) r^2], which the token
// reduction adds up instead of streaming L^T for the Gram once more.
// ---------------------------------------------------------------------------
// waves w with (w & S1T_LATE) != 0 issue their k-tile DMAs after two rows of MFMAs
constexpr int S1T_LATE = 4;
__global__ __launch_bounds__(512, 1) void s1_tile_kernel(const bf16_t* __restrict__ X,
                                                         const bf16_t* __restrict__ UPt, bf16_t* __restrict__ A,
                                                         bf16_t* __restrict__ Lt, int n, int c1, int k, int r,
                                                         int64_t ldt, float* __restrict__ Gp, SegMap sg) {
  constexpr int BM = S1T_BM, BN = S1T_BN, RBY = S1T_BK * 2;   // 64-byte k-tile rows
  constexpr int NS = 4, NP = 3, NW = 8, FB = 5;   // UPt slots, X pair regions, waves, 16-blocks per wave side
  constexpr int USLOT = BN * RBY, XPAIR = BM * 2 * RBY;       // 20 KB each
  constexpr int XOFF = NS * USLOT, RING = XOFF + NP * XPAIR;  // 140 KB
  constexpr int DW = 5;                                       // DMA blocks per wave
  constexpr int SP = BN * 2 + 16;                             // staged row pitch (bytes)
  static_assert(USLOT == 20 * 1024 && XPAIR == 20 * 1024, "20 UPt + 20 X one-KB blocks over 8 waves");
  static_assert(BM * SP <= RING, "staging fits the ring");
  constexpr int LTP = BM * 2 + 16;                            // L^T tile row pitch (bytes), 64 rows
  constexpr int LT_OFF = BM * SP;                             // after the staged tile
  static_assert(LT_OFF % 16 == 0 && LT_OFF + 64 * LTP <= RING, "L^T tile fits the ring");
  static_assert(2 * FB * 16 == BM && 4 * FB * 16 == BN, "2 x 4 waves of 80 x 80");
  __shared__ __attribute__((aligned(1024))) char ring[RING];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w >> 2, wn = w & 3;
  const int l16 = lane & 15, kg = lane >> 4;
  const int m0 = blockIdx.x * BM;
  const int rows = min(BM, n - m0);
  const int nkt = c1 / S1T_BK;                                // c1 % 64 == 0: nkt even
  const int ldx = c1 * 2;                                     // bytes per X row
  const uint32_t ring_s = lds_addr(ring);
  // UPt is k-tile-major in the plan: k-tile t is one 20 KB run, 320 rows of
  // 64 bytes, loaded into UPt slot t % 4.  X is loaded two k-tiles at a time,
  // so that every row segment is a whole 128-byte line: 160 rows of 128 bytes
  // in pair region (t / 2) % 3.  One-KB blocks: UPt block b holds rows
  // 16 b .. 16 b + 15, lane L writing row 16 b + L / 4 at physical chunk L % 4,
  // which holds logical chunk (L % 4) ^ ((row / 4) % 4); X block b holds rows
  // 8 b .. 8 b + 7, lane L writing row 8 b + L / 8 at physical chunk L % 8,
  // which holds logical chunk (L % 8) ^ ((row / 2) % 8) (chunks 0-3 the even
  // k-tile, 4-7 the odd one).  Both make a 16-lane fragment read of 16
  // consecutive rows conflict-free.  Waves 0-3 take 3 UPt and 2 X blocks,
  // waves 4-7 2 and 3: for an even k-tile a wave issues its UPt blocks and its
  // blocks of the pair's X (5 DMAs), for an odd one its UPt blocks (nU).
  const i32x4v xrs = rsrc_words(reinterpret_cast<const char*>(X) + (int64_t)m0 * ldx, (uint32_t)rows * ldx);
  const i32x4v urs = rsrc_words(UPt, (uint32_t)BN * ldx);
  const int nU = w < 4 ? 3 : 2;
  const int u0 = w < 4 ? 3 * w : 2 * w + 4, x0 = w < 4 ? 2 * w : 3 * w - 4;
  int voff[DW], loff[DW];
  i32x4v drs[DW];
#pragma unroll
  for (int j = 0; j < DW; ++j) {
    const bool isu = j < nU;
    const int blk = isu ? u0 + j : x0 + j - nU;
    if (isu) {
      const int row = 16 * blk + (lane >> 2);
      voff[j] = row * RBY + (((lane & 3) ^ ((row >> 2) & 3)) << 4);
    } else {
      const int row = 8 * blk + (lane >> 3);
      voff[j] = row * ldx + (((lane & 7) ^ ((row >> 1) & 7)) << 4);
    }
    loff[j] = __builtin_amdgcn_readfirstlane(blk * 1024);
    drs[j] = isu ? urs : xrs;
    drs[j].x = __builtin_amdgcn_readfirstlane(drs[j].x);
    drs[j].y = __builtin_amdgcn_readfirstlane(drs[j].y);
    drs[j].z = __builtin_amdgcn_readfirstlane(drs[j].z);
    drs[j].w = __builtin_amdgcn_readfirstlane(drs[j].w);
  }
  // k-tile t's DMAs (with EV, t even: the X of k-tiles t and t + 1 too);
  // k-tiles past the end read at an offset past every descriptor's records
  auto issue = [&](int t, auto ev) {
    constexpr bool EV = decltype(ev)::value;
    const bool live = t < nkt;
    const int su = live ? t * USLOT : 0x7fff0000;
    const int sx = live ? t * RBY : 0x7fff0000;
    const uint32_t lu = ring_s + (t & (NS - 1)) * USLOT;
    const uint32_t lx = ring_s + XOFF + ((t >> 1) % NP) * XPAIR;
#pragma unroll
    for (int j = 0; j < DW; ++j) {
      if (j < nU) dma16(drs[j], voff[j], su, lu + loff[j]);
      else if (EV) dma16(drs[j], voff[j], sx, lx + loff[j]);
    }
  };
  // fragments of k-tile t (H = t % 2): block f of this wave's rows (A) or
  // columns (B), lane (l16, kg): row 16 f + l16 at logical chunk kg of the
  // k-tile
  uint4 af[2][FB], bfr[2][FB];
  auto load_frags = [&](int t, auto hb) {
    constexpr int H = decltype(hb)::value;
    const char* su = ring + (t & (NS - 1)) * USLOT;
    const char* sx = ring + XOFF + ((t >> 1) % NP) * XPAIR;
#pragma unroll
    for (int f = 0; f < FB; ++f) {
      const int ra = wm * 80 + f * 16 + l16, rb = wn * 80 + f * 16 + l16;
      af[H][f] = *reinterpret_cast<const uint4*>(sx + ra * (2 * RBY) + (((H * 4 + kg) ^ ((ra >> 1) & 7)) << 4));
      bfr[H][f] = *reinterpret_cast<const uint4*>(su + rb * RBY + ((kg ^ ((rb >> 2) & 3)) << 4));
    }
  };
  f32x4 acc[FB][FB];
#pragma unroll
  for (int a = 0; a < FB; ++a)
#pragma unroll
    for (int b = 0; b < FB; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  using Even = std::integral_constant<bool, true>;
  using Odd = std::integral_constant<bool, false>;
  issue(0, Even());
  issue(1, Odd());
  issue(2, Even());
  issue(3, Odd());
  // k-tile 0 (UPt and the X pair in its DMAs; k-tiles 1 .. 3 issued after it)
  if (w < 4) wait_vm_lgkm0<3 + 5 + 3>();
  else wait_vm_lgkm0<2 + 5 + 2>();
  bare_barrier();
  load_frags(0, std::integral_constant<int, 0>());
  // two k-tiles per trip: fragment buffers 0 and 1 alternate statically
  auto step = [&](int kt, auto cur) {
    constexpr int C = decltype(cur)::value, NX = 1 - C;
    // this wave's part of k-tile kt + 1 (the DMAs of the two k-tiles issued
    // after it stay in flight); fragments of kt
    if (w < 4) wait_vm_lgkm0<5 + 3>();
    else wait_vm_lgkm0<5 + 2>();
    bare_barrier();                       // k-tile kt + 1 everywhere; k-tile kt is read
    // Half of the waves issue their DMAs now, the other half after two rows
    // of MFMAs: a wave waiting on the address path cannot issue MFMAs, and
    // the two waves of a SIMD then do not wait at the same time.
    const bool late = (w & S1T_LATE) != 0;
    if (!late) issue(kt + NS, std::integral_constant<bool, C == 0>());
    if (kt + 1 < nkt) load_frags(kt + 1, std::integral_constant<int, NX>());
    __builtin_amdgcn_sched_barrier(0);
    // lane (l16, kg) of block (a, b) receives row 16 a + l16, columns
    // 16 b + 4 kg .. + 3 (the B fragment is the first operand)
#pragma unroll
    for (int a = 0; a < FB; ++a) {
#pragma unroll
      for (int b = 0; b < FB; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, bfr[C][b]),
                                                            __builtin_bit_cast(bf16x8_t, af[C][a]), acc[a][b], 0, 0, 0);
      if (a == 1) {
        __builtin_amdgcn_sched_barrier(0);
        if (late) issue(kt + NS, std::integral_constant<bool, C == 0>());
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int kt = 0; kt < nkt; kt += 2) {
    step(kt, std::integral_constant<int, 0>());
    step(kt + 1, std::integral_constant<int, 1>());
  }
  wait_vm_lgkm0<0>();                     // the trailing zero-fill loads too
  bare_barrier();
  // stage the tile (bf16, row pitch SP)
#pragma unroll
  for (int a = 0; a < FB; ++a)
#pragma unroll
    for (int b = 0; b < FB; ++b) {
      const int row = wm * 80 + a * 16 + l16, col = wn * 80 + b * 16 + 4 * kg;
      uint2 pk;
      pk.x = pack_bf16x2(acc[a][b][0], acc[a][b][1]);
      pk.y = pack_bf16x2(acc[a][b][2], acc[a][b][3]);
      *reinterpret_cast<uint2*>(ring + row * SP + col * 2) = pk;
    }
  __syncthreads();
  // [T | L] rows: 40 chunks of 16 bytes each
  for (int q = tid; q < BM * (BN / 8); q += NW * 64) {
    const int row = q / (BN / 8), c = q - row * (BN / 8);
    if (row >= rows) break;
    const uint4 v = *reinterpret_cast<const uint4*>(ring + row * SP + c * 16);
    *reinterpret_cast<uint4*>(A + (int64_t)(m0 + row) * BN + c * 8) = v;
  }
  // L^T (tokens past n hold zeros: their X rows were read as zeros), in
  // 8 x 8 blocks: 8 token rows of 8 L columns read as 16-byte chunks, an
  // in-register transpose, 8 runs of 8 tokens.  Neighbouring lanes take
  // neighbouring column blocks (distinct banks); the 8 lanes of one column
  // block write a 128-byte run of each L^T row.
  for (int q = tid; q < (BM / 8) * (r / 8); q += NW * 64) {
    const int j8 = (q % (r / 8)) * 8, tt = (q / (r / 8)) * 8;
    if (m0 + tt >= ldt) continue;
    uint4 in[8], out[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) in[e] = *reinterpret_cast<const uint4*>(ring + (tt + e) * SP + (k + j8) * 2);
    transpose8x8_b16(in, out);
#pragma unroll
    for (int c = 0; c < 8; ++c) *reinterpret_cast<uint4*>(Lt + (int64_t)(j8 + c) * ldt + m0 + tt) = out[c];
    if (Gp) {
#pragma unroll
      for (int c = 0; c < 8; ++c) *reinterpret_cast<uint4*>(ring + LT_OFF + (j8 + c) * LTP + tt * 2) = out[c];
    }
  }
  if (!Gp) return;
  // Gram partials: waves 0 .. 3 take the first segment's tokens of the tile,
  // waves 4 .. 7 the next segment's (if the tile reaches it); wave w & 3 one
  // 32 x 32 block of the r x r partial
  __syncthreads();
  const int64_t b0 = sg.of(m0);
  const int bnd = (int)(sg.hi(b0) - m0);                       // tile-local first token of segment b0 + 1
  const int slot = w >> 2, blk = w & 3, nbr = r >> 5;
  const int tlo = slot ? bnd : 0, thi = slot ? rows : min(bnd, rows);
  if (blk >= nbr * nbr || tlo >= thi) return;
  const int ib = blk / nbr, jb = blk - ib * nbr;
  const int l = lane & 31, g = lane >> 5;
  f32x16 gacc;
#pragma unroll
  for (int v = 0; v < 16; ++v) gacc[v] = 0.f;
#pragma unroll
  for (int ks = 0; ks < BM / 16; ++ks) {
    const int t0 = ks * 16 + 8 * g;
    const uint4 fa = mask_tokens<bf16_t>(
        *reinterpret_cast<const uint4*>(ring + LT_OFF + (ib * 32 + l) * LTP + t0 * 2), t0, tlo, thi);
    const uint4 fb = mask_tokens<bf16_t>(
        *reinterpret_cast<const uint4*>(ring + LT_OFF + (jb * 32 + l) * LTP + t0 * 2), t0, tlo, thi);
    gacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, fa), __builtin_bit_cast(bf16x8_t, fb),
                                                   gacc, 0, 0, 0);
  }
  // element v of lane (l, g): G[ib 32 + 8 (v / 4) + 4 g + v % 4][jb 32 + l]
  float* out = Gp + ((int64_t)blockIdx.x * 2 + slot) * r * r;
#pragma unroll
  for (int v = 0; v < 16; ++v) out[(ib * 32 + (v >> 2) * 8 + g * 4 + (v & 3)) * r + jb * 32 + l] = gacc[v];
}

// ===========================================================================
// S6 (low-rank): Y = T V + L R_b + bias, segments handled by row masks
// ===========================================================================

// ONE_STAGE: single operand stage.  WPE: minimum waves per SIMD the
// registers must allow (the second launch bound), i.e. how many workgroups
// share a CU; their epilogues then overlap each other's k-loops.
template <class C, bool ONE_STAGE = false, bool STREAM = true, int WPE = 1, bool DMA = false>
__global__ __launch_bounds__(C::NT, WPE) void s6_lowrank_kernel(const typename C::elem* TL,
                                                           const typename C::elem* Vt,
                                                           const typename C::elem* Rt,
                                                           const typename C::elem* bias,
                                                           typename C::elem* Y, int64_t n, int64_t c2,
                                                           int k, int r, SegMap sg, int64_t B,
                                                           int tiles_n) {
  typedef typename C::elem T;
  constexpr int E = TT<T>::ESZ;
  __shared__ __attribute__((aligned(16))) char lds[ONE_STAGE ? C::LDS1 : C::LDS];
  const int t = xcd_tile_id(blockIdx.x, gridDim.x);
  const int64_t m0 = (int64_t)(t / tiles_n) * C::BM, n0 = (int64_t)(t % tiles_n) * C::BN;
  const int64_t lda = (int64_t)(k + r) * E;
  const int64_t bfirst = sg.of(imin64(m0, n - 1));
  const int64_t blast = imin64(B - 1, sg.of(imin64(m0 + C::BM, n) - 1));
  const char* TLc = reinterpret_cast<const char*>(TL);
  const int nk0 = ktiles((int64_t)k * E), nkr = ktiles((int64_t)r * E);
  const int total = nk0 + (int)(blast - bfirst + 1) * nkr;
  auto src = [=](int t, Phase& ph, int& kt) {
    if (t < nk0) {
      ph.a = OpK{TLc, lda, m0, 0, n, (int64_t)k * E};
      ph.b = OpK{reinterpret_cast<const char*>(Vt), (int64_t)k * E, n0, 0, c2, (int64_t)k * E};
      kt = t;
      return;
    }
    const int u = t - nk0;
    const int64_t b = bfirst + u / nkr;
    kt = u % nkr;
    ph.a = OpK{TLc + (int64_t)k * E, lda, m0, sg.lo(b), sg.hi(b), (int64_t)r * E};
    ph.b = OpK{reinterpret_cast<const char*>(Rt + b * r), B * r * E, n0, 0, c2, (int64_t)r * E};
  };
  f32x16 acc[C::FM][C::FN];
  if constexpr (DMA) gemm_mainloop1_dma<C>(src, total, lds, acc);
  else if constexpr (ONE_STAGE) gemm_mainloop1<C>(src, total, lds, acc);
  else gemm_mainloop<C>(src, total, lds, acc);
  stage_out<C>(lds, acc, bias ? bias + n0 : nullptr, (int)(c2 - n0));
  copy_out<C, STREAM>(lds, reinterpret_cast<char*>(Y) + (m0 * c2 + n0) * E, c2 * E,
              (int)imin64(C::BM, n - m0), (c2 - n0) * E);
}

// ---------------------------------------------------------------------------
// S6 (low-rank, bf16), persistent and wave-specialised.
//
// One workgroup per CU walks a contiguous range of BM x BN output tiles of
// its XCD (workgroups are dispatched round-robin over the 8 XCDs, so the
// tiles an XCD works on at a time share their T|L rows and V^T / R_b rows in
// its L2).  The k-tiles of consecutive tiles (nk0 of [T|V], then nkr per
// segment the tile overlaps) form one stream that flows through an NS-slot
// LDS ring:
//   * NL loader waves issue LDS-DMA loads NS - 1 k-tiles ahead and wait on
//     them (vmcnt);
//   * the compute waves run the MFMAs and the epilogue stores and never wait
//     on vmcnt.  On gfx9 vmcnt counts loads and stores in one queue, so a
//     wave that both stored Y and waited for its next operands would wait
//     for its 256 KB of streaming stores first.
// One barrier per k-tile hands a landed slot to the compute waves and the
// slot they finished back to the loaders.  Each slot carries the tile's bias
// in a 256-byte tail; the first MFMA of a tile takes it as its addend, so the
// epilogue only converts, stages 32 rows per wave in that wave's part of the
// consumed slot, and writes whole 128-byte lines non-temporally.
// ---------------------------------------------------------------------------
//
// The first part's A operand is A0 (row pitch lda0 bytes; with acolb > 0 its
// columns start at (n0 / acolb) k for the tile at output column n0: the
// BLAST coupled output W'_j of block column j), the residual part's A1
// (pitch lda1: L).  Low-rank: A0 = [T | L], A1 = its L columns.
template <class C, int NS, int NL, bool HAS_BIAS>
__global__ __launch_bounds__(C::NT + NL * 64, 1) void s6_lowrank_ws_kernel(
    const bf16_t* __restrict__ A0, int lda0, int acolb, const bf16_t* __restrict__ A1, int lda1,
    const bf16_t* __restrict__ Vt, const bf16_t* __restrict__ Rt,
    const bf16_t* __restrict__ bias, bf16_t* __restrict__ Y, int n, int c2, int k, int r, SegMap sg, int B,
    int tiles_n, int tiles) {
  static_assert(NS >= 2 && NS <= 4, "ring depth");
  static_assert(NL % 2 == 0 && (C::BM / 8) % NL == 0 && (C::BN / 8) % NL == 0, "loader blocks");
  constexpr int NWC = C::NT / 64;                            // compute waves
  constexpr int LA = C::BM / 8 / NL, LB = C::BN / 8 / NL;    // 1 KB blocks per loader per k-tile
  constexpr int PTL = LA + LB + 1;                           // DMAs per loader lane per k-tile
  constexpr int TAIL = 256;
  static_assert(C::BN * 2 == TAIL, "bias tail: one 4-byte DMA lane per column pair");
  constexpr int SLOT = C::STAGE + TAIL;
  constexpr int RING = NS * SLOT;
  constexpr int WAREA = C::STAGE / NWC;                      // per-wave staging area
  constexpr int RB = C::WN * 2;                              // staged row bytes
  static_assert(RB == 128 && WAREA >= 32 * RB, "per-wave staging of 32 rows of 128 bytes");
  __shared__ __attribute__((aligned(1024))) char ring[RING];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = lane & 31, gq = lane >> 5;
  const int kE = k * 2, rE = r * 2, ldr = B * rE;
  const int nk0 = (kE + 127) >> 7, nkr = (rE + 127) >> 7;
  const int G8 = gridDim.x >> 3, xcd = blockIdx.x & 7, lw = blockIdx.x >> 3;
  const int chunk = (tiles + 7) >> 3;
  const int hi_tile = min(tiles, (xcd + 1) * chunk);
  // Tile cursors advance by G8 tiles without integer division: the row and
  // column steps are precomputed, and the first and last segment of the
  // tile's rows move forward with the rows.
  const int dtm = G8 / tiles_n, dtn = G8 - dtm * tiles_n;
  struct Cur {
    int t, tm, tn, m0, n0, b0, bl, tot;
  };
  auto settle = [&](Cur& c) {   // segments, k-tile count of the tile at (tm, tn)
    c.m0 = c.tm * C::BM;
    c.n0 = c.tn * C::BN;
    while (sg.lo(c.b0 + 1) <= c.m0) ++c.b0;
    const int last = min(c.m0 + C::BM, n) - 1;
    if (c.bl < c.b0) c.bl = c.b0;
    while (c.bl + 1 < B && sg.lo(c.bl + 1) <= last) ++c.bl;
    c.tot = nk0 + (c.bl - c.b0 + 1) * nkr;
  };
  auto start = [&](Cur& c, int t) {
    c.t = t;
    c.tm = t / tiles_n;
    c.tn = t - c.tm * tiles_n;
    c.b0 = 0;
    c.bl = 0;
    if (t < hi_tile) {
      c.b0 = (int)sg.of(c.tm * C::BM);
      c.bl = c.b0;
      settle(c);
    }
  };
  auto advance = [&](Cur& c) {
    c.t += G8;
    c.tm += dtm;
    c.tn += dtn;
    if (c.tn >= tiles_n) { c.tn -= tiles_n; ++c.tm; }
    if (c.t < hi_tile) settle(c);
  };
  Cur cc;
  start(cc, xcd * chunk + lw);
  int ckt = 0;
  bool live = cc.t < hi_tile;
  if (w >= NWC) {
    // ------------------------------ loaders ------------------------------
    const int q = w - NWC;
    const uint32_t ring_s = lds_addr(ring);
    // loader q fills 8-row blocks q + j NL of each operand: lane L loads row
    // 8 (q + j NL) + L / 8 at 16-byte chunk (L % 8) ^ ((row / 2) % 8) (the
    // lds_off swizzle), which is the same chunk for every j as NL is even
    const int row0 = q * 8 + (lane >> 3);
    const int ch16 = ((lane & 7) ^ ((row0 >> 1) & 7)) << 4;
    const int a_v0 = row0 * lda0 + ch16, a_v1 = row0 * lda1 + ch16, v_v = row0 * kE + ch16, r_v = row0 * ldr + ch16;
    // Issue state: the k-tiles of a tile come in parts, [T | V] (nk0
    // k-tiles) and then [L_b | R_b] per segment b the tile meets (nkr each);
    // descriptors, row bounds and fast-path flags are set once per part, so
    // a k-tile costs its DMAs and a k offset.  Block j of this loader sits
    // j NL 8 rows below its block 0, an offset the scalar operand carries.
    Cur ic = cc;
    const int sA0 = NL * 8 * lda0, sA1 = NL * 8 * lda1, sV = NL * 8 * kE, sR = NL * 8 * ldr;
    const uint32_t lq0 = ring_s + q * 1024;   // this loader's block 0 in slot 0
    int p_kind = 0, p_left = 0, p_kb = 0, p_kbytes = 0, p_alo = 0, p_ahi = 0, p_ib = 0;
    int p_fa = 0, p_fb = 0, p_live = 0;   // ints, not bools: kept in registers
    int p_av = a_v0, p_sa = sA0;          // the part's A row offset and block step
    i32x4v p_ars, p_brs, p_rsb;
    auto set_tv = [&]() __attribute__((always_inline)) {
      p_live = ic.t < hi_tile ? 1 : 0;
      p_kind = 0; p_left = nk0; p_kb = 0; p_kbytes = kE; p_ib = ic.b0;
      p_av = a_v0; p_sa = sA0;
      p_ars = rsrc_words(reinterpret_cast<const char*>(A0) + (int64_t)ic.m0 * lda0 +
                             (acolb ? (int64_t)(ic.n0 / acolb) * kE : 0), 0x7fffffffu);
      p_brs = rsrc_words(reinterpret_cast<const char*>(Vt) + (int64_t)ic.n0 * kE, 0x7fffffffu);
      p_rsb = rsrc_words(bias + ic.n0, HAS_BIAS && p_live ? (uint32_t)(c2 - ic.n0) * 2u : 0u);
      p_alo = -ic.m0; p_ahi = n - ic.m0;
      p_fa = p_live && p_ahi >= C::BM ? 1 : 0;
      p_fb = p_live && ic.n0 + C::BN <= c2 ? 1 : 0;
    };
    auto set_lr = [&](int ibx) __attribute__((always_inline)) {
      p_kind = 1; p_left = nkr; p_kb = 0; p_kbytes = rE; p_ib = ibx;
      p_av = a_v1; p_sa = sA1;
      p_ars = rsrc_words(reinterpret_cast<const char*>(A1) + (int64_t)ic.m0 * lda1, 0x7fffffffu);
      p_brs = rsrc_words(reinterpret_cast<const char*>(Rt) + (int64_t)ibx * rE + (int64_t)ic.n0 * ldr, 0x7fffffffu);
      p_alo = (int)sg.lo(ibx) - ic.m0; p_ahi = (int)sg.hi(ibx) - ic.m0;
      p_fa = p_live && p_alo <= 0 && p_ahi >= C::BM ? 1 : 0;
    };
    // a tile's first part: [T | V], or with no static part (k = 0) its
    // first segment's [L_b | R_b] (the bias descriptor comes from set_tv)
    auto begin_tile = [&]() __attribute__((always_inline)) {
      set_tv();
      if (nk0 == 0) set_lr(ic.b0);
    };
    begin_tile();
    // one k-tile into the slot at byte offset `slot`; past the last tile
    // every lane reads out of range, so the DMA count (and with it every
    // wait) stays the same at each step
    auto issue = [&](uint32_t slot) __attribute__((always_inline)) {
      const uint32_t lb = lq0 + slot;
      const bool fullk = p_kb + 128 <= p_kbytes;
      const bool kok = ch16 < p_kbytes - p_kb;
      // interior parts take the branch without any per-lane test
      if (p_fa && fullk) {
        static_for<0, LA>([&](auto jc) __attribute__((always_inline)) {
          constexpr int j = decltype(jc)::value;
          dma16k<j * NL * 1024>(p_ars, p_av, p_kb + j * p_sa, lb);
        });
      } else {
        static_for<0, LA>([&](auto jc) __attribute__((always_inline)) {
          constexpr int j = decltype(jc)::value;
          const int rr = row0 + j * NL * 8;
          const int v = p_live && kok && rr >= p_alo && rr < p_ahi ? p_av : (int)0x80000000u;
          dma16k<j * NL * 1024>(p_ars, v, p_kb + j * p_sa, lb);
        });
      }
      auto bdmas = [&](int vb, int sb) __attribute__((always_inline)) {
        if (p_fb && fullk) {
          static_for<0, LB>([&](auto jc) __attribute__((always_inline)) {
            constexpr int j = decltype(jc)::value;
            dma16k<C::BM * 128 + j * NL * 1024>(p_brs, vb, p_kb + j * sb, lb);
          });
        } else {
          static_for<0, LB>([&](auto jc) __attribute__((always_inline)) {
            constexpr int j = decltype(jc)::value;
            const int v = p_live && kok && ic.n0 + row0 + j * NL * 8 < c2 ? vb : (int)0x80000000u;
            dma16k<C::BM * 128 + j * NL * 1024>(p_brs, v, p_kb + j * sb, lb);
          });
        }
      };
      if (p_kind == 0) bdmas(v_v, sV);
      else bdmas(r_v, sR);
      // the tile's bias into the slot tail (every loader writes the same bytes)
      dma4(p_rsb, lane * 4, 0, ring_s + slot + C::STAGE);
      if (p_live) {
        p_kb += 128;
        if (--p_left == 0) {
          if (p_kind == 0 && nkr > 0) set_lr(ic.b0);
          else if (p_kind == 1 && p_ib < ic.bl) set_lr(p_ib + 1);
          else {
            // the tile's last part (with no residual part, r = 0: its
            // [T | V] part), so the next part is the next tile's first
            advance(ic);
            begin_tile();
          }
        }
      }
    };
    uint32_t slot_i = 0;
#pragma unroll
    for (int s = 0; s < NS - 1; ++s) {
      issue(slot_i);
      slot_i += SLOT;
    }
    while (live) {
      wait_vm_lgkm0<(NS - 2) * PTL>();   // this loader's part of k-tile t has landed
      bare_barrier();                     // ... everyone's; slot t - 1 is free again
      issue(slot_i);
      slot_i = slot_i + SLOT == RING ? 0u : slot_i + SLOT;
      if (++ckt == cc.tot) {
        bare_barrier();                   // the compute waves' epilogue barrier
        advance(cc);
        ckt = 0;
        live = cc.t < hi_tile;
      }
    }
    wait_vm_lgkm0<0>();                   // no DMA may still be writing LDS at exit
    return;
  }
  // ------------------------------- compute -------------------------------
  const int wm = w / C::NWN, wn = w % C::NWN;
  const int h = (l >> 1) & 7;
  f32x16 acc[C::FM][C::FN];
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[fm][fn][v] = 0.f;
  // acc (+)= one k-tile of the slot.  Lane (l, g) reads chunk 2 ks + g of
  // rows l + 32 f, whose swizzled position depends on l only; substep ks + 1
  // is read while ks runs.  FIRST: the first MFMA of each block adds the bias
  // tuple instead of acc.
  auto compute = [&](const char* stage, auto first, const f32x16 (&cinit)[C::FN]) {
    constexpr bool FIRST = decltype(first)::value;
    const char* as = stage + (wm * C::WM + l) * 128;
    const char* bs = stage + C::BM * 128 + (wn * C::WN + l) * 128;
    uint4 af[2][C::FM], bfr[2][C::FN];
    auto load = [&](int ks, int buf) {
      const int co = (((2 * ks + gq) ^ h) & 7) << 4;
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm) af[buf][fm] = *reinterpret_cast<const uint4*>(as + fm * 4096 + co);
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn) bfr[buf][fn] = *reinterpret_cast<const uint4*>(bs + fn * 4096 + co);
    };
    load(0, 0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks + 1 < 4) load(ks + 1, (ks + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8_t, bfr[ks & 1][fn]), __builtin_bit_cast(bf16x8_t, af[ks & 1][fm]),
              (FIRST && ks == 0) ? cinit[fn] : acc[fm][fn], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  uint32_t slot_c = 0;
  while (live) {
    wait_lgkm0();
    bare_barrier();
    const char* stage = ring + slot_c;
    if (HAS_BIAS && ckt == 0) {
      f32x16 cinit[C::FN];
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const uint2 b2 = *reinterpret_cast<const uint2*>(stage + C::STAGE + (wn * C::WN + fn * 32 + 8 * qq + 4 * gq) * 2);
          cinit[fn][4 * qq + 0] = __uint_as_float(b2.x << 16);
          cinit[fn][4 * qq + 1] = __uint_as_float(b2.x & 0xffff0000u);
          cinit[fn][4 * qq + 2] = __uint_as_float(b2.y << 16);
          cinit[fn][4 * qq + 3] = __uint_as_float(b2.y & 0xffff0000u);
        }
      compute(stage, std::true_type(), cinit);
    } else {
      compute(stage, std::false_type(), acc[0]);
    }
    if (++ckt == cc.tot) {
      char* st = ring + slot_c;
      const int rows_valid = min(C::BM, n - cc.m0);
      const int colbytes = min(C::BN * 2, (c2 - cc.n0) * 2);
      const __amdgpu_buffer_rsrc_t yrs = __builtin_amdgcn_make_buffer_rsrc(
          reinterpret_cast<char*>(Y) + ((int64_t)cc.m0 * c2 + cc.n0) * 2, (short)0, 0x7fffffff, 0x00020000);
      const int ldy = c2 * 2;
      wait_lgkm0();
      bare_barrier();                     // every compute wave is done reading slot t
      char* wa = st + w * WAREA;
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm) {
        // rows l of this 32-row block: chunk c of row l at ((c ^ l / 2) % 8),
        // which spreads the 8-byte writes of the 32 rows over the bank window
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            const int col = fn * 32 + 8 * qq + 4 * gq;
            uint2 pk;
            pk.x = pack_bf16x2(acc[fm][fn][4 * qq + 0], acc[fm][fn][4 * qq + 1]);
            pk.y = pack_bf16x2(acc[fm][fn][4 * qq + 2], acc[fm][fn][4 * qq + 3]);
            *reinterpret_cast<uint2*>(wa + l * RB + (((col >> 3) ^ (l >> 1)) & 7) * 16 + (col & 4) * 2) = pk;
          }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int i = 0; i < 32 * 8 / 64; ++i) {
          const int c = lane + i * 64;
          const int rr = c >> 3, ch = c & 7;
          const uint4 v = *reinterpret_cast<const uint4*>(wa + rr * RB + ((ch ^ (rr >> 1)) & 7) * 16);
          const int row = wm * C::WM + fm * 32 + rr;
          const bool ok = row < rows_valid && wn * C::WN * 2 + ch * 16 < colbytes;
          const int off = ok ? row * ldy + wn * C::WN * 2 + ch * 16 : (int)0x80000000u;
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4v, v), yrs, off, 0, 2);   // nt
        }
        __builtin_amdgcn_wave_barrier();
      }
      if constexpr (!HAS_BIAS) {
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
          for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[fm][fn][v] = 0.f;
      }
      advance(cc);
      ckt = 0;
      live = cc.t < hi_tile;
    }
    slot_c = slot_c + SLOT == RING ? 0u : slot_c + SLOT;
  }
}

// ===========================================================================
// Left ALS step (t > 1): L_b = X_b W_res R_b^T (R_b R_b^T + lambda I)^-1.
// The thin products R_b R_b^T and R_b W_res^T come from the token-reduction
// kernel in relative addressing (R_b's rows as "L^T", W_res^T as "X",
// c2 playing the token axis); the inverse is applied by apply_inverse_kernel
// (Z_b^T = (K_b + lambda I)^-1 Q_b^T); then L_b = X_b Z_b here.
// ===========================================================================

// out [cols x rows] = in [rows x cols]^T, 16-bit elements, 64 x 64 tiles
// through LDS (the padded pitch keeps the column reads off one bank).
__global__ __launch_bounds__(256) void transpose_b16_kernel(const bf16_t* __restrict__ in, bf16_t* __restrict__ out,
                                                            int64_t rows, int64_t cols) {
  __shared__ bf16_t tile[64][66];
  const int64_t tiles_c = (cols + 63) / 64;
  const int64_t r0 = (int64_t)(blockIdx.x / tiles_c) * 64, c0 = (int64_t)(blockIdx.x % tiles_c) * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int y = ty; y < 64; y += 4) {
    const int64_t rr = r0 + y, cc = c0 + tx;
    tile[y][tx] = (rr < rows && cc < cols) ? in[rr * cols + cc] : (bf16_t)0;
  }
  __syncthreads();
  for (int y = ty; y < 64; y += 4) {
    const int64_t oc = c0 + y, orr = r0 + tx;   // out row oc, column orr
    if (oc < cols && orr < rows) out[oc * rows + orr] = tile[tx][y];
  }
}

// out (cols x rows, row pitch ldo) = in (rows x cols, row pitch ldi)^T for
// 32-bit elements, 64 x 64 tiles through LDS (the padded pitch keeps the
// column reads off one bank).
__global__ __launch_bounds__(256) void transpose_b32_kernel(const float* __restrict__ in, int64_t ldi,
                                                            float* __restrict__ out, int64_t ldo, int64_t rows,
                                                            int64_t cols) {
  __shared__ float tile[64][65];
  const int64_t tiles_c = (cols + 63) / 64;
  const int64_t r0 = (int64_t)(blockIdx.x / tiles_c) * 64, c0 = (int64_t)(blockIdx.x % tiles_c) * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int y = ty; y < 64; y += 4) {
    const int64_t rr = r0 + y, cc = c0 + tx;
    tile[y][tx] = (rr < rows && cc < cols) ? in[rr * ldi + cc] : 0.f;
  }
  __syncthreads();
  for (int y = ty; y < 64; y += 4) {
    const int64_t oc = c0 + y, orr = r0 + tx;   // out row oc, column orr
    if (oc < cols && orr < rows) out[oc * ldo + orr] = tile[tx][y];
  }
}

// L_b = X_b Z_b for every segment: out [n x r] at TL columns k .. k + r - 1
// (pitch ldo) and L^T.  Zt: [B r x c1] (Z_b^T, row-major).  A tile whose rows
// span several segments (uniform or ragged, sg) accumulates one k-loop per
// segment with the rows of the others masked off.
template <class C>
__global__ __launch_bounds__(C::NT) void s1_left_kernel(const bf16_t* X, const bf16_t* Zt, bf16_t* TL, bf16_t* Lt,
                                                        int64_t n, int64_t c1, int k, int r, SegMap sg,
                                                        int64_t ldt, int tiles_n, int64_t ldo) {
  constexpr int E = 2, KPC = 8;
  __shared__ __attribute__((aligned(16))) char lds[C::LDS];
  const int t = xcd_tile_id(blockIdx.x, gridDim.x);
  const int64_t m0 = (int64_t)(t / tiles_n) * C::BM, n0 = (int64_t)(t % tiles_n) * C::BN;
  const int64_t bfirst = sg.of(m0);
  const int64_t blast = sg.of(imin64(m0 + C::BM, n) - 1);
  const int nkc = ktiles(c1 * E);
  const int total = (int)(blast - bfirst + 1) * nkc;
  auto src = [=](int tt, Phase& ph, int& kt) {
    const int64_t b = bfirst + tt / nkc;
    kt = tt % nkc;
    ph.a = OpK{reinterpret_cast<const char*>(X), c1 * E, m0, sg.lo(b), sg.hi(b), c1 * E};
    ph.b = OpK{reinterpret_cast<const char*>(Zt + b * r * c1), c1 * E, n0, 0, r, c1 * E};
  };
  f32x16 acc[C::FM][C::FN];
  gemm_mainloop<C>(src, total, lds, acc);
  stage_out<C>(lds, acc, nullptr, 0);
  copy_out<C>(lds, reinterpret_cast<char*>(TL) + (m0 * ldo + k + n0) * E, ldo * E, (int)imin64(C::BM, n - m0),
              (r - n0) * E);
  // the same columns, transposed: Lt[j][m0 + rows]
  const int ncol = (int)imin64(C::BN, r - n0);
  const int groups = C::BM / KPC;
  for (int c = threadIdx.x; c < ncol * groups; c += C::NT) {
    const int jl = c / groups, rg = c % groups;
    const int64_t row = m0 + (int64_t)rg * KPC;
    if (row >= ldt) continue;
    bf16_t v[KPC];
#pragma unroll
    for (int e = 0; e < KPC; ++e) v[e] = staged_elem<C>(lds, rg * KPC + e, jl);
    *reinterpret_cast<uint4*>(Lt + (n0 + jl) * ldt + row) = *reinterpret_cast<const uint4*>(v);
  }
}

// ===========================================================================
// Monarch static branch (m = 32 blocks of 32 x 32, c = 1024), bf16.
// W_hat = blockdiag(B1_a) . Pi . blockdiag(B2_j), Pi the reshape(32, 32)
// transpose: u_a = x_a B1_a, v[j*32 + a] = u[a*32 + j], y_j = v_j B2_j.
// The block products are tiny: both kernels are bound by streaming X and Y
// and by load latency, so X is loaded for a whole row block at once, weights
// come in fragment order a few products ahead, and Y leaves as whole rows.
// ===========================================================================

constexpr int MO = 32;

// First stage (L only): one pass over X.  A workgroup owns 32 rows; wave w
// takes the 8 blocks a = 8w .. 8w + 7 and accumulates its K slice
// (a*32 .. a*32 + 31 for its 8 blocks) of L = X P; the output kernel
// recomputes the Monarch stage 1 from X, so V is never stored.  Pt is in
// fragment order: a wave's operand of one MFMA step is one contiguous 1 KB
// run.  The four partial L sums are added through LDS in a fixed order;
// wave 0 writes L and L^T.
constexpr int S1M_VP = MO * MO * 2 + 16;                  // V row pitch in LDS (bytes), output kernel
template <int RB>
__global__ __launch_bounds__(256, 2) void s1_monarch_kernel(const bf16_t* __restrict__ X,
                                                         const bf16_t* __restrict__ Pt,
                                                         bf16_t* __restrict__ A, bf16_t* __restrict__ Lt,
                                                         int64_t n, int r, int64_t ldt) {
  constexpr int C = MO * MO;
  __shared__ __attribute__((aligned(16))) float part[3 * RB * 16 * 64];   // waves 1..3's partial L
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int l = lane & 31, g = lane >> 5;
  const int64_t row = (int64_t)blockIdx.x * 32 + l;
  const bool rok = row < n;
  const int64_t lda = C + r;
  f32x16 lacc[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int v = 0; v < 16; ++v) lacc[rb][v] = 0.f;
  // one (block, k step) at a time: at about 130 registers three workgroups
  // share a CU, which hides the X loads better than issuing the row block's
  // sixteen loads up front at two (measured 35 against 40-53 us)
#pragma unroll
  for (int ai = 0; ai < 8; ++ai) {
    const int a = w * 8 + ai;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int kk = a * MO + 16 * s + 8 * g;
      const uint4 xa = rok ? *reinterpret_cast<const uint4*>(X + row * C + kk) : zero4();
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int p = rb * 32 + l;
        const uint4 pb =
            p < r ? *reinterpret_cast<const uint4*>(Pt + ((int64_t)((rb * MO + a) * 2 + s) * 64 + lane) * 8) : zero4();
        TT<bf16_t>::mma(lacc[rb], pb, xa);
      }
    }
  }
  // L partials: waves 1..3 -> LDS, wave 0 adds them in order
  if (w > 0) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int v = 0; v < 16; ++v) part[(((w - 1) * RB + rb) * 16 + v) * 64 + lane] = lacc[rb][v];
  }
  __syncthreads();
  if (w != 0 || !rok) return;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int v = 0; v < 16; ++v)
      lacc[rb][v] = ((lacc[rb][v] + part[((0 * RB + rb) * 16 + v) * 64 + lane]) + part[((1 * RB + rb) * 16 + v) * 64 + lane]) +
                    part[((2 * RB + rb) * 16 + v) * 64 + lane];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int p0 = rb * 32 + 8 * q + 4 * g;
      if (p0 >= r) continue;
      const float v[4] = {lacc[rb][4 * q], lacc[rb][4 * q + 1], lacc[rb][4 * q + 2], lacc[rb][4 * q + 3]};
      uint2 pk;
      pk.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
      pk.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
      *reinterpret_cast<uint2*>(A + row * lda + C + p0) = pk;
#pragma unroll
      for (int e = 0; e < 4; ++e) Lt[(int64_t)(p0 + e) * ldt + row] = f2bf(v[e]);
    }
}

// One-pass Monarch output: a workgroup owns 32 rows and all 1024 output
// columns, and recomputes stage 1 from X instead of reading a stored V.
//   phase 1: wave w forms U_a = x_a B1_a for a = 8w .. 8w + 7 (as the first
//            stage does) and writes the permuted V[row][j*32 + a] into an LDS
//            copy of the 32 V rows;
//   phase 2: wave w forms y_j = V_j B2_j + L R_b[:, j] for j = 8w .. 8w + 7,
//            V_j from LDS (bytes 512 w .. 512 w + 511 of each row: the
//            wave's own slice, so it then stages its output rows there
//            without a workgroup barrier), B2t and R^T rows straight from L2
//            (each lane's 16-byte runs of one 128-byte line are read by the
//            same wave in consecutive k steps);
//   store:   the bias is added on packing, and every store instruction
//            writes two whole 512-byte row slices.
// X is read once here and once by the first stage (L only), V never touches
// HBM.
__global__ __launch_bounds__(256, 2) void s6_monarch_fused_kernel(const bf16_t* __restrict__ X,
                                                               const bf16_t* __restrict__ B1t,
                                                               const bf16_t* __restrict__ B2t,
                                                               const bf16_t* __restrict__ A,
                                                               const bf16_t* __restrict__ Rt,
                                                               const bf16_t* __restrict__ bias,
                                                               bf16_t* __restrict__ Y, int64_t n, int r, SegMap sg,
                                                               int64_t B) {
  constexpr int C = MO * MO;
  __shared__ __attribute__((aligned(16))) char sm[32 * S1M_VP];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int l = lane & 31, g = lane >> 5;
  const int64_t m0 = (int64_t)blockIdx.x * 32;
  const int64_t row = m0 + l;
  const bool rok = row < n;
  const int64_t lda = C + r;
  f32x16 acc[8];
  // ---- phase 1: U_a for the wave's 8 blocks, permuted into LDS ----
  // All 16 X loads are issued before the first product (rows past n read
  // row n - 1 and are zeroed afterwards), so a wave waits on HBM once.
  const int64_t rowc = rok ? row : n - 1;
  uint4 xa[8][2];
#pragma unroll
  for (int ai = 0; ai < 8; ++ai)
#pragma unroll
    for (int s = 0; s < 2; ++s)
      xa[ai][s] = *reinterpret_cast<const uint4*>(X + rowc * C + (w * 8 + ai) * MO + 16 * s + 8 * g);
  // B1t fragments (L2-resident) stream four products ahead of the MFMAs
  auto ld_b1 = [&](int q) {   // q = 2 ai + s
    return *reinterpret_cast<const uint4*>(B1t + (((w * 8 + (q >> 1)) * 2 + (q & 1)) * 64 + lane) * 8);
  };
  uint4 bq[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) bq[q] = ld_b1(q);
#pragma unroll
  for (int ai = 0; ai < 8; ++ai)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[ai][v] = 0.f;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const uint4 cur = bq[q & 3];
    if (q + 4 < 16) bq[q & 3] = ld_b1(q + 4);
    TT<bf16_t>::mma(acc[q >> 1], cur, rok ? xa[q >> 1][q & 1] : zero4());
  }
  // lane holds U[row][a*32 + j] for j = 8q + 4g + e (reg 4q + e), a = 8w + ai
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = 8 * q + 4 * g + e;
      uint32_t pk[4];
#pragma unroll
      for (int h = 0; h < 4; ++h)
        pk[h] = (uint32_t)f2bf(acc[2 * h][4 * q + e]) | ((uint32_t)f2bf(acc[2 * h + 1][4 * q + e]) << 16);
      *reinterpret_cast<uint4*>(sm + l * S1M_VP + (j * MO + w * 8) * 2) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    }
  __syncthreads();
  // ---- phase 2: y_j = V_j B2_j (K = 32: two 16-wide k steps); the B2t
  // loads of all 8 blocks are issued first ----
  uint4 b2[8][2];
#pragma unroll
  for (int jj = 0; jj < 8; ++jj)
#pragma unroll
    for (int s = 0; s < 2; ++s)
      b2[jj][s] = *reinterpret_cast<const uint4*>(B2t + ((int64_t)((w * 8 + jj) * MO + l) * MO + 16 * s + 8 * g));
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[jj][v] = 0.f;
    const int j = w * 8 + jj;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const uint4 va = *reinterpret_cast<const uint4*>(sm + l * S1M_VP + (j * MO + 16 * s + 8 * g) * 2);
      TT<bf16_t>::mma(acc[jj], b2[jj][s], va);
    }
  }
  // + L R_b for every segment meeting the 32 rows
  const int64_t mend = imin64(m0 + 32, n);
  const int64_t bf = sg.of(imin64(m0, n - 1)), bl = imin64(B - 1, sg.of(mend - 1));
  const int64_t ldr = B * r;
  for (int64_t b = bf; b <= bl; ++b) {
    const int64_t blo = sg.lo(b), bhi = sg.hi(b);
    const bool in = rok && row >= blo && row < bhi;
    // r % 16 == 0 (r a multiple of 8 split over the two lane halves is not
    // enough: a k step past r reads a clamped column and is zeroed)
    for (int k0 = 0; k0 < r; k0 += 16) {
      const int kk = k0 + 8 * g;
      const bool kok = kk < r;
      const int kc = kok ? kk : 0;
      uint4 rt[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj)
        rt[jj] = *reinterpret_cast<const uint4*>(Rt + (int64_t)((w * 8 + jj) * MO + l) * ldr + b * r + kc);
      uint4 la = *reinterpret_cast<const uint4*>(A + rowc * lda + C + kc);
      if (!(in && kok)) la = zero4();
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) TT<bf16_t>::mma(acc[jj], kok ? rt[jj] : zero4(), la);
    }
  }
  // ---- stage the wave's 32 x 256 output slice over its own V slice ----
  // accumulator (jj) element 4 q + e: row l, column 32 (8w + jj) + 8 q + 4 g + e
#pragma unroll
  for (int jj = 0; jj < 8; ++jj)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int cl = (w * 8 + jj) * MO + 8 * q + 4 * g;
      float v[4];
      if (bias) {
        const uint2 bb = *reinterpret_cast<const uint2*>(bias + cl);
        v[0] = acc[jj][4 * q] + __uint_as_float(bb.x << 16);
        v[1] = acc[jj][4 * q + 1] + __uint_as_float(bb.x & 0xffff0000u);
        v[2] = acc[jj][4 * q + 2] + __uint_as_float(bb.y << 16);
        v[3] = acc[jj][4 * q + 3] + __uint_as_float(bb.y & 0xffff0000u);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[jj][4 * q + e];
      }
      uint2 pk;
      pk.x = pack_bf16x2(v[0], v[1]);
      pk.y = pack_bf16x2(v[2], v[3]);
      *reinterpret_cast<uint2*>(sm + l * S1M_VP + cl * 2) = pk;
    }
  __builtin_amdgcn_wave_barrier();
  // 32 rows x 512 bytes: 32 lanes per row slice, two rows per store
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int rl = 2 * i + (lane >> 5), ch = lane & 31;
    const int64_t yr = m0 + rl;
    if (yr < n)
      *reinterpret_cast<uint4*>(Y + yr * C + w * 256 + ch * 8) =
          *reinterpret_cast<const uint4*>(sm + rl * S1M_VP + w * 512 + ch * 16);
  }
}

// ===========================================================================
// BLAST fused output: for output block column j (width b2 = c2 / nb), the
// static part is W'_j V_j^T with W' = Z S (the coupled block-row outputs),
// then the residual correction L R_b and the bias, as one phased GEMM.
// The tile width divides b2, so every tile lies inside one block column.
// ===========================================================================

// Diagonal couplings (DYRA_BLAST_DIAG): W'_j[t][p] = sum_i Z_i[t][p] s_ij[p]
// for every token t, output block j and p < rb, an elementwise weighted sum
// over the nb input blocks (2 n nb^2 rb flops, HBM bound: Z read once, W'
// written once).  A workgroup stages ZT token rows of Z in LDS; thread
// chunks of 8 outputs (16 bytes) walk the NR = nb rb outputs of each row.
// Sd: [nb (j)][nb (i)][rb]; fp32 accumulation, bf16 W'.
constexpr int BDC_LDS = 64 * 1024;
__global__ __launch_bounds__(256) void blast_diag_coupling_kernel(const bf16_t* __restrict__ Z, int64_t ldz,
                                                                  const bf16_t* __restrict__ Sd,
                                                                  bf16_t* __restrict__ Wp, int64_t ldw, int64_t n,
                                                                  int nb, int rb, int zt) {
  __shared__ __attribute__((aligned(16))) bf16_t zs[BDC_LDS / 2];
  const int NR = nb * rb, chunks = NR / 8, rc = rb / 8;
  for (int64_t t0 = (int64_t)blockIdx.x * zt; t0 < n; t0 += (int64_t)gridDim.x * zt) {
    const int rows = (int)imin64(zt, n - t0);
    __syncthreads();   // the previous rows are consumed
    for (int e = threadIdx.x; e < rows * chunks; e += 256) {
      const int row = e / chunks, c = e % chunks;
      *reinterpret_cast<uint4*>(zs + row * NR + 8 * c) =
          *reinterpret_cast<const uint4*>(Z + (t0 + row) * ldz + 8 * c);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < rows * chunks; e += 256) {
      const int row = e / chunks, c = e % chunks;
      const int j = c / rc, p8 = (c % rc) * 8;
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int i = 0; i < nb; ++i) {
        const uint4 zv = *reinterpret_cast<const uint4*>(zs + row * NR + i * rb + p8);
        const uint4 sv = *reinterpret_cast<const uint4*>(Sd + ((int64_t)j * nb + i) * rb + p8);
        const uint32_t zw[4] = {zv.x, zv.y, zv.z, zv.w}, sw[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          acc[2 * h] = fmaf(bf2f((bf16_t)(zw[h] & 0xffffu)), bf2f((bf16_t)(sw[h] & 0xffffu)), acc[2 * h]);
          acc[2 * h + 1] = fmaf(bf2f((bf16_t)(zw[h] >> 16)), bf2f((bf16_t)(sw[h] >> 16)), acc[2 * h + 1]);
        }
      }
      uint4 o;
      o.x = (uint32_t)f2bf(acc[0]) | ((uint32_t)f2bf(acc[1]) << 16);
      o.y = (uint32_t)f2bf(acc[2]) | ((uint32_t)f2bf(acc[3]) << 16);
      o.z = (uint32_t)f2bf(acc[4]) | ((uint32_t)f2bf(acc[5]) << 16);
      o.w = (uint32_t)f2bf(acc[6]) | ((uint32_t)f2bf(acc[7]) << 16);
      *reinterpret_cast<uint4*>(Wp + (t0 + row) * ldw + j * rb + p8) = o;
    }
  }
}

template <class C>
__global__ __launch_bounds__(C::NT) void s6_blast_kernel(const bf16_t* Wp, int64_t ldw, const bf16_t* ZL,
                                                         int64_t ldzl, int64_t loff, const bf16_t* Vb,
                                                         const bf16_t* Rt, const bf16_t* bias, bf16_t* Y,
                                                         int64_t n, int64_t c2, int64_t b2, int rb, int r,
                                                         SegMap sg, int64_t B, int tiles_n) {
  constexpr int E = 2;
  __shared__ __attribute__((aligned(16))) char lds[C::LDS];
  // column-major tile order, so that the contiguous tile range each XCD
  // takes is a band of output columns over all rows: its V_j and R^T rows,
  // and the W'_j and L rows of the few block columns j it meets, fit its L2
  // (row-major bands made every XCD stream all of V and R^T once per row
  // block: 9x the algorithmic read bytes at the LM BLAST shape)
  const int t = xcd_tile_id(blockIdx.x, gridDim.x);
  const int tiles_m = (int)(gridDim.x / tiles_n);
  const int64_t m0 = (int64_t)(t % tiles_m) * C::BM, n0 = (int64_t)(t / tiles_m) * C::BN;
  const int64_t j = n0 / b2;
  const int64_t bfirst = sg.of(m0);
  const int64_t blast = imin64(B - 1, sg.of(imin64(m0 + C::BM, n) - 1));
  const int nk0 = ktiles((int64_t)rb * E), nkr = ktiles((int64_t)r * E);
  const int total = nk0 + (int)(blast - bfirst + 1) * nkr;
  const char* Wpc = reinterpret_cast<const char*>(Wp + j * rb);
  const char* Vbc = reinterpret_cast<const char*>(Vb + j * b2 * rb);
  const char* Lc = reinterpret_cast<const char*>(ZL + loff);
  auto src = [=](int tt, Phase& ph, int& kt) {
    if (tt < nk0) {
      ph.a = OpK{Wpc, ldw * E, m0, 0, n, (int64_t)rb * E};
      ph.b = OpK{Vbc, (int64_t)rb * E, n0 - j * b2, 0, b2, (int64_t)rb * E};
      kt = tt;
      return;
    }
    const int u = tt - nk0;
    const int64_t b = bfirst + u / nkr;
    kt = u % nkr;
    ph.a = OpK{Lc, ldzl * E, m0, sg.lo(b), sg.hi(b), (int64_t)r * E};
    ph.b = OpK{reinterpret_cast<const char*>(Rt + b * r), B * r * E, n0, 0, c2, (int64_t)r * E};
  };
  f32x16 acc[C::FM][C::FN];
  gemm_mainloop<C>(src, total, lds, acc);
  stage_out<C>(lds, acc, bias ? bias + n0 : nullptr, (int)(c2 - n0));
  copy_out<C, true>(lds, reinterpret_cast<char*>(Y) + (m0 * c2 + n0) * E, c2 * E, (int)imin64(C::BM, n - m0),
              (c2 - n0) * E);
}

// ===========================================================================
// S3: M_b = L_b^T X_b (r x c1) and G_b = L_b^T L_b (r x r), fp32 outputs.
// The reduction runs over the tokens of one segment inside one workgroup
// (no atomics, fixed order), double-buffered through LDS.  X arrives
// token-major, so its tiles are transposed on the way into LDS.
// ===========================================================================

template <class C>
__global__ __launch_bounds__(C::NT) void s3_gram_kernel(const typename C::elem* Lt, int64_t ldt,
                                                        const typename C::elem* X, int64_t c1, int r,
                                                        SegMap sg, int64_t n, float* M, float* G,
                                                        int tiles_r, int tiles_cm, int tiles_cg) {
  typedef typename C::elem T;
  constexpr int E = TT<T>::ESZ, KPC = TT<T>::KPC, BKE = 8 * KPC;
  constexpr int XCH = C::BN / KPC;   // chunks per token row of an X tile
  static_assert(C::BCH * C::NT == BKE * XCH, "X tile chunks");
  __shared__ __attribute__((aligned(16))) char lds[C::LDS];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w / C::NWN, wn = w % C::NWN;
  const int per_seg = tiles_r * (tiles_cm + tiles_cg);
  const int t = blockIdx.x;
  const int64_t b = t / per_seg;
  const int rem = t % per_seg;
  const int tr = rem / (tiles_cm + tiles_cg), tc = rem % (tiles_cm + tiles_cg);
  const bool is_g = tc >= tiles_cm;
  const int p0 = tr * C::BM;
  const int64_t c0 = (int64_t)(is_g ? tc - tiles_cm : tc) * C::BN;
  const int64_t lo = sg.lo(b), hi = sg.hi(b);
  const int64_t kt0 = lo / BKE, kt1 = (hi + BKE - 1) / BKE;

  f32x16 acc[C::FM][C::FN];
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[fm][fn][v] = 0.f;

  uint4 ra[C::ACH], rb[C::BCH];
  auto load = [&](int64_t kt) {
    const int64_t tb = kt * BKE;
#pragma unroll
    for (int i = 0; i < C::ACH; ++i) {
      const int c = tid + i * C::NT;
      const int row = c >> 3, ch = c & 7;
      const int64_t t0 = tb + ch * KPC;
      uint4 v = zero4();
      if (p0 + row < r && t0 < ldt) v = *reinterpret_cast<const uint4*>(Lt + (p0 + row) * ldt + t0);
      ra[i] = mask_tokens<T>(v, t0, lo, hi);
    }
#pragma unroll
    for (int i = 0; i < C::BCH; ++i) {
      const int c = tid + i * C::NT;
      uint4 v = zero4();
      if (is_g) {
        const int row = c >> 3, ch = c & 7;
        const int64_t t0 = tb + ch * KPC;
        if (c0 + row < r && t0 < ldt) v = *reinterpret_cast<const uint4*>(Lt + (c0 + row) * ldt + t0);
        v = mask_tokens<T>(v, t0, lo, hi);
      } else {
        const int tok = c / XCH, cc = c % XCH;
        const int64_t tt = tb + tok, col = c0 + (int64_t)cc * KPC;
        if (tt >= lo && tt < hi && col < c1) v = *reinterpret_cast<const uint4*>(X + tt * c1 + col);
      }
      rb[i] = v;
    }
  };
  auto store = [&](char* stage) {
#pragma unroll
    for (int i = 0; i < C::ACH; ++i) {
      const int c = tid + i * C::NT;
      *reinterpret_cast<uint4*>(stage + lds_off(c >> 3, c & 7)) = ra[i];
    }
    char* bs = stage + C::BM * 128;
#pragma unroll
    for (int i = 0; i < C::BCH; ++i) {
      const int c = tid + i * C::NT;
      if (is_g) {
        *reinterpret_cast<uint4*>(bs + lds_off(c >> 3, c & 7)) = rb[i];
      } else {
        // token tok, channels cc*KPC .. +KPC-1  ->  rows (channels), column tok
        const int tok = c / XCH, cc = c % XCH;
        const T* v = reinterpret_cast<const T*>(&rb[i]);
#pragma unroll
        for (int e = 0; e < KPC; ++e) {
          const int nrow = cc * KPC + e;
          *reinterpret_cast<T*>(bs + lds_off(nrow, tok / KPC) + (tok % KPC) * E) = v[e];
        }
      }
    }
  };

  if (kt0 < kt1) {
    load(kt0);
    store(lds);
    __syncthreads();
    int it = 0;
    for (int64_t kt = kt0; kt < kt1; ++kt, ++it) {
      const bool more = kt + 1 < kt1;
      if (more) load(kt + 1);
      compute_tile<C>(lds + (it & 1) * C::STAGE, acc, lane, wm, wn);
      if (!more) break;
      store(lds + ((it + 1) & 1) * C::STAGE);
      __syncthreads();
    }
  }
  // write fp32 results (lane: one output row, 4 consecutive columns per q)
  const int l = lane & 31, g = lane >> 5;
  const int64_t ncols = is_g ? r : c1;
  float* out = is_g ? G + b * r * r : M + b * r * c1;
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm) {
    const int p = p0 + wm * C::WM + fm * 32 + l;
    if (p >= r) continue;
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t col = c0 + wn * C::WN + fn * 32 + 8 * q + 4 * g;
        if (col < ncols)
          *reinterpret_cast<float4*>(out + p * ncols + col) =
              make_float4(acc[fm][fn][4 * q], acc[fm][fn][4 * q + 1], acc[fm][fn][4 * q + 2],
                          acc[fm][fn][4 * q + 3]);
      }
  }
}

// ===========================================================================
// block reductions
// ===========================================================================

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <int NT>
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) s += red[i];
  return s;
}

// ===========================================================================
// S4a: (G + lambda I)^-1 by the symmetric sweep operator, SW_BK pivots at a
// time.  Sweeping an index block K of a symmetric A gives
//   A'_KK = -A_KK^-1,  A'_KJ = A_KK^-1 A_KJ,  A'_JJ = A_JJ - A_JK A_KK^-1 A_KJ
// (J: the other indices), i.e. a'_ij = [i, j not in K] a_ij - (C A_KK^-1 C^T)_ij
// with C = A_{:,K} whose rows in K are replaced by -I.  Sweeping every block
// in turn leaves -(G + lambda I)^-1, the same operator as one pivot at a time
// (the sweep is order independent) with one barrier per block instead of per
// pivot.  Thread t owns a TB x TB tile of A.  The pivot rows of a block (its
// columns, by symmetry) are broadcast through LDS, double-buffered; every
// thread inverts the SW_BK x SW_BK pivot block itself by sweeping its pivots
// one by one.  A pivot <= 0 (or not finite) marks the matrix as not positive
// definite.
// ===========================================================================

constexpr int SW_BK = 4;
struct SweepLds {
  double pv[2][SW_BK][128];
  double diag0[128];   // diagonal of G before the ridge (rank test at eps = 0)
  float red[16];
};

// A solve whose smallest relative pivot d_j / A_jj (A = G + lambda I) falls
// below this is applied in fp64 (near-singular A: Ginv's entries of order
// 1 / lambda cancel in Ginv M).
constexpr double kWidePivot = 1.0 / 32.0;

// eps = 0 (no ridge): a pivot d_j at or below 2^-16 times the diagonal G_jj
// (sin^2 of the angle between column j of L and the span of the earlier
// columns) marks G as singular: status NOT_SPD and R_b = 0.  With a ridge,
// only a non-positive or non-finite pivot does.
constexpr double kSingularPivotRel = 1.0 / 65536.0;

// 1 / D for D > 0: hardware reciprocal estimate refined by two Newton steps
// (x <- x + x (1 - D x)), which reach full double precision.
__device__ __forceinline__ double recip_pos(double D) {
  double x = __builtin_amdgcn_rcp(D);
  double e = fma(-D, x, 1.0);
  x = fma(x, e, x);
  e = fma(-D, x, 1.0);
  return fma(x, e, x);
}

// 1 / D for D > 0 in fp32: the hardware reciprocal (1 ulp) and one Newton step.
__device__ __forceinline__ float recip_pos(float D) {
  const float x = __builtin_amdgcn_rcpf(D);
  return fmaf(x, fmaf(-D, x, 1.f), x);
}
template <typename S> struct SwPair;
template <> struct SwPair<double> {
  using T = double2;
  static __device__ __forceinline__ T make(double a, double b) { return make_double2(a, b); }
};
template <> struct SwPair<float> {
  using T = float2;
  static __device__ __forceinline__ T make(float a, float b) { return make_float2(a, b); }
};
// Returned by the fp32 pass (S = float, PASS32) when the segment needs the
// fp64 sweep: a relative pivot below kWidePivot, or any pivot failure.
constexpr int kSweepRedo64 = -1;

// Gb: r x r row-major fp32 (global or LDS); Ob: r x r row-major fp64,
// receives the inverse (zeros unless the status is OK).  S is the
// arithmetic: fp64, since the ridge bounds cond(G + lambda I) only by about
// r / eps (~1e8 for eps = 1e-6), past what fp32 elimination survives; or fp32
// for the first pass of sweep_inverse_mixed (PASS32), which stops at the
// first relative pivot below kWidePivot (or any pivot failure), writes
// nothing and returns kSweepRedo64.  Needs r % SW_BK == 0, r <= 128 and
// ceil(r / TB)^2 <= NT.  Returns the status (same in every thread).
template <int NT, int TB, int TBJ = TB, typename S = double, bool PASS32 = false>
__device__ __forceinline__ int sweep_inverse(const float* Gb, double* Ob, float* Ob32, int r, float eps,
                                             SweepLds& sh, bool& wide) {
  static_assert(!PASS32 || sizeof(S) == 4, "the stopping pass is the fp32 one");
  using P2 = SwPair<S>;
  using V2 = typename P2::T;
  // the pivot-row buffers hold S values (fp32 uses the first half)
  S(*pvs)[SW_BK][128] = reinterpret_cast<S(*)[SW_BK][128]>(&sh.pv[0][0][0]);
  // thread tiles of TB rows x TBJ columns
  static_assert(TB % SW_BK == 0 && TB % 2 == 0 && TBJ % SW_BK == 0 && TBJ % 2 == 0, "tile");
  const int tid = threadIdx.x;
  const int tpr = (r + TBJ - 1) / TBJ;
  const int i0 = (tid / tpr) * TB, j0 = (tid % tpr) * TBJ;
  const bool own = i0 < r;
  S a[TB][TBJ];
  float trf = 0.f;
#pragma unroll
  for (int x = 0; x < TB; ++x)
#pragma unroll
    for (int y = 0; y < TBJ; ++y) {
      const bool v = own && i0 + x < r && j0 + y < r;
      const float g = v ? Gb[(i0 + x) * r + j0 + y] : 0.f;
      a[x][y] = g;
      if (v && x + i0 == y + j0) {
        trf += g;
        sh.diag0[i0 + x] = g;
      }
    }
  const float tr = block_sum<NT>(trf, sh.red);   // its barriers also publish diag0
  int st = DYRA_SOLVE_OK;
  if (tr == 0.f) st = DYRA_SOLVE_ZERO;
  else if (!(tr > 0.f) || !isfinite(tr)) st = DYRA_SOLVE_NOT_SPD;
  // rows k0 .. k0 + SW_BK - 1 of this tile (if it holds them) -> pv[buf]
  auto publish_row = [&](int x, int k0, int buf) {
    const int i = i0 + x;
    if (own && i >= k0 && i < k0 + SW_BK) {
#pragma unroll
      for (int y = 0; y < TBJ; y += 2)
        if (j0 + y < r)
          *reinterpret_cast<V2*>(&pvs[buf][i - k0][j0 + y]) = P2::make(a[x][y], a[x][y + 1]);
    }
  };
  wide = false;
  if (st == DYRA_SOLVE_OK) {
    const S lam = (S)(eps * tr / (float)r);
#pragma unroll
    for (int x = 0; x < TB; ++x)
#pragma unroll
      for (int y = 0; y < TBJ; ++y)
        if (own && x + i0 == y + j0) a[x][y] += lam;
#pragma unroll
    for (int x = 0; x < TB; ++x) publish_row(x, 0, 0);
    __syncthreads();
    for (int kb = 0, blk = 0; kb < r; kb += SW_BK, ++blk) {
      const S(*buf)[128] = pvs[blk & 1];
      // Q <- -A_KK^-1 by sweeping the pivot block's own pivots
      S Q[SW_BK][SW_BK];
#pragma unroll
      for (int x = 0; x < SW_BK; ++x)
#pragma unroll
        for (int y = 0; y < SW_BK; y += 2) {
          const V2 v = *reinterpret_cast<const V2*>(&buf[x][kb + y]);
          Q[x][y] = v.x;
          Q[x][y + 1] = v.y;
        }
      bool bad = false;
#pragma unroll
      for (int p = 0; p < SW_BK; ++p) {
        const S D = Q[p][p];
        if (!(D > (S)0) || !isfinite(D)) bad = true;
        const S dg = (S)sh.diag0[kb + p];
        if (eps == 0.f && !(D > (S)kSingularPivotRel * dg)) bad = true;
        if (D < (S)kWidePivot * (dg + lam)) wide = true;   // relative pivot below 2^-5
        const S invD = recip_pos(D);
        S c[SW_BK];
#pragma unroll
        for (int x = 0; x < SW_BK; ++x) c[x] = x == p ? (S)-1 : Q[x][p];
#pragma unroll
        for (int x = 0; x < SW_BK; ++x) {
          const S f = -c[x] * invD;
#pragma unroll
          for (int y = 0; y < SW_BK; ++y) Q[x][y] = fma(f, c[y], (x == p || y == p) ? (S)0 : Q[x][y]);
        }
      }
      if (PASS32 && (bad || wide)) {   // uniform: the fp64 sweep takes this segment
        st = kSweepRedo64;
        break;
      }
      if (bad) {   // uniform: every thread read the same pivot block
        st = DYRA_SOLVE_NOT_SPD;
        break;
      }
      // the block's rows/columns sit at tile offset kb - i0 / kb - j0
      // (a multiple of SW_BK) when this tile holds them
      const int oi = kb - i0, oj = kb - j0;
      // C_j = pivot rows at this tile's columns
      S cj[SW_BK][TBJ];
#pragma unroll
      for (int p = 0; p < SW_BK; ++p)
#pragma unroll
        for (int y = 0; y < TBJ; y += 2) {
          const V2 v = *reinterpret_cast<const V2*>(&buf[p][j0 + y]);
          cj[p][y] = v.x;
          cj[p][y + 1] = v.y;
        }
#pragma unroll
      for (int x = 0; x < TB; x += 2) {
        // C_i for rows x, x + 1: pivot rows at column i (symmetry)
        S ci[2][SW_BK];
#pragma unroll
        for (int q = 0; q < SW_BK; ++q) {
          const V2 v = own ? *reinterpret_cast<const V2*>(&buf[q][i0 + x]) : P2::make(0, 0);
          ci[0][q] = v.x;
          ci[1][q] = v.y;
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int xx = x + h;
          const bool iK = oi == (xx & ~(SW_BK - 1));
          // d = C_i A_KK^-1 = -C_i Q; a row inside the block has C_i = -e_i
          S d[SW_BK];
#pragma unroll
          for (int p = 0; p < SW_BK; ++p) {
            S v = 0;
#pragma unroll
            for (int q = 0; q < SW_BK; ++q) v = fma(ci[h][q], Q[q][p], v);
            d[p] = iK ? Q[xx & (SW_BK - 1)][p] : -v;
          }
#pragma unroll
          for (int y = 0; y < TBJ; ++y) {
            const bool jK = oj == (y & ~(SW_BK - 1));
            S v = iK ? (S)0 : a[xx][y];
#pragma unroll
            for (int p = 0; p < SW_BK; ++p) v = fma(-d[p], cj[p][y], v);
            // a column inside the block has C_j = -e_j: a_ij <- d_j
            a[xx][y] = jK ? d[y & (SW_BK - 1)] : v;
          }
          publish_row(xx, kb + SW_BK, (blk + 1) & 1);
        }
      }
      __syncthreads();
    }
  }
  if (PASS32 && st != DYRA_SOLVE_OK) return kSweepRedo64;
#pragma unroll
  for (int x = 0; x < TB; ++x)
#pragma unroll
    for (int y = 0; y < TBJ; ++y)
      if (own && i0 + x < r && j0 + y < r) {
        const double v = st == DYRA_SOLVE_OK ? -(double)a[x][y] : 0.0;
        Ob[(i0 + x) * r + j0 + y] = v;
        Ob32[(i0 + x) * r + j0 + y] = (float)v;
      }
  return st;
}

// The sweep in two passes: fp32 first (half the fp64 chain latency and LDS
// bytes per step); a segment whose fp32 pass meets a relative pivot below
// kWidePivot, or any pivot failure, is swept again in fp64, which then sets
// its status and its apply precision.  So every decision near a threshold
// (singular at eps = 0, fp64 apply) is taken in fp64, and an accepted fp32
// inverse has all relative pivots at or above 2^-5.
template <int NT, int TB, int TBJ = TB>
__device__ __forceinline__ int sweep_inverse_mixed(const float* Gb, double* Ob, float* Ob32, int r, float eps,
                                                   SweepLds& sh, bool& wide) {
  const int st = sweep_inverse<NT, TB, TBJ, float, true>(Gb, Ob, Ob32, r, eps, sh, wide);
  if (st != kSweepRedo64) return st;
  __syncthreads();   // every thread is past the fp32 pass's reads of the shared buffers
  return sweep_inverse<NT, TB, TBJ, double>(Gb, Ob, Ob32, r, eps, sh, wide);
}

// ===========================================================================
// S4a (Cholesky route): (G + lambda I)^-1 from the Cholesky factor, in fp64,
// with the sweep's tile distribution (thread t owns a TB x TB tile) and its
// double-buffered broadcast of SW_BK rows per barrier:
//   1. factor A = G + lambda I = C C^T, right-looking by SW_BK-column panels:
//      every thread factors the panel's diagonal block C_KK itself (from the
//      broadcast pivot rows), forms the panel rows L_iK = A_iK C_KK^-T for its
//      own rows and columns (A_iK = A_Ki by symmetry, read from the broadcast
//      rows) and updates its trailing tile A_IJ -= L_IK L_JK^T; the panel is
//      written to LDS as a packed lower triangle (fp64);
//   2. W = C^-1 by blocked forward substitution on the identity (C W = I):
//      the threads holding block row K solve it with C_KK, broadcast it, and
//      every lower row block subtracts C_IK W_K;
//   3. (G + lambda I)^-1 = W^T W, accumulated from W's broadcast row blocks.
// The apply that follows (M' = Ginv M on fp32 MFMAs) is the two triangular
// solves C^-T (C^-1 M) with the triangular inverses formed explicitly.
// Three sequences of r / SW_BK barrier steps against the sweep's one: on
// this chip the sweep is the faster route and AUTO takes it.
// ===========================================================================

__device__ __forceinline__ int packed_lower(int i, int j) { return ((i * (i + 1)) >> 1) + j; }

// Needs r % TB == 0, r <= 128, ceil(r / TB)^2 <= NT and Cp: LDS for
// r (r + 1) / 2 doubles.  Returns the status (same in every thread).
template <int NT, int TB>
__device__ __forceinline__ int chol_inverse(const float* Gb, double* Ob, float* Ob32, int r, float eps,
                                            SweepLds& sh, double* Cp, bool& wide) {
  constexpr int PB = SW_BK;
  static_assert(TB % PB == 0 && TB % 2 == 0, "tile");
  const int tid = threadIdx.x;
  const int tpr = (r + TB - 1) / TB;
  const int i0 = (tid / tpr) * TB, j0 = (tid % tpr) * TB;
  const bool own = i0 < r;
  double a[TB][TB];
  float trf = 0.f;
#pragma unroll
  for (int x = 0; x < TB; ++x)
#pragma unroll
    for (int y = 0; y < TB; ++y) {
      const bool v = own && i0 + x < r && j0 + y < r;
      const float g = v ? Gb[(i0 + x) * r + j0 + y] : 0.f;
      a[x][y] = g;
      if (v && x + i0 == y + j0) {
        trf += g;
        sh.diag0[i0 + x] = g;
      }
    }
  const float tr = block_sum<NT>(trf, sh.red);   // its barriers also publish diag0
  int st = DYRA_SOLVE_OK;
  if (tr == 0.f) st = DYRA_SOLVE_ZERO;
  else if (!(tr > 0.f) || !isfinite(tr)) st = DYRA_SOLVE_NOT_SPD;
  auto publish_row = [&](double (&t)[TB][TB], int x, int k0, int buf) {
    const int i = i0 + x;
    if (own && i >= k0 && i < k0 + PB) {
#pragma unroll
      for (int y = 0; y < TB; y += 2)
        *reinterpret_cast<double2*>(&sh.pv[buf][i - k0][j0 + y]) = make_double2(t[x][y], t[x][y + 1]);
    }
  };
  wide = false;
  if (st == DYRA_SOLVE_OK) {
    const double lam = (double)(eps * tr / (float)r);
#pragma unroll
    for (int x = 0; x < TB; ++x)
#pragma unroll
      for (int y = 0; y < TB; ++y)
        if (own && x + i0 == y + j0) a[x][y] += lam;
    // ---- 1. A = C C^T ----
#pragma unroll
    for (int x = 0; x < TB; ++x) publish_row(a, x, 0, 0);
    __syncthreads();
    for (int kb = 0, blk = 0; kb < r; kb += PB, ++blk) {
      const double(*buf)[128] = sh.pv[blk & 1];
      double Ck[PB][PB], ic[PB];
      bool bad = false;
#pragma unroll
      for (int p = 0; p < PB; ++p) {
        double d = buf[p][kb + p];
#pragma unroll
        for (int q = 0; q < p; ++q) d = fma(-Ck[p][q], Ck[p][q], d);
        const bool ok = d > 0.0 && isfinite(d) && (eps > 0.f || d > kSingularPivotRel * sh.diag0[kb + p]);
        if (d < kWidePivot * (sh.diag0[kb + p] + lam)) wide = true;   // relative pivot below 2^-5
        if (!ok) bad = true;
        const double c = sqrt(ok ? d : 1.0);
        ic[p] = recip_pos(c);
        Ck[p][p] = c;
#pragma unroll
        for (int i = p + 1; i < PB; ++i) {
          double v = buf[i][kb + p];
#pragma unroll
          for (int q = 0; q < p; ++q) v = fma(-Ck[i][q], Ck[p][q], v);
          Ck[i][p] = v * ic[p];
        }
      }
      if (bad) {   // uniform: every thread read the same pivot block
        st = DYRA_SOLVE_NOT_SPD;
        break;
      }
      // Zk = C_KK^-1 (lower), so L_iK[p] = sum_q A_iK[q] Zk[p][q]
      double Zk[PB][PB];
#pragma unroll
      for (int q = 0; q < PB; ++q)
#pragma unroll
        for (int p = 0; p < PB; ++p) {
          if (p < q) {
            Zk[p][q] = 0.0;
          } else {
            double v = p == q ? 1.0 : 0.0;
#pragma unroll
            for (int t = q; t < p; ++t) v = fma(-Ck[p][t], Zk[t][q], v);
            Zk[p][q] = v * ic[p];
          }
        }
      double li[TB][PB], lj[TB][PB];
#pragma unroll
      for (int x = 0; x < TB; ++x) {
        double aq[PB], bq[PB];
#pragma unroll
        for (int q = 0; q < PB; ++q) {
          aq[q] = own ? buf[q][i0 + x] : 0.0;
          bq[q] = buf[q][j0 + x];
        }
#pragma unroll
        for (int p = 0; p < PB; ++p) {
          double u = 0.0, v = 0.0;
#pragma unroll
          for (int q = 0; q <= p; ++q) {
            u = fma(aq[q], Zk[p][q], u);
            v = fma(bq[q], Zk[p][q], v);
          }
          li[x][p] = u;
          lj[x][p] = v;
        }
      }
      // the panel into the packed factor: the tile whose columns hold block K
      if (own && j0 <= kb && kb < j0 + TB) {
        const int oi = kb - i0;
#pragma unroll
        for (int x = 0; x < TB; ++x) {
          const int i = i0 + x;
          if (i >= kb + PB) {
#pragma unroll
            for (int p = 0; p < PB; ++p) Cp[packed_lower(i, kb + p)] = li[x][p];
          } else if (oi == (x & ~(PB - 1))) {
#pragma unroll
            for (int p = 0; p <= (x & (PB - 1)); ++p) Cp[packed_lower(i, kb + p)] = Ck[x & (PB - 1)][p];
          }
        }
      }
#pragma unroll
      for (int x = 0; x < TB; ++x)
#pragma unroll
        for (int y = 0; y < TB; ++y)
          if (own && i0 + x >= kb + PB && j0 + y >= kb + PB) {
            double v = a[x][y];
#pragma unroll
            for (int p = 0; p < PB; ++p) v = fma(-li[x][p], lj[y][p], v);
            a[x][y] = v;
          }
#pragma unroll
      for (int x = 0; x < TB; ++x) publish_row(a, x, kb + PB, (blk + 1) & 1);
      __syncthreads();
    }
  }
  if (st == DYRA_SOLVE_OK) {
    // ---- 2. W = C^-1 (C W = I), row block by row block ----
#pragma unroll
    for (int x = 0; x < TB; ++x)
#pragma unroll
      for (int y = 0; y < TB; ++y) a[x][y] = (own && i0 + x == j0 + y) ? 1.0 : 0.0;
    for (int kb = 0, blk = 0; kb < r; kb += PB, ++blk) {
      const int oi = kb - i0;
      if (own && oi >= 0 && oi < TB) {
        double ck[PB][PB], icd[PB];
#pragma unroll
        for (int p = 0; p < PB; ++p) {
#pragma unroll
          for (int q = 0; q <= p; ++q) ck[p][q] = Cp[packed_lower(kb + p, kb + q)];
          icd[p] = recip_pos(ck[p][p]);
        }
#pragma unroll
        for (int x = 0; x < TB; ++x)
          if (oi == (x & ~(PB - 1))) {
            const int p = x & (PB - 1);
#pragma unroll
            for (int y = 0; y < TB; ++y) {
              double v = a[x][y];
#pragma unroll
              for (int q = 0; q < PB; ++q)
                if (q < p) v = fma(-ck[p][q], a[(x & ~(PB - 1)) + q][y], v);
              a[x][y] = v * icd[p];
            }
          }
      }
#pragma unroll
      for (int x = 0; x < TB; ++x) publish_row(a, x, kb, blk & 1);
      __syncthreads();
      const double(*buf)[128] = sh.pv[blk & 1];
#pragma unroll
      for (int x = 0; x < TB; ++x) {
        const int i = i0 + x;
        if (own && i >= kb + PB) {
          double c[PB];
#pragma unroll
          for (int p = 0; p < PB; ++p) c[p] = Cp[packed_lower(i, kb + p)];
#pragma unroll
          for (int y = 0; y < TB; ++y) {
            double v = a[x][y];
#pragma unroll
            for (int p = 0; p < PB; ++p) v = fma(-c[p], buf[p][j0 + y], v);
            a[x][y] = v;
          }
        }
      }
    }
    __syncthreads();
    // ---- 3. (G + lambda I)^-1 = W^T W ----
    double g[TB][TB];
#pragma unroll
    for (int x = 0; x < TB; ++x)
#pragma unroll
      for (int y = 0; y < TB; ++y) g[x][y] = 0.0;
    for (int kb = 0, blk = 0; kb < r; kb += PB, ++blk) {
#pragma unroll
      for (int x = 0; x < TB; ++x) publish_row(a, x, kb, blk & 1);
      __syncthreads();
      const double(*buf)[128] = sh.pv[blk & 1];
#pragma unroll
      for (int x = 0; x < TB; ++x) {
        double wi[PB];
#pragma unroll
        for (int p = 0; p < PB; ++p) wi[p] = own ? buf[p][i0 + x] : 0.0;
#pragma unroll
        for (int y = 0; y < TB; ++y) {
          double v = g[x][y];
#pragma unroll
          for (int p = 0; p < PB; ++p) v = fma(wi[p], buf[p][j0 + y], v);
          g[x][y] = v;
        }
      }
    }
#pragma unroll
    for (int x = 0; x < TB; ++x)
#pragma unroll
      for (int y = 0; y < TB; ++y) a[x][y] = g[x][y];
  }
#pragma unroll
  for (int x = 0; x < TB; ++x)
#pragma unroll
    for (int y = 0; y < TB; ++y)
      if (own && i0 + x < r && j0 + y < r) {
        const double v = st == DYRA_SOLVE_OK ? a[x][y] : 0.0;
        Ob[(i0 + x) * r + j0 + y] = v;
        Ob32[(i0 + x) * r + j0 + y] = (float)v;
      }
  return st;
}

// G_b = the sum of segment b's Gram partials, in order, into `out` (r x r
// fp32, LDS or global; float4 columns, up to 8 partials' loads in flight per
// thread): gchunks token chunks of the segment, or (gprows > 0) the first
// stage's per-tile partials of the tiles of gprows tokens that the segment
// meets, in slot 1 of its first tile when that tile starts in the previous
// segment, else in slot 0.  The caller synchronises before reading `out`.
template <int NT>
__device__ __forceinline__ void gram_sum(const float* __restrict__ gpart, int gchunks, int64_t gprows, int64_t b,
                                         int64_t lo, int64_t hi, int r, float* out) {
  const int nq = r * r / 4;   // r % 8 == 0
  const int64_t rb_lo = gprows > 0 ? lo / gprows : 0;
  const int nparts = gprows > 0 ? (int)((hi - 1) / gprows - rb_lo + 1) : gchunks;
  auto part_ptr = [&](int p) -> const float4* {
    int64_t idx;
    if (gprows > 0) {
      const int64_t rb = rb_lo + p;
      idx = rb * 2 + ((p == 0 && lo > rb * gprows) ? 1 : 0);
    } else {
      idx = b * gchunks + p;
    }
    return reinterpret_cast<const float4*>(gpart + idx * r * r);
  };
  for (int e0 = threadIdx.x; e0 < nq; e0 += 4 * NT) {
    float4 acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int c0 = 0; c0 < nparts; c0 += 8) {
      float4 v[8][4];
#pragma unroll
      for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = e0 + i * NT;
          v[c][i] = (c0 + c < nparts && e < nq) ? part_ptr(c0 + c)[e] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
      for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[i].x += v[c][i].x;
          acc[i].y += v[c][i].y;
          acc[i].z += v[c][i].z;
          acc[i].w += v[c][i].w;
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (e0 + i * NT < nq) reinterpret_cast<float4*>(out)[e0 + i * NT] = acc[i];
  }
}

// ===========================================================================
// S4a': Newton-Schulz inverse of one segment by one workgroup of 8 waves
// on the 128 x 128 iterate.  Jacobi-scaled A' = D^-1/2 (G + lambda I) D^-1/2 (unit diagonal,
// padded with the identity up to 128), X_0 = I / ||A'||_F, and the
// Newton-Schulz step X <- X (2 I - A' X) = X + X E with E = I - A' X, until
// ||E||_F <= tol; then Ginv = D^-1/2 X D^-1/2.  Every product runs on bf16
// MFMAs with fp32 accumulation, in two phases:
//   * coarse, while far from the inverse (the iteration corrects its own
//     rounding there): T = A' X and X T from the bf16 parts alone, one MFMA
//     each, X <- 2 X - X T;
//   * fine, from the first coarse step that fails to reduce ||E||_F, or
//     once it is below 1/4: A' and X are held as three bf16 terms each
//     (hi + mid + lo, about 24 significant bits, as fp32) and A' X is
//     formed from the six products whose terms reach 2^-24 relative, so the
//     residual E = I - A' X is as accurate as an fp32 product would make it,
//     while an fp32 MFMA product would cost sixteen MFMAs at gfx950's rates
//     against these six.  The correction X E takes X's three terms and E
//     rounded to bf16: rounding X would add about 2^-9 cond(A') ||E|| to
//     the next residual (A' amplifies it), rounding E only about 2^-9 ||E||
//     (A' X is close to I), which slows the quadratic convergence by no more
//     than that factor per step.
// X and E (T in the coarse phase) stay in LDS, stored transposed (row c
// holds column c) so that every MFMA operand is one 16-byte row read; X is
// a polynomial in A', hence symmetric, so its stored rows also serve as its
// rows in X E.  The iteration stops at the tolerance, or flags the segment
// for the sweep when a fine step stops reducing ||E||_F (its rounding floor)
// above `accept`; from ||E||_F <= accept / 4 one more step leaves about its
// square and is taken without another residual.
// ===========================================================================

constexpr int NSS_N = 128;
__device__ __forceinline__ int nss_off(int row, int k) {   // bf16 element (row, k), 16-byte chunks swizzled
  return row * 256 + ((((k >> 3) ^ row) & 15) << 4) + ((k & 7) << 1);
}
// x = h + m + l (bf16 terms; each difference is exact in fp32)
__device__ __forceinline__ void split3_bf16(float x, uint16_t& h, uint16_t& m, uint16_t& l) {
  h = f2bf(x);
  const float r1 = x - bf2f(h);
  m = f2bf(r1);
  l = f2bf(r1 - bf2f(m));
}
__device__ __forceinline__ uint4 pack8_b16(const uint16_t (&v)[8]) {
  return make_uint4(v[0] | (uint32_t)v[1] << 16, v[2] | (uint32_t)v[3] << 16, v[4] | (uint32_t)v[5] << 16,
                    v[6] | (uint32_t)v[7] << 16);
}
// LDS of one Newton-Schulz solve: X (three bf16 planes), T or E, the Jacobi
// scales and a reduction scratch.
constexpr int NSL_XS = 0, NSL_TS = 3 * NSS_N * 256, NSL_DSC = 4 * NSS_N * 256, NSL_RED = NSL_DSC + NSS_N * 4;
constexpr int NS_LDS = NSL_RED + 16 * 4;
// bf16 storage: ||I - A' X||_F <= 1e-4 is far below the bf16 rounding of
// M'; a floor above 1e-2 goes to the sweep
constexpr float kNsTolBf16 = 1e-4f, kNsAcceptBf16 = 1e-2f;
constexpr int kNsMaxit = 60;

// One segment's inverse by 8 waves: wave (bi, bh) owns rows 32 bi .. + 31
// and the two 32-column blocks from 64 bh.  Gb: G_b (r x r row-major); sm:
// NS_LDS bytes of LDS.  Writes Ob / Ob32 (zeros unless the status is OK)
// when the iteration converges; returns the status, with `conv` false when
// a positive definite G_b could not be solved (the caller then has it
// re-solved by the sweep).
__device__ __forceinline__ int ns_solve(const float* Gb, int r, float eps, int maxit, float tol, float accept, char* sm,
                                        double* Ob, float* Ob32, bool& conv) {
  constexpr int NT = 512, WPR = 2, JB = 2;   // threads, waves per row block, column blocks per wave
  char(*XS)[NSS_N * 256] = reinterpret_cast<char(*)[NSS_N * 256]>(sm + NSL_XS);
  char* TS = sm + NSL_TS;
  float* dsc = reinterpret_cast<float*>(sm + NSL_DSC);
  float* red = reinterpret_cast<float*>(sm + NSL_RED);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l = lane & 31, g = lane >> 5;
  const int bi = w / WPR, bh = w % WPR;   // rows bi 32 .. + 31, columns bh 32 JB .. + 32 JB - 1
  auto col_of = [&](int j) { return bh * 32 * JB + 32 * j + l; };
  float dv = 0.f;
  for (int i = tid; i < r; i += NT) dv += Gb[i * r + i];
  const float tr = block_sum<NT>(dv, red);
  const float lam = eps * tr / (float)r;
  float badf = 0.f;
  for (int i = tid; i < NSS_N; i += NT) {
    const float d = i < r ? Gb[i * r + i] + lam : 1.f;
    dsc[i] = d > 0.f ? rsqrtf(d) : 0.f;
    if (!(d > 0.f) || !isfinite(d)) badf = 1.f;
  }
  badf = block_sum<NT>(badf, red);   // barriers: dsc complete afterwards
  int st = DYRA_SOLVE_OK;
  if (tr == 0.f) st = DYRA_SOLVE_ZERO;
  else if (!(tr > 0.f) || !isfinite(tr) || badf > 0.f) st = DYRA_SOLVE_NOT_SPD;
  // A' fragments of rows bi 32 + l, k = 16 ks + 8 g .. + 7, as three bf16 terms
  uint4 Ah[8], Am[8], Al[8];
  float fro2 = 0.f;
  const int arow = bi * 32 + l;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    uint16_t h[8], m[8], lo[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int col = 16 * ks + 8 * g + e;
      float v;
      if (arow < r && col < r) v = (Gb[arow * r + col] + (arow == col ? lam : 0.f)) * dsc[arow] * dsc[col];
      else v = arow == col ? 1.f : 0.f;
      if (bh == 0) fro2 += v * v;
      split3_bf16(v, h[e], m[e], lo[e]);
    }
    Ah[ks] = pack8_b16(h);
    Am[ks] = pack8_b16(m);
    Al[ks] = pack8_b16(lo);
  }
  fro2 = block_sum<NT>(fro2, red);
  const float x0 = 1.f / sqrtf(fro2);
  // accumulator element v of lane (l, g) in column block j is (rr, cc) with
  // rr = bi 32 + 8 (v / 4) + 4 g + v % 4, cc = col_of(j); stored at row cc,
  // k = rr (four consecutive v at one 8-byte place)
  auto store_x = [&](int cc, const float (&x)[16]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint16_t h[4], m[4], lo[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) split3_bf16(x[4 * q + e], h[e], m[e], lo[e]);
      const int off = nss_off(cc, bi * 32 + 8 * q + 4 * g);
      *reinterpret_cast<uint2*>(XS[0] + off) = make_uint2(h[0] | (uint32_t)h[1] << 16, h[2] | (uint32_t)h[3] << 16);
      *reinterpret_cast<uint2*>(XS[1] + off) = make_uint2(m[0] | (uint32_t)m[1] << 16, m[2] | (uint32_t)m[3] << 16);
      *reinterpret_cast<uint2*>(XS[2] + off) = make_uint2(lo[0] | (uint32_t)lo[1] << 16, lo[2] | (uint32_t)lo[3] << 16);
    }
  };
  auto load_x = [&](int cc, float (&x)[16]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int off = nss_off(cc, bi * 32 + 8 * q + 4 * g);
      const uint2 h = *reinterpret_cast<const uint2*>(XS[0] + off);
      const uint2 m = *reinterpret_cast<const uint2*>(XS[1] + off);
      const uint2 lo = *reinterpret_cast<const uint2*>(XS[2] + off);
      const uint32_t hw[2] = {h.x, h.y}, mw[2] = {m.x, m.y}, lw[2] = {lo.x, lo.y};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int sh = 16 * (e & 1);
        x[4 * q + e] = bf2f((bf16_t)(hw[e >> 1] >> sh)) + (bf2f((bf16_t)(mw[e >> 1] >> sh)) +
                                                          bf2f((bf16_t)(lw[e >> 1] >> sh)));
      }
    }
  };
  auto store_t = [&](int cc, const float (&t)[16]) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<uint2*>(TS + nss_off(cc, bi * 32 + 8 * q + 4 * g)) =
          make_uint2(f2bf(t[4 * q]) | (uint32_t)f2bf(t[4 * q + 1]) << 16,
                     f2bf(t[4 * q + 2]) | (uint32_t)f2bf(t[4 * q + 3]) << 16);
  };
#pragma unroll
  for (int j = 0; j < JB; ++j) {
    const int cc = col_of(j);
    float x[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int rr = bi * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
      x[v] = rr == cc ? x0 : 0.f;
    }
    store_x(cc, x);
  }
  __syncthreads();
  // 16-byte operand row (row, k = 16 ks + 8 g .. + 7) of a transposed tile
  auto frag = [&](const char* S, int row, int ks) {
    return *reinterpret_cast<const uint4*>(S + row * 256 + ((((2 * ks + g)) ^ row) & 15) * 16);
  };
  auto mma = [&](f32x16 acc, uint4 a, uint4 bq) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, bq),
                                                   acc, 0, 0, 0);
  };
  float prev = 1e30f;
  int it = 0;
  bool ok = st == DYRA_SOLVE_OK;
  bool converged = false, coarse = true;
  while (ok && it < maxit) {
    // T = A' X (this wave's column blocks); X column cc is stored as row cc
    f32x16 acc[JB];
#pragma unroll
    for (int j = 0; j < JB; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[j][v] = 0.f;
    if (coarse) {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int j = 0; j < JB; ++j) acc[j] = mma(acc[j], Ah[ks], frag(XS[0], col_of(j), ks));
    } else {
#pragma unroll
      for (int j = 0; j < JB; ++j)
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const int cc = col_of(j);
          const uint4 xh = frag(XS[0], cc, ks), xm = frag(XS[1], cc, ks), xl = frag(XS[2], cc, ks);
          acc[j] = mma(acc[j], Al[ks], xh);
          acc[j] = mma(acc[j], Am[ks], xm);
          acc[j] = mma(acc[j], Ah[ks], xl);
          acc[j] = mma(acc[j], Am[ks], xh);
          acc[j] = mma(acc[j], Ah[ks], xm);
          acc[j] = mma(acc[j], Ah[ks], xh);
        }
    }
    float e2 = 0.f;
#pragma unroll
    for (int j = 0; j < JB; ++j) {
      const int cc = col_of(j);
      float tv[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int rr = bi * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
        const float d = (rr == cc ? 1.f : 0.f) - acc[j][v];
        e2 += d * d;
        tv[v] = coarse ? acc[j][v] : d;
      }
      store_t(cc, tv);
    }
    e2 = block_sum<NT>(e2, red);   // barriers: T / E complete afterwards
    const float err = sqrtf(e2);
    if (!isfinite(err)) {
      ok = false;
      break;
    }
    if (err <= tol) {
      converged = true;
      break;
    }
    bool last = false;
    if (coarse) {
      // a coarse step that stopped reducing the error: redo the residual of
      // the same X in the fine phase (its first error is not compared with
      // the coarse ones)
      if (err >= prev) {
        coarse = false;
        prev = 1e30f;
        continue;
      }
    } else {
      // the fine floor: the error stopped falling, or fell less than 4-fold
      // where exact arithmetic would square it
      if (err >= prev || (prev < 0.1f && err > 0.25f * prev)) {
        converged = err < accept;
        break;
      }
      last = 4.f * err <= accept;
    }
    prev = err;
    // coarse: X <- 2 X - X T; fine: X <- X + X E.  X row bi 32 + l (X
    // symmetric: its stored row), T / E column cc
#pragma unroll
    for (int j = 0; j < JB; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[j][v] = 0.f;
    if (coarse) {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const uint4 ah = frag(XS[0], arow, ks);
#pragma unroll
        for (int j = 0; j < JB; ++j) acc[j] = mma(acc[j], ah, frag(TS, col_of(j), ks));
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const uint4 ah = frag(XS[0], arow, ks), am = frag(XS[1], arow, ks), al = frag(XS[2], arow, ks);
#pragma unroll
        for (int j = 0; j < JB; ++j) {
          const uint4 ej = frag(TS, col_of(j), ks);
          acc[j] = mma(acc[j], al, ej);
          acc[j] = mma(acc[j], am, ej);
          acc[j] = mma(acc[j], ah, ej);
        }
      }
    }
    float xo[JB][16];
#pragma unroll
    for (int j = 0; j < JB; ++j) load_x(col_of(j), xo[j]);
    __syncthreads();   // every wave is done reading X
#pragma unroll
    for (int j = 0; j < JB; ++j) {
#pragma unroll
      for (int v = 0; v < 16; ++v) xo[j][v] = coarse ? 2.f * xo[j][v] - acc[j][v] : xo[j][v] + acc[j][v];
      store_x(col_of(j), xo[j]);
    }
    __syncthreads();
    ++it;
    if (last) {
      converged = true;
      break;
    }
    if (coarse && err < 0.25f) {
      coarse = false;
      prev = 1e30f;
    }
  }
  conv = !(st == DYRA_SOLVE_OK && !(ok && converged));
  if (!conv) return st;   // broke down, or stalled above `accept`
  const bool good = st == DYRA_SOLVE_OK;
  for (int e = tid; e < r * r; e += NT) {
    const int i = e / r, jj = e % r;
    // X (i, jj) is stored at row jj, k = i
    const int off = nss_off(jj, i);
    const float x = bf2f(*reinterpret_cast<const bf16_t*>(XS[0] + off)) +
                    (bf2f(*reinterpret_cast<const bf16_t*>(XS[1] + off)) +
                     bf2f(*reinterpret_cast<const bf16_t*>(XS[2] + off)));
    const double v = good ? (double)dsc[i] * (double)x * (double)dsc[jj] : 0.0;
    Ob[e] = v;
    Ob32[e] = (float)v;
  }
  return st;
}

// One 512-thread workgroup per segment.  A segment the iteration cannot
// solve is re-solved in the same workgroup by the fp64 sweep (its buffers
// overlay the iteration's) and reports DYRA_SOLVE_FALLBACK.
static_assert(sizeof(SweepLds) <= NS_LDS, "the sweep's LDS fits in the iteration's");
// With gpart, the workgroup first sums segment b's Gram partials into G_b
// (gram_sum), so the launch needs only the partials and can run beside the
// M strips.
__global__ __launch_bounds__(512) void ns_inverse_kernel(float* G, double* Ginv, float* Ginv32, int32_t* status,
                                                          int32_t* prec, int r, float eps, int maxit, float tol,
                                                          float accept, const float* __restrict__ gpart,
                                                          int gchunks, int64_t gprows, SegMap sg) {
  __shared__ __attribute__((aligned(16))) char sm[NS_LDS];
  const int64_t b = blockIdx.x;
  if (gpart) {
    gram_sum<512>(gpart, gchunks, gprows, b, sg.lo(b), sg.hi(b), r, G + b * r * r);
    __threadfence_block();
    __syncthreads();   // G_b complete (the workgroup's own global writes)
  }
  bool conv;
  const int st = ns_solve(G + b * r * r, r, eps, maxit, tol, accept, sm, Ginv + b * r * r, Ginv32 + b * r * r,
                          conv);
  if (conv) {
    if (threadIdx.x == 0) {
      status[b] = st;
      // the fp32 apply: the iteration's own tolerance, not the apply's
      // rounding, bounds the accuracy of M' for a Newton-Schulz inverse
      prec[b] = 0;
    }
    return;
  }
  __syncthreads();   // every wave is done with the iteration's buffers
  bool wide;
  const int st2 = sweep_inverse<512, 4, 8>(G + b * r * r, Ginv + b * r * r, Ginv32 + b * r * r, r, eps,
                                           *reinterpret_cast<SweepLds*>(sm), wide);
  if (threadIdx.x == 0) {
    status[b] = st2 == DYRA_SOLVE_OK ? DYRA_SOLVE_FALLBACK : st2;
    prec[b] = st2 == DYRA_SOLVE_OK && wide ? 1 : 0;
  }
}


// ===========================================================================
// S3 (bf16): token reductions without an LDS transpose.
// Workgroups [0, B): G_b = L_b^T L_b and its inverse (the r x r solve runs
// here, concurrently with the M strips).  Workgroups [B, ...): one
// 128-channel strip of M_b = L_b^T X_b each.  Each wave streams a quarter of
// the segment's tokens: a lane loads 8 token rows x 8 channels of X (16 B per
// row, coalesced along channels), transposes the 8 x 8 bf16 block in
// registers (v_perm) and feeds it as the B operand of 16x16x32 MFMAs whose A
// operand is L^T (token-contiguous).  Output block q then holds channels
// 8j + q.  Partial sums of the 4 waves are reduced through LDS in a fixed
// order (deterministic, no atomics).
// ===========================================================================

constexpr int S3_NT = 256;
constexpr int S3_STRIP = 128;
// LDS: M strips use 64 KB of partials; the G/solve role uses 16 KB of
// partials + r*r fp32 G + the sweep's pivot-row buffers.
template <int NB>
struct S3Lds {
  static constexpr int G_OFF = 16 * 1024;
  static constexpr int SW_OFF = G_OFF + NB * 32 * NB * 32 * 4;
  static constexpr int G_END = SW_OFF + (int)sizeof(SweepLds);
  static constexpr int BYTES = G_END > 64 * 1024 ? G_END : 64 * 1024;
};

// tbase: the token index of column 0 of the L^T rows (0 unless the rows are
// addressed relative to the segment).
template <int NRB, bool B32>
__device__ __forceinline__ void s3_m_strip(const bf16_t* __restrict__ Lt, int64_t ldt,
                                           const bf16_t* __restrict__ X, int64_t c1, int r, int64_t lo,
                                           int64_t hi, int64_t c0, float* __restrict__ Mb, char* lds, int64_t tbase) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int j = lane & 15, g = lane >> 4;
  f32x4 acc[NRB][8];
#pragma unroll
  for (int ib = 0; ib < NRB; ++ib)
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[ib][q] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int64_t a0 = lo & ~(int64_t)7;
  const int nsteps = (int)((hi - a0 + 31) / 32);
  const int s0 = w * nsteps / 4, s1 = (w + 1) * nsteps / 4;
  const int64_t col = c0 + 8 * j;
  const bool colok = col < c1;
  // Branch-free buffer loads relative to the step's first token (32-bit
  // offsets): X rows outside [lo, hi) and L^T rows past r or ldt read as
  // zero, so every load of a step is in flight at once.  A zero X row
  // cancels its token's L^T column, so L^T is masked only on the steps that
  // reach past the segment (where it may hold unwritten padding past n).
  auto load = [&](int st, uint4 (&xv)[8], uint4 (&av)[NRB]) {
    const int64_t ts = a0 + 32 * (int64_t)st;
    const int64_t t0 = ts + 8 * g;
    if constexpr (B32) {
      const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<bf16_t*>(X + ts * c1), (short)0, 0x7fffffff, 0x00020000);
      const __amdgpu_buffer_rsrc_t lr = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<bf16_t*>(Lt + ts), (short)0, 0x7fffffff, 0x00020000);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int64_t tt = t0 + e;
        const int off = colok && tt >= lo && tt < hi ? ((8 * g + e) * (int)c1 + (int)col) * 2 : (int)0x80000000u;
        xv[e] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
      }
#pragma unroll
      for (int ib = 0; ib < NRB; ++ib) {
        const int row = ib * 16 + j;
        const int off = row < r && t0 - tbase < ldt ? (row * (int)ldt + 8 * g) * 2 : (int)0x80000000u;
        av[ib] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(lr, off, 0, 0));
      }
    } else {   // offsets past 32 bits: 64-bit loads, every L^T column masked
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int64_t tt = t0 + e;
        xv[e] = (colok && tt >= lo && tt < hi) ? *reinterpret_cast<const uint4*>(X + tt * c1 + col) : zero4();
      }
#pragma unroll
      for (int ib = 0; ib < NRB; ++ib) {
        const int row = ib * 16 + j;
        const uint4 v = (row < r && t0 - tbase < ldt) ? *reinterpret_cast<const uint4*>(Lt + row * ldt + t0) : zero4();
        av[ib] = mask_tokens<bf16_t>(v, t0, lo, hi);
      }
    }
  };
  auto edge_mask = [&](int st, uint4 (&av)[NRB]) {
    const int64_t ts = a0 + 32 * (int64_t)st;
    if (B32 && (ts < lo || ts + 32 > hi)) {
#pragma unroll
      for (int ib = 0; ib < NRB; ++ib) av[ib] = mask_tokens<bf16_t>(av[ib], ts + 8 * g, lo, hi);
    }
  };
  if constexpr (NRB <= 2) {
    // registers allow a one-step software prefetch
    if (s0 < s1) {
      uint4 xv[8], av[NRB];
      load(s0, xv, av);
      for (int st = s0; st < s1; ++st) {
        uint4 bv[8];
        transpose8x8_b16(xv, bv);
        uint4 ac[NRB];
#pragma unroll
        for (int ib = 0; ib < NRB; ++ib) ac[ib] = av[ib];
        edge_mask(st, ac);
        if (st + 1 < s1) load(st + 1, xv, av);
#pragma unroll
        for (int ib = 0; ib < NRB; ++ib)
#pragma unroll
          for (int q = 0; q < 8; ++q) mma16(acc[ib][q], ac[ib], bv[q]);
      }
    }
  } else {
    // latency hidden by the second resident workgroup instead
    for (int st = s0; st < s1; ++st) {
      uint4 xv[8], av[NRB], bv[8];
      load(st, xv, av);
      edge_mask(st, av);
      transpose8x8_b16(xv, bv);
#pragma unroll
      for (int ib = 0; ib < NRB; ++ib)
#pragma unroll
        for (int q = 0; q < 8; ++q) mma16(acc[ib][q], av[ib], bv[q]);
    }
  }
  // Reduce the 4 wave partials pairwise through LDS (fixed order: ((w0 + w2)
  // + (w1 + w3))), 4 row blocks (16 KB per wave) per round, then wave 0
  // writes the strip: lane (j, g) holds rows 4g + v of each 16-row block and
  // channels 8j .. 8j + 7 -> two 16-byte fp32 stores per (block, v).
  float* part = reinterpret_cast<float*>(lds);
  constexpr int RB = NRB < 4 ? NRB : 4;
  constexpr int PW = RB * 8 * 4;   // floats per lane per round
#pragma unroll
  for (int rb0 = 0; rb0 < NRB; rb0 += RB) {
    auto slot = [&](int sl, int ib, int q, int v) -> float& {
      return part[((sl * RB + ib) * 32 + q * 4 + v) * 64 + lane];
    };
    __syncthreads();
    if (w >= 2) {
#pragma unroll
      for (int ib = 0; ib < RB; ++ib)
#pragma unroll
        for (int q = 0; q < 8; ++q)
#pragma unroll
          for (int v = 0; v < 4; ++v) slot(w - 2, ib, q, v) = acc[rb0 + ib][q][v];
    }
    __syncthreads();
    if (w < 2) {
#pragma unroll
      for (int ib = 0; ib < RB; ++ib)
#pragma unroll
        for (int q = 0; q < 8; ++q)
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[rb0 + ib][q][v] += slot(w, ib, q, v);
    }
    __syncthreads();
    if (w == 1) {
#pragma unroll
      for (int ib = 0; ib < RB; ++ib)
#pragma unroll
        for (int q = 0; q < 8; ++q)
#pragma unroll
          for (int v = 0; v < 4; ++v) slot(0, ib, q, v) = acc[rb0 + ib][q][v];
    }
    __syncthreads();
    if (w == 0 && colok) {
#pragma unroll
      for (int ib = 0; ib < RB; ++ib)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int row = (rb0 + ib) * 16 + 4 * g + v;
          if (row >= r) continue;
          float sum[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) sum[q] = acc[rb0 + ib][q][v] + slot(0, ib, q, v);
          float4* dst = reinterpret_cast<float4*>(Mb + (int64_t)row * c1 + col);
          dst[0] = make_float4(sum[0], sum[1], sum[2], sum[3]);
          dst[1] = make_float4(sum[4], sum[5], sum[6], sum[7]);
        }
    }
    (void)PW;
  }
}

// G_b = L_b^T L_b (fp32, into LDS as a dense r x r matrix at `Gs`), from
// L^T rows with 32x32x16 MFMAs; the 4 waves split the tokens.
template <int NB>
__device__ __forceinline__ void s3_gram(const bf16_t* __restrict__ Lt, int64_t ldt, int r, int64_t lo, int64_t hi,
                                        float* Gs, char* lds, int64_t tbase) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l = lane & 31, g = lane >> 5;
  f32x16 acc[NB][NB];
#pragma unroll
  for (int a = 0; a < NB; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;
  const int64_t a0 = lo & ~(int64_t)7;
  const int nsteps = (int)((hi - a0 + 15) / 16);
  const int s0 = w * nsteps / 4, s1 = (w + 1) * nsteps / 4;
  // PF token steps per round: their loads are all issued before the MFMAs
  constexpr int PF = NB <= 2 ? 8 : 2;
  for (int st0 = s0; st0 < s1; st0 += PF) {
    uint4 f[PF][NB];
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int64_t t0 = a0 + 16 * (int64_t)(st0 + u) + 8 * g;
      const bool in = st0 + u < s1;
#pragma unroll
      for (int rb = 0; rb < NB; ++rb) {
        const int row = rb * 32 + l;
        uint4 v = (in && row < r && t0 - tbase < ldt) ? *reinterpret_cast<const uint4*>(Lt + row * ldt + t0) : zero4();
        f[u][rb] = mask_tokens<bf16_t>(v, t0, lo, hi);
      }
    }
#pragma unroll
    for (int u = 0; u < PF; ++u)
#pragma unroll
      for (int a = 0; a < NB; ++a)
#pragma unroll
        for (int b = 0; b < NB; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, f[u][a]),
                                                              __builtin_bit_cast(bf16x8_t, f[u][b]), acc[a][b], 0, 0,
                                                              0);
  }
  // reduce: wave partials through LDS, one 32x32 block pair at a time
  float* part = reinterpret_cast<float*>(lds);   // [4 waves][16 regs][64 lanes]
#pragma unroll
  for (int a = 0; a < NB; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      __syncthreads();
#pragma unroll
      for (int v = 0; v < 16; ++v) part[(w * 16 + v) * 64 + lane] = acc[a][b][v];
      __syncthreads();
      for (int u = tid; u < 16 * 64; u += S3_NT) {
        const int ln = u & 63, v = u >> 6;
        const float sum = part[(0 * 16 + v) * 64 + ln] + part[(1 * 16 + v) * 64 + ln] +
                          part[(2 * 16 + v) * 64 + ln] + part[(3 * 16 + v) * 64 + ln];
        const int i = a * 32 + (v >> 2) * 8 + (ln >> 5) * 4 + (v & 3), jj = b * 32 + (ln & 31);
        if (i < r && jj < r) Gs[i * r + jj] = sum;
      }
    }
  __syncthreads();
}

// SOLVE: the r x r solve its solve role runs (0 none, 1 the sweep, 2 the
// Cholesky route), a template parameter so each instantiation carries the
// registers of its own solver only.
template <int NRB, int NB, int SOLVE>
__global__ __launch_bounds__(S3_NT, NRB <= 4 ? 2 : 1) void s3_reduce_solve_kernel(
    const bf16_t* __restrict__ Lt, int64_t ldt, const bf16_t* __restrict__ X, int64_t c1, int r, SegMap sg,
    int64_t n, int64_t B, float* __restrict__ M, float* __restrict__ G, double* __restrict__ Gi,
    float* __restrict__ Gi32,
    int32_t* __restrict__ status, int32_t* __restrict__ prec, float eps, int strips, int64_t lt_seg_rows,
    int x_rel,
    const float* __restrict__ gpart, int gchunks, int64_t gprows, int msplit, float* __restrict__ Mpart,
    int64_t nsr) {
  __shared__ __attribute__((aligned(16))) char lds[S3Lds<NB>::BYTES];
  SweepLds* sl = reinterpret_cast<SweepLds*>(lds + S3Lds<NB>::SW_OFF);
  const int64_t bid = blockIdx.x;
  // Relative addressing (the left ALS step reuses this kernel): segment b's
  // L^T rows start at row b * lt_seg_rows with their token 0 at column 0, and
  // with x_rel the segment's X rows start at row 0 of X.
  auto seg_ptrs = [&](int64_t b, int64_t lo, const bf16_t*& Ltb, const bf16_t*& Xb, int64_t& tbase) {
    Ltb = lt_seg_rows ? Lt + b * lt_seg_rows * ldt - lo : Lt;
    Xb = x_rel ? X - lo * c1 : X;
    tbase = lt_seg_rows ? lo : 0;
  };
  // Roles: nsr solve workgroups (B, or 0 when the solve runs in a launch of
  // its own), then B * strips strip workgroups.  Workgroups
  // go to the 8 XCDs in turn (block id mod 8); when B is a multiple of 8,
  // segment b's solve role and all its strips run on XCD b mod 8, so the
  // strips of a segment share one L2 copy of its L^T rows instead of every
  // XCD fetching every segment's rows from HBM.
  // r > 64: a strip workgroup takes 64 of the r rows of M_b (the r / 64
  // row blocks of a strip are consecutive roles): 8 row blocks of
  // accumulators per wave would not fit the registers
  constexpr int SNRB = NRB > 4 ? 4 : NRB;
  constexpr int RH = NRB / SNRB;
  int64_t b, strip;   // strip < 0: solve role
  int part = 0;       // token part of the strip (msplit > 1)
  int rh = 0;         // row block of 16 SNRB rows (r > 64)
  if (msplit > 1 || RH > 1) {
    if (bid < nsr) {
      b = bid;
      strip = -1;
    } else {
      const int64_t u = bid - nsr;
      b = u / (strips * msplit * RH);
      strip = (u / (msplit * RH)) % strips;
      part = (int)((u / RH) % msplit);
      rh = (int)(u % RH);
    }
  } else if ((B & 7) == 0) {
    const int64_t x = bid & 7, j = bid >> 3, per = nsr >> 3;
    if (j < per) {
      b = x + 8 * j;
      strip = -1;
    } else {
      const int64_t u = j - per;
      b = x + 8 * (u / strips);
      strip = u % strips;
    }
  } else if (bid < nsr) {
    b = bid;
    strip = -1;
  } else {
    b = (bid - nsr) / strips;
    strip = (bid - nsr) % strips;
  }
  if (strip < 0) {
    const int64_t lo = sg.lo(b), hi = sg.hi(b);
    const bf16_t *Ltb, *Xb;
    int64_t tbase;
    seg_ptrs(b, lo, Ltb, Xb, tbase);
    float* Gs = reinterpret_cast<float*>(lds + S3Lds<NB>::G_OFF);
    if (gpart) {
      gram_sum<S3_NT>(gpart, gchunks, gprows, b, lo, hi, r, Gs);
      __syncthreads();
    } else {
      s3_gram<NB>(Ltb, ldt, r, lo, hi, Gs, lds, tbase);
    }
    // publish G (the Newton-Schulz path and diagnostics read it)
    for (int e = threadIdx.x; e < r * r; e += S3_NT) G[b * r * r + e] = Gs[e];
    if constexpr (SOLVE != 0) {
      // TB x TB tiles: ceil(r / TB)^2 <= 256 threads for r <= 32 NB.  The
      // Cholesky route keeps its packed factor in the LDS below the sweep's
      // buffers (G has been read into registers by then)
      constexpr int TB = NB <= 2 ? 4 : 8;
      static_assert(32 * NB * (32 * NB + 1) / 2 * 8 <= S3Lds<NB>::SW_OFF, "packed factor fits");
      int st;
      bool wide;
      if constexpr (SOLVE == 2)
        st = chol_inverse<S3_NT, TB>(Gs, Gi + b * r * r, Gi32 + b * r * r, r, eps, *sl,
                                     reinterpret_cast<double*>(lds), wide);
      else
        st = sweep_inverse_mixed<S3_NT, TB>(Gs, Gi + b * r * r, Gi32 + b * r * r, r, eps, *sl, wide);
      if (threadIdx.x == 0) {
        status[b] = st;
        prec[b] = st == DYRA_SOLVE_OK && wide ? 1 : 0;
      }
    }
    return;
  }
  const int64_t c0 = strip * S3_STRIP;
  const int64_t lo = sg.lo(b), hi = sg.hi(b);
  const bf16_t *Ltb, *Xb;
  int64_t tbase;
  seg_ptrs(b, lo, Ltb, Xb, tbase);
  // this workgroup's tokens: the whole segment, or part `part` of msplit
  // (32-token aligned; an empty part writes zeros)
  int64_t plo = lo, phi = hi;
  float* Mb = M + b * r * c1;
  if (msplit > 1) {
    const int64_t chunk = ((hi - lo + msplit - 1) / msplit + 31) & ~(int64_t)31;
    plo = imin64(hi, lo + part * chunk);
    phi = imin64(hi, plo + chunk);
    Mb = Mpart + ((int64_t)part * B + b) * r * c1;
  }
  // this role's rows: 16 SNRB rows from row 16 SNRB rh of L^T and M_b
  const int r0 = rh * 16 * SNRB;
  const int rr = r - r0 < 16 * SNRB ? r - r0 : 16 * SNRB;
  if (rr <= 0) return;
  Ltb += (int64_t)r0 * ldt;
  Mb += (int64_t)r0 * c1;
  // 32-bit buffer offsets reach every X row of a 32-token step and every
  // L^T row of a step
  const bool b32 = 32 * c1 * 2 < ((int64_t)1 << 31) && ((int64_t)rr * ldt + 64) * 2 < ((int64_t)1 << 31);
  if (b32) s3_m_strip<SNRB, true>(Ltb, ldt, Xb, c1, rr, plo, phi, c0, Mb, lds, tbase);
  else s3_m_strip<SNRB, false>(Ltb, ldt, Xb, c1, rr, plo, phi, c0, Mb, lds, tbase);
}

// M = sum over the msplit token parts of the strips' fp32 partials, in part
// order (float4 per thread).
__global__ __launch_bounds__(256) void m_split_reduce_kernel(const float* __restrict__ Mpart, float* __restrict__ M,
                                                             int64_t count4, int msplit) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= count4) return;
  const float4* src = reinterpret_cast<const float4*>(Mpart);
  float4 acc = src[i];
  for (int p = 1; p < msplit; ++p) {
    const float4 v = src[(int64_t)p * count4 + i];
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  reinterpret_cast<float4*>(M)[i] = acc;
}

// Gram partials over token chunks: workgroup (b, c) writes
// sum_{t in chunk c of segment b} L_t^T L_t, so the solve role of the token
// reduction only adds a few r x r partials before its sweep instead of
// streaming the segment's L^T itself (which put the Gram's load latency on the
// critical path of that launch).
template <int NB>
__global__ __launch_bounds__(64 * NB) void gram_partial_kernel(const bf16_t* __restrict__ Lt, int64_t ldt, int r,
                                                               SegMap sg, int64_t n, int gchunks, int64_t gchunk,
                                                               float* __restrict__ Gp) {
  // one workgroup of NB waves per chunk: wave a forms block row a (the
  // 32 x 32 blocks (a, 0 .. NB - 1)); every token step's L^T loads are
  // issued before the MFMAs, and the blocks go from the accumulators
  // straight to memory
  constexpr int MAXST = 32;   // L^T row loads in flight per lane: 32 / NB steps of NB rows
  const int lane = threadIdx.x & 63, l = lane & 31, g = lane >> 5;
  const int a = threadIdx.x >> 6;
  const int64_t b = blockIdx.x / gchunks, c = blockIdx.x % gchunks;
  const int64_t lo = sg.lo(b) + c * gchunk;
  const int64_t hi = imin64(lo + gchunk, sg.hi(b));
  f32x16 acc[NB];
#pragma unroll
  for (int bb = 0; bb < NB; ++bb)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[bb][v] = 0.f;
  const int64_t a0 = lo & ~(int64_t)7;
  const int nsteps = lo < hi ? (int)((hi - a0 + 15) / 16) : 0;
  auto load = [&](int row, int64_t t0, bool in) {
    const uint4 v = (in && row < r && t0 < ldt) ? *reinterpret_cast<const uint4*>(Lt + row * ldt + t0) : zero4();
    return mask_tokens<bf16_t>(v, t0, lo, hi);
  };
  for (int st0 = 0; st0 < nsteps; st0 += MAXST / NB) {
    constexpr int PF = MAXST / NB;
    uint4 f[PF][NB];
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int64_t t0 = a0 + 16 * (int64_t)(st0 + u) + 8 * g;
      const bool in = st0 + u < nsteps;
#pragma unroll
      for (int rb = 0; rb < NB; ++rb) f[u][rb] = load(rb * 32 + l, t0, in);
    }
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      // this wave's block row among the loaded ones (a is wave-uniform)
      uint4 fa = f[u][0];
#pragma unroll
      for (int rb = 1; rb < NB; ++rb)
        if (a == rb) fa = f[u][rb];
      if (st0 + u < nsteps) {   // uniform: steps past the chunk's end are skipped
#pragma unroll
        for (int bb = 0; bb < NB; ++bb)
          acc[bb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, fa),
                                                            __builtin_bit_cast(bf16x8_t, f[u][bb]), acc[bb], 0, 0, 0);
      }
    }
  }
  // accumulator element v of lane (l, g) in block (a, bb) is
  // G[a 32 + 8 (v / 4) + 4 g + v % 4][bb 32 + l]
  float* out = Gp + (int64_t)blockIdx.x * r * r;
#pragma unroll
  for (int bb = 0; bb < NB; ++bb)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int i = a * 32 + (v >> 2) * 8 + g * 4 + (v & 3), jj = bb * 32 + l;
      if (i < r && jj < r) out[i * r + jj] = acc[bb][v];
    }
}

// S4a as its own launch (fp32 storage, whose token reduction has no solve
// role): one workgroup per segment.
template <int NT, int TB, int TBJ = TB>
__global__ __launch_bounds__(NT) void sweep_inverse_kernel(const float* G, double* Ginv, float* Ginv32,
                                                           int32_t* status, int32_t* prec, int r, float eps) {
  __shared__ SweepLds sl;
  const int64_t b = blockIdx.x;
  bool wide;
  const int st = sweep_inverse_mixed<NT, TB, TBJ>(G + b * r * r, Ginv + b * r * r, Ginv32 + b * r * r, r, eps, sl, wide);
  if (threadIdx.x == 0) {
    status[b] = st;
    prec[b] = st == DYRA_SOLVE_OK && wide ? 1 : 0;
  }
}

// r <= 64: 256 threads of 4 x 4 tiles; r <= 128: 512 threads of 4 x 8
// tiles (two waves per SIMD, 212 registers a lane; 1024 threads of 4 x 4
// leave 128 registers a lane and the sweep spilled to scratch).
void launch_sweep(const float* G, double* Ginv, float* Ginv32, int32_t* status, int32_t* prec, int r, float eps,
                  int64_t B, hipStream_t st) {
  if (r <= 64)
    hipLaunchKernelGGL((sweep_inverse_kernel<256, 4>), dim3((unsigned)B), dim3(256), 0, st, G, Ginv, Ginv32, status, prec,
                       r, eps);
  else
    hipLaunchKernelGGL((sweep_inverse_kernel<512, 4, 8>), dim3((unsigned)B), dim3(512), 0, st, G, Ginv, Ginv32, status,
                       prec, r, eps);
}

// The Cholesky route as its own launch (fp32 storage): one workgroup per
// segment, the packed factor in LDS.
template <int NT, int TB, int RMAX>
__global__ __launch_bounds__(NT) void chol_inverse_kernel(const float* G, double* Ginv, float* Ginv32,
                                                          int32_t* status, int32_t* prec, int r, float eps) {
  __shared__ SweepLds sl;
  __shared__ double cp[RMAX * (RMAX + 1) / 2];
  const int64_t b = blockIdx.x;
  bool wide;
  const int st = chol_inverse<NT, TB>(G + b * r * r, Ginv + b * r * r, Ginv32 + b * r * r, r, eps, sl, cp, wide);
  if (threadIdx.x == 0) {
    status[b] = st;
    prec[b] = st == DYRA_SOLVE_OK && wide ? 1 : 0;
  }
}

void launch_chol(const float* G, double* Ginv, float* Ginv32, int32_t* status, int32_t* prec, int r, float eps,
                 int64_t B, hipStream_t st) {
  if (r <= 64)
    hipLaunchKernelGGL((chol_inverse_kernel<256, 4, 64>), dim3((unsigned)B), dim3(256), 0, st, G, Ginv, Ginv32, status,
                       prec, r, eps);
  else   // 8 x 8 tiles: 256 threads, registers for both tiles without spills
    hipLaunchKernelGGL((chol_inverse_kernel<256, 8, 128>), dim3((unsigned)B), dim3(256), 0, st, G, Ginv, Ginv32, status,
                       prec, r, eps);
}



// ===========================================================================
// S4b: M'_b = Ginv_b M_b in fp32, stored as T (the S5 GEMM operand).
// Applying the inverse before rounding keeps the rounding error relative to
// the least-squares coefficients themselves, which stays well-behaved when
// L_b is ill-conditioned.
// ===========================================================================

// One wave per (segment, RB 16-row blocks of M', 64-column tile), with both
// operands read straight from memory.  The reduction index is permuted so
// that each lane's operands are 4-element runs: in 16-wide chunk t, lane
// group g = lane / 16 holds q = 16 t + 4 g + e for e = 0..3, and MFMA e of
// the chunk takes element e of the lane's Ginv run (row 16 rb + lane % 16)
// and of its M runs (rows q, columns c0 + 4 (lane % 16) .. + 3).  MFMA e of
// column block jb therefore sums over q = 16 t + e, + 4, + 8, + 12 and
// writes column c0 + 4 (lane % 16) + jb.
//
// Precision per segment (prec[b], set by the solve): a well-conditioned
// G_b + lambda_b I runs here, on v_mfma_f32_16x16x4f32 with the fp32 copy
// of Ginv (its rounding and the fp32 sums stay far below the storage
// rounding of M'); a segment whose solve met a relative pivot below 2^-5
// (near-singular: fewer tokens than r, or nearly collinear columns of L_b)
// takes the same task in fp64 (apply_rows_f64 on the fp64 inverse), since
// there Ginv has entries of order 1 / lambda_b that cancel in Ginv M; the
// choice is per wave (a task lies in one segment), in one launch.  The RB
// row blocks share the
// wave's M loads (accumulator of lane (i, g): rows 4 g .. + 3).  With
// NTC > 0 (r <= 16 NTC) every chunk is loaded before the first product, so
// a wave waits on memory once; otherwise the next chunk is loaded before
// the current one is multiplied.
// Rows 16 rb .. 16 rb + 15 of M'_b = Ginv_b M_b at 64-column tile ct in
// fp64, for a segment the solve flagged (prec[b] = 1): the same
// reduction-index permutation as the fp32 path, on v_mfma_f64_16x16x4f64 (operands one double per lane, k = lane / 16;
// accumulator rows interleaved: element v of lane (i, g) is row g + 4 v).
// With NTC > 0 (r <= 16 NTC) every chunk's loads are issued before the
// first product, so a wave waits on memory once.
template <typename T, int NTC>
__device__ __forceinline__ void apply_rows_f64(const double* __restrict__ Gb, const float* __restrict__ Mb,
                                               T* __restrict__ Mp, int r, int64_t c1, int64_t b, int rb,
                                               int64_t ct, int lane) {
  const int i = lane & 15, g = lane >> 4;
  const int64_t col = ct * 64 + 4 * i;          // c1 % 8 == 0: all four columns or none
  const bool cok = col < c1;
  const int row = rb * 16 + i;
  const int nt = (r + 15) >> 4;
  f64x4 acc[4];
#pragma unroll
  for (int jb = 0; jb < 4; ++jb) acc[jb] = f64x4{0.0, 0.0, 0.0, 0.0};
  // chunk t: the lane's Ginv run (row `row`, q = 16 t + 4 g .. + 3) and its
  // four M runs (rows q, columns col .. col + 3); past r or c1 they read as
  // zeros (loads clamped to valid addresses, values selected afterwards)
  auto load = [&](int t, double4& a, float4 (&m)[4]) {
    const int q0 = 16 * t + 4 * g;              // r % 4 == 0: all four q or none
    const bool aok = row < r && q0 < r, mok = cok && q0 < r;
    const double4 av = *reinterpret_cast<const double4*>(Gb + (int64_t)(aok ? row : 0) * r + (aok ? q0 : 0));
    a = aok ? av : make_double4(0.0, 0.0, 0.0, 0.0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float4 mv = *reinterpret_cast<const float4*>(Mb + (int64_t)(mok ? q0 + e : 0) * c1 + (mok ? col : 0));
      m[e] = mok ? mv : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto mul = [&](const double4& a, const float4 (&m)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const double av = e == 0 ? a.x : e == 1 ? a.y : e == 2 ? a.z : a.w;
      acc[0] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, (double)m[e].x, acc[0], 0, 0, 0);
      acc[1] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, (double)m[e].y, acc[1], 0, 0, 0);
      acc[2] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, (double)m[e].z, acc[2], 0, 0, 0);
      acc[3] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, (double)m[e].w, acc[3], 0, 0, 0);
    }
  };
  if constexpr (NTC > 0) {
    double4 a[NTC];
    float4 m[NTC][4];
#pragma unroll
    for (int t = 0; t < NTC; ++t) load(t, a[t], m[t]);
#pragma unroll
    for (int t = 0; t < NTC; ++t) mul(a[t], m[t]);
  } else {
    for (int t = 0; t < nt; ++t) {
      double4 a;
      float4 m[4];
      load(t, a, m);
      mul(a, m);
    }
  }
  if (!cok) return;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int orow = rb * 16 + g + 4 * v;
    if (orow >= r) continue;
    const int64_t o = (b * r + orow) * c1 + col;
    if constexpr (TT<T>::ESZ == 2) {
      uint2 pk;
      pk.x = (uint32_t)f2bf((float)acc[0][v]) | ((uint32_t)f2bf((float)acc[1][v]) << 16);
      pk.y = (uint32_t)f2bf((float)acc[2][v]) | ((uint32_t)f2bf((float)acc[3][v]) << 16);
      *reinterpret_cast<uint2*>(Mp + o) = pk;
    } else {
      *reinterpret_cast<float4*>(Mp + o) =
          make_float4((float)acc[0][v], (float)acc[1][v], (float)acc[2][v], (float)acc[3][v]);
    }
  }
}

constexpr int AI_WAVES = 4;
template <typename T, int RB, int NTC = 0>
__global__ __launch_bounds__(64 * AI_WAVES) void apply_inverse_kernel(const double* __restrict__ Ginv,
                                                                      const float* __restrict__ Ginv32,
                                                                      const float* __restrict__ M,
                                                                      T* __restrict__ Mp, int r, int64_t c1,
                                                                      int64_t tasks,
                                                                      const int32_t* __restrict__ status,
                                                                      const int32_t* __restrict__ prec) {
  const int lane = threadIdx.x & 63;
  const int64_t task = (int64_t)blockIdx.x * AI_WAVES + (threadIdx.x >> 6);
  if (task >= tasks) return;
  const int ngr = (r + 16 * RB - 1) / (16 * RB);  // row-block groups
  const int64_t tiles = (c1 + 63) >> 6;
  const int grp = (int)(task % ngr);            // the waves of a workgroup share an M tile
  const int64_t ct = (task / ngr) % tiles, b = task / (ngr * tiles);
  // a segment without a solve (NOT_SPD, ZERO) gets M'_b = 0, hence R_b = 0
  // exactly, even where M_b is not finite: its output is the static branch,
  // and the zero rows that mask it inside a neighbour's output tile never
  // meet a non-finite R_b
  const int sb = status[b];
  const bool solved = sb == DYRA_SOLVE_OK || sb == DYRA_SOLVE_FALLBACK;
  const bool wide = solved && prec[b] != 0;
  const int i = lane & 15, g = lane >> 4;
  const float* Gb32 = Ginv32 + b * r * r;
  const float* Mb = M + b * r * c1;
  const int64_t col = ct * 64 + 4 * i;          // c1 % 8 == 0: all four columns or none
  const bool cok = col < c1;
  const int nt = (r + 15) >> 4;
  auto load_m = [&](int t, float4 (&m)[4]) {
    const int q0 = 16 * t + 4 * g;              // r % 4 == 0: all four q or none
#pragma unroll
    for (int e = 0; e < 4; ++e)
      m[e] = (cok && q0 < r) ? *reinterpret_cast<const float4*>(Mb + (int64_t)(q0 + e) * c1 + col)
                             : make_float4(0.f, 0.f, 0.f, 0.f);
  };
  auto store_row = [&](int orow, float v0, float v1, float v2, float v3) {
    T* dst = Mp + (b * r + orow) * c1 + col;
    if constexpr (TT<T>::ESZ == 2) {
      uint2 pk;
      pk.x = (uint32_t)f2bf(v0) | ((uint32_t)f2bf(v1) << 16);
      pk.y = (uint32_t)f2bf(v2) | ((uint32_t)f2bf(v3) << 16);
      *reinterpret_cast<uint2*>(dst) = pk;
    } else {
      *reinterpret_cast<float4*>(dst) = make_float4(v0, v1, v2, v3);
    }
  };
  if (wide) {
    // fp64 for this task's row blocks; the M runs are re-read per block (in
    // cache), which only flagged segments pay
#pragma unroll 1
    for (int j = 0; j < RB; ++j)
      apply_rows_f64<T, RB == 1 ? NTC : 0>(Ginv + b * r * r, Mb, Mp, r, c1, b, grp * RB + j, ct, lane);
    return;
  }
  // ---- fp32 (zeros for an unsolved segment) ----
  auto load = [&](int t, float4 (&a)[RB], float4 (&m)[4]) {
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      const int row = (grp * RB + j) * 16 + i, q0 = 16 * t + 4 * g;
      a[j] = (row < r && q0 < r) ? *reinterpret_cast<const float4*>(Gb32 + (int64_t)row * r + q0)
                                 : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    load_m(t, m);
  };
  f32x4 acc[RB][4];
#pragma unroll
  for (int j = 0; j < RB; ++j)
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) acc[j][jb] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto mul = [&](const float4 (&a)[RB], const float4 (&m)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float mv[4] = {m[e].x, m[e].y, m[e].z, m[e].w};
#pragma unroll
      for (int j = 0; j < RB; ++j) {
        const float av = e == 0 ? a[j].x : e == 1 ? a[j].y : e == 2 ? a[j].z : a[j].w;
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) acc[j][jb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, mv[jb], acc[j][jb], 0, 0, 0);
      }
    }
  };
  if (!solved) {
    // accumulators stay zero
  } else if constexpr (NTC > 0) {
    float4 a[NTC][RB], m[NTC][4];                // chunks past r load as zeros
#pragma unroll
    for (int t = 0; t < NTC; ++t) load(t, a[t], m[t]);
#pragma unroll
    for (int t = 0; t < NTC; ++t) mul(a[t], m[t]);
  } else {
    float4 a[RB], m[4];
    load(0, a, m);
    for (int t = 0; t < nt; ++t) {
      float4 an[RB], mn[4];
      if (t + 1 < nt) load(t + 1, an, mn);
      mul(a, m);
      if (t + 1 < nt) {
#pragma unroll
        for (int j = 0; j < RB; ++j) a[j] = an[j];
#pragma unroll
        for (int e = 0; e < 4; ++e) m[e] = mn[e];
      }
    }
  }
  if (!cok) return;
#pragma unroll
  for (int j = 0; j < RB; ++j)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int orow = (grp * RB + j) * 16 + 4 * g + v;
      if (orow < r) store_row(orow, acc[j][0][v], acc[j][1][v], acc[j][2][v], acc[j][3][v]);
    }
}

// M'_b = Ginv_b M_b for B segments of r x c1: four row blocks per wave when
// that still leaves at least two waves per SIMD of a 256-CU chip, else one.
template <typename T>
void launch_apply_inverse(const double* Gi, const float* Gi32, const float* M, T* Mp, int64_t B, int r, int64_t c1,
                          const int32_t* stat, const int32_t* prec, hipStream_t st) {
  const int64_t tiles = (c1 + 63) / 64, nrb = (r + 15) / 16;
  const int64_t wide = B * tiles * ((nrb + 3) / 4);
  if (nrb >= 4 && wide >= 2048) {
    const dim3 grid((unsigned)((wide + AI_WAVES - 1) / AI_WAVES)), block(64 * AI_WAVES);
    if (r <= 64)
      hipLaunchKernelGGL((apply_inverse_kernel<T, 4, 4>), grid, block, 0, st, Gi, Gi32, M, Mp, r, c1, wide, stat, prec);
    else
      hipLaunchKernelGGL((apply_inverse_kernel<T, 4>), grid, block, 0, st, Gi, Gi32, M, Mp, r, c1, wide, stat, prec);
  } else {
    const int64_t tasks = B * tiles * nrb;
    const dim3 grid((unsigned)((tasks + AI_WAVES - 1) / AI_WAVES)), block(64 * AI_WAVES);
    if (r <= 32)
      hipLaunchKernelGGL((apply_inverse_kernel<T, 1, 2>), grid, block, 0, st, Gi, Gi32, M, Mp, r, c1, tasks, stat, prec);
    else if (r <= 64)
      hipLaunchKernelGGL((apply_inverse_kernel<T, 1, 4>), grid, block, 0, st, Gi, Gi32, M, Mp, r, c1, tasks, stat, prec);
    else
      hipLaunchKernelGGL((apply_inverse_kernel<T, 1>), grid, block, 0, st, Gi, Gi32, M, Mp, r, c1, tasks, stat, prec);
  }
}

// ===========================================================================
// host-side launch helpers
// ===========================================================================

typedef GemmCfg<bf16_t, 128, 128, 2, 2> CfgB;   // bf16 GEMMs
typedef GemmCfg<bf16_t, 160, 320, 5, 2> CfgB1W; // bf16 S1 when 256 < k + r <= 320: whole [T | L] row per tile
// bf16 fused output GEMM: short reduction (k + r), 270 MB written; single
// operand stage loaded straight into LDS, four workgroups per CU
typedef GemmCfg<bf16_t, 128, 128, 2, 2> CfgB6;
constexpr int S6_WPE = 4;
typedef GemmCfg<float, 64, 64, 2, 2> CfgF;      // fp32 GEMMs
typedef GemmCfg<bf16_t, 64, 128, 2, 2> CfgB3;   // S3, bf16
typedef GemmCfg<float, 64, 64, 2, 2> CfgF3;     // S3, fp32

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Host view of a forward's segments: B uniform segments of `seg` rows, or
// ragged ones given by a device copy of the row offsets (off_dev, [B + 1]).
struct SegInfo {
  int64_t B = 0, n = 0, seg = 0, max_len = 0, min_len = 0;
  const int32_t* off_dev = nullptr;
  const int64_t* off_host = nullptr;   // the caller's host offsets (ragged), valid during the call
  SegMap map() const { return SegMap{off_dev, seg, B, n}; }
  WsLayout layout(const dyra_spec& s, int dtype, int half_steps = 2) const {
    return ws_layout_n(s, B, n, max_len, dtype, half_steps);
  }
  static SegInfo uniform(int64_t B, int64_t seg) {
    SegInfo si;
    si.B = B;
    si.n = B * seg;
    si.seg = si.max_len = si.min_len = seg;
    return si;
  }
};

// 256 x 128 tiles: 4 compute waves of 128 x 64, 4 loaders, 3-slot ring (148 KB)
typedef GemmCfg<bf16_t, 256, 128, 2, 2> CfgB6W;
constexpr int S6W_NS = 3, S6W_NL = 4;

// Whether the persistent S6 applies: every 32-bit offset it forms stays in range.
bool s6_ws_fits(int64_t n, int64_t c2, int k, int r, int64_t B, int64_t lda_el = 0) {
  const int64_t lda = (lda_el ? lda_el : (int64_t)(k + r)) * 2, ldr = B * r * 2, ldy = c2 * 2;
  const int64_t tiles = cdiv(n, CfgB6W::BM) * cdiv(c2, CfgB6W::BN);
  return n < ((int64_t)1 << 30) && lda * CfgB6W::BM < ((int64_t)1 << 30) && ldr * CfgB6W::BN < ((int64_t)1 << 30) &&
         ldy * CfgB6W::BM < ((int64_t)1 << 30) && tiles < ((int64_t)1 << 30);
}

// Compute units of the current device, queried once per device (calls from
// several host threads may query it concurrently; they store the same value).
int device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int v = cus[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cus[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

// A0 / lda0_el / acolb and A1 / lda1_el: the two A operands (element
// pitches; A1 null: the L columns of A0 after its k static columns).
void launch_s6_ws(const bf16_t* A0, int64_t lda0_el, int64_t acolb, const bf16_t* A1, int64_t lda1_el,
                  const bf16_t* Vt, const bf16_t* Rt, const bf16_t* bias, bf16_t* Y, int64_t n, int64_t c2, int k,
                  int r, SegMap sg, int64_t B, hipStream_t st) {
  typedef CfgB6W C;
  if (!A1) {
    A1 = A0 + k;
    lda1_el = lda0_el;
  }
  const int lda0 = (int)(lda0_el * 2), lda1 = (int)(lda1_el * 2), ac = (int)acolb;
  const int tiles_n = (int)cdiv(c2, C::BN);
  const int tiles = (int)(cdiv(n, C::BM) * tiles_n);
  const int cus = device_cus();
  // a multiple of 8 workgroups (one per CU): the tile ranges are per XCD
  const int grid = cus >= 16 ? (cus / 8) * 8 : 8;
  if (bias)
    hipLaunchKernelGGL((s6_lowrank_ws_kernel<C, S6W_NS, S6W_NL, true>), dim3(grid), dim3(C::NT + S6W_NL * 64), 0, st,
                       A0, lda0, ac, A1, lda1, Vt, Rt, bias, Y, (int)n, (int)c2, k, r, sg, (int)B, tiles_n, tiles);
  else
    hipLaunchKernelGGL((s6_lowrank_ws_kernel<C, S6W_NS, S6W_NL, false>), dim3(grid), dim3(C::NT + S6W_NL * 64), 0, st,
                       A0, lda0, ac, A1, lda1, Vt, Rt, bias, Y, (int)n, (int)c2, k, r, sg, (int)B, tiles_n, tiles);
}


// C[M x N] (+)= A[M x K] B[N x K]^T (+ bias) for `batch` problems whose
// operands are `sA/sB/sC` elements apart.
template <class C>
void launch_gemm_tn(const void* A, int64_t lda_el, const void* B, int64_t ldb_el, void* Cm, int64_t ldc_el,
                    int64_t M, int64_t N, int64_t K, const void* bias, hipStream_t st, int batch = 1,
                    int64_t sA = 0, int64_t sB = 0, int64_t sC = 0) {
  typedef typename C::elem T;
  constexpr int E = TT<T>::ESZ;
  const int tiles_n = (int)cdiv(N, C::BN);
  const int64_t tiles = cdiv(M, C::BM) * tiles_n;
  if (tiles <= 0 || batch <= 0) return;
  // bf16 128 x 128 tiles: single operand stage loaded straight into LDS,
  // four workgroups per CU
  constexpr bool ONE = E == 2 && C::BM == 128 && C::BN == 128;
  hipLaunchKernelGGL((gemm_tn_kernel<C, ONE, ONE ? 4 : 1, ONE>), dim3((unsigned)(tiles * batch)), dim3(C::NT), 0, st,
                     reinterpret_cast<const char*>(A), lda_el * E, reinterpret_cast<const char*>(B), ldb_el * E,
                     reinterpret_cast<char*>(Cm), ldc_el * E, M, N, K, reinterpret_cast<const T*>(bias), tiles_n,
                     sA * E, sB * E, sC * E, (int)tiles);
}

inline int64_t lt_pitch(int64_t n) { return cdiv(n, 256) * 256; }

// Stage-boundary events (profiling aid): ev[0] before the first kernel,
// ev[i] after stage i (1 stage-1 pass, 2 token reductions, 3 solve + apply,
// 4 right-factor GEMM, 5 fused output GEMM).
struct StageEvents {
  void* const* ev;
  int n;
  // the solve may run on the library's side stream (off for the
  // allocation-free entry point, which creates nothing)
  bool fork = true;
  void mark(int i, hipStream_t st) const {
    if (ev && i < n && ev[i]) (void)hipEventRecord(reinterpret_cast<hipEvent_t>(ev[i]), st);
  }
};

template <int NRB, int NB>
void launch_s3_bf16(const bf16_t* Lt, int64_t ldt, const bf16_t* X, int64_t c1, int r, SegMap sg, int64_t n,
                    int64_t B, float* M, float* G, double* Gi, float* Gi32, int32_t* stat, int32_t* prec,
                    float eps,
                    int solve_mode,
                    hipStream_t st, int64_t lt_seg_rows = 0, bool x_rel = false, float* gpart = nullptr,
                    int gchunks = 0, int64_t gchunk = 0, int64_t gprows = 0, int msplit = 1,
                    float* Mpart = nullptr, bool solve_roles = true, bool partials_done = false) {
  const int strips = (int)cdiv(c1, S3_STRIP);
  // without solve roles the launch has the M strips only (and writes no G)
  const int64_t nsr = solve_roles ? B : 0;
  if (gpart && gprows == 0 && !partials_done)   // chunk Gram partials first (absolute L^T addressing only)
    hipLaunchKernelGGL((gram_partial_kernel<NB>), dim3((unsigned)(B * gchunks)), dim3(64 * NB), 0, st, Lt, ldt, r,
                       sg, n, gchunks, gchunk, gpart);
  auto go = [&](auto kern) {
    constexpr int RH = NRB > 4 ? NRB / 4 : 1;   // row blocks per strip (the kernel's SNRB split)
    hipLaunchKernelGGL(kern, dim3((unsigned)(nsr + B * strips * msplit * RH)), dim3(S3_NT), 0, st, Lt, ldt, X, c1,
                       r, sg, n,
                       B, M, G, Gi, Gi32, stat, prec, eps, strips, lt_seg_rows, x_rel ? 1 : 0, gpart, gchunks,
                       gprows, msplit, Mpart, nsr);
  };
  if (solve_mode == 2) go(s3_reduce_solve_kernel<NRB, NB, 2>);
  else if (solve_mode == 1) go(s3_reduce_solve_kernel<NRB, NB, 1>);
  else go(s3_reduce_solve_kernel<NRB, NB, 0>);
  if (msplit > 1) {
    const int64_t count4 = B * r * c1 / 4;   // c1 % 8 == 0
    hipLaunchKernelGGL(m_split_reduce_kernel, dim3((unsigned)cdiv(count4, 256)), dim3(256), 0, st, Mpart, M, count4,
                       msplit);
  }
}

// The library's side stream per device, with a fork and a join event, so a
// solve that needs only the Gram partials runs beside the M strips: the
// caller's stream records `fork`, the side stream waits for it and runs the
// solve, records `join`, and the caller's stream waits for `join` before the
// apply.  Created on a device's first such forward (never while the caller's
// stream is being captured: that forward then runs the solve after the
// strips); default priority; kept until the process ends.  The lock spans
// each forward's record / wait sequence, so concurrent forwards on one
// device (from several host threads) each wait on their own records.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
constexpr int kSideDevices = 64;
std::mutex g_side_mu;
SideStream g_side[kSideDevices];

// Under g_side_mu: the current device's side stream, created if absent and
// the caller's stream is not capturing; false if unavailable.
bool side_stream_locked(hipStream_t caller, SideStream& out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kSideDevices) return false;
  SideStream& ss = g_side[dev];
  if (!ss.s) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(caller, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return false;
    SideStream n;
    if (hipStreamCreateWithFlags(&n.s, hipStreamNonBlocking) != hipSuccess) return false;
    if (hipEventCreateWithFlags(&n.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&n.join, hipEventDisableTiming) != hipSuccess) {
      if (n.fork) (void)hipEventDestroy(n.fork);
      (void)hipStreamDestroy(n.s);
      return false;
    }
    ss = n;
  }
  out = ss;
  return true;
}

// S3, S4 and S5, shared by every structure: M_b, G_b, Ginv_b, M'_b and
// R^T = W_res^T M'^T.  Needs L^T (Lt, pitch ldt) and X.
template <class C, class C3>
// gram_rows > 0: the first stage left Gram partials per tile of that many
// tokens in the workspace (else the chunk Gram kernel computes them here).
void forward_residual(const dyra_spec& s, const char* plan, const void* X, const SegInfo& si, float eps,
                      int solver, char* ws, hipStream_t st, const StageEvents& E, int64_t gram_rows = 0) {
  typedef typename C::elem T;
  constexpr bool BF = TT<T>::ESZ == 2;
  const int dtype = BF ? DYRA_BF16 : DYRA_F32;
  const PlanLayout PL = plan_layout(s, dtype);
  const WsLayout WL = si.layout(s, dtype);
  const int64_t B = si.B, n = si.n, c1 = s.c1, c2 = s.c2;
  const SegMap sg = si.map();
  const int r = s.r;
  const T* Wrt = reinterpret_cast<const T*>(plan + PL.Wrt);
  T* Lt = reinterpret_cast<T*>(ws + WL.Lt);
  float* G = reinterpret_cast<float*>(ws + WL.G);
  float* M = reinterpret_cast<float*>(ws + WL.M);
  double* Gi = reinterpret_cast<double*>(ws + WL.Ginv);
  float* Gi32 = reinterpret_cast<float*>(ws + WL.Gi32);
  T* Mp = reinterpret_cast<T*>(ws + WL.Mp);
  T* Rt = reinterpret_cast<T*>(ws + WL.Rt);
  int32_t* stat = reinterpret_cast<int32_t*>(ws + WL.status);
  int32_t* prec = reinterpret_cast<int32_t*>(ws + WL.prec);
  const int64_t ldt = lt_pitch(n);
  // AUTO takes the sweep at every supported r: on MI355X the sweep on one
  // workgroup, overlapping the strips inside the token-reduction launch,
  // beats Newton-Schulz at r = 64 (32 solves: about 23 against 120 us) and
  // matches it at r = 128, where Newton-Schulz runs beside the strips on the
  // side stream; Newton-Schulz and the Cholesky route stay selectable.
  const bool ns = solver == DYRA_SOLVER_NS;
  // solve inside the token-reduction launch: 1 the sweep, 2 the Cholesky
  // route, 0 none (Newton-Schulz runs after it: as the launch's 4-wave solve
  // role at r = 128 it took 155 us against 99 us for its own 8-wave launch,
  // more than the overlap with the strips gained).  At r = 128 a separate
  // 512-thread sweep launch is faster on its own (110 us against the
  // launch's 256-thread solve role) but the forward is slower, since the
  // solve role overlaps the strips.
  const int mode = ns ? 0 : (solver == DYRA_SOLVER_CHOL ? 2 : 1);
  // S3: M_b, G_b (bf16: with the sweep solve in the same launch)
  bool solved = false;
  if constexpr (BF) {
    const bf16_t* Xb = reinterpret_cast<const bf16_t*>(X);
    float* Gp = reinterpret_cast<float*>(ws + WL.Gp);
    const int gc = (int)WL.gchunks;
    const int64_t gk = WL.gchunk;
    const int ms = WL.msplit;
    float* Mpt = reinterpret_cast<float*>(ws + WL.Mpart);
    auto s3 = [&](bool roles, bool parts_done) {
      if (r <= 16) launch_s3_bf16<1, 1>(Lt, ldt, Xb, c1, r, sg, n, B, M, G, Gi, Gi32, stat, prec, eps, mode, st, 0, false, Gp, gc, gk, gram_rows, ms, Mpt, roles, parts_done);
      else if (r <= 32) launch_s3_bf16<2, 1>(Lt, ldt, Xb, c1, r, sg, n, B, M, G, Gi, Gi32, stat, prec, eps, mode, st, 0, false, Gp, gc, gk, gram_rows, ms, Mpt, roles, parts_done);
      else if (r <= 64) launch_s3_bf16<4, 2>(Lt, ldt, Xb, c1, r, sg, n, B, M, G, Gi, Gi32, stat, prec, eps, mode, st, 0, false, Gp, gc, gk, gram_rows, ms, Mpt, roles, parts_done);
      else launch_s3_bf16<8, 4>(Lt, ldt, Xb, c1, r, sg, n, B, M, G, Gi, Gi32, stat, prec, eps, mode, st, 0, false, Gp, gc, gk, gram_rows, ms, Mpt, roles, parts_done);
    };
    // Newton-Schulz needs only the Gram partials: on the side stream it runs
    // beside the M strips (a launch with no solve roles) instead of after
    // them; its workgroup sums G_b from the partials itself
    std::unique_lock<std::mutex> side_lock;
    SideStream side;
    bool fork = false;
    if (ns && E.fork && (gram_rows > 0 || gc > 0)) {
      side_lock = std::unique_lock<std::mutex>(g_side_mu);
      fork = side_stream_locked(st, side);
      if (!fork) side_lock.unlock();
    }
    if (fork) {
      if (gram_rows == 0) {   // chunk Gram partials first, on the caller's stream
        if (r <= 32)
          hipLaunchKernelGGL((gram_partial_kernel<1>), dim3((unsigned)(B * gc)), dim3(64), 0, st, Lt, ldt, r, sg, n,
                             gc, gk, Gp);
        else if (r <= 64)
          hipLaunchKernelGGL((gram_partial_kernel<2>), dim3((unsigned)(B * gc)), dim3(128), 0, st, Lt, ldt, r, sg, n,
                             gc, gk, Gp);
        else
          hipLaunchKernelGGL((gram_partial_kernel<4>), dim3((unsigned)(B * gc)), dim3(256), 0, st, Lt, ldt, r, sg, n,
                             gc, gk, Gp);
      }
      const float tol = kNsTolBf16, accept = kNsAcceptBf16;
      (void)hipEventRecord(side.fork, st);
      (void)hipStreamWaitEvent(side.s, side.fork, 0);
      hipLaunchKernelGGL(ns_inverse_kernel, dim3((unsigned)B), dim3(512), 0, side.s, G, Gi, Gi32, stat, prec, r, eps,
                         kNsMaxit, tol, accept, Gp, gc, gram_rows, sg);
      (void)hipEventRecord(side.join, side.s);
      s3(false, true);
      (void)hipStreamWaitEvent(st, side.join, 0);
      side_lock.unlock();
      solved = true;
    } else {
      s3(true, false);
      solved = mode != 0;
    }
  } else {
    const int tr = (int)cdiv(r, C3::BM), tcm = (int)cdiv(c1, C3::BN), tcg = (int)cdiv(r, C3::BN);
    const int64_t grid = B * tr * (tcm + tcg);
    hipLaunchKernelGGL(s3_gram_kernel<C3>, dim3((unsigned)grid), dim3(C3::NT), 0, st, Lt, ldt,
                       reinterpret_cast<const T*>(X), c1, r, sg, n, M, G, tr, tcm, tcg);
  }
  E.mark(2, st);
  // S4: Ginv_b (unless solved above), M'_b = Ginv_b M_b
  if (!solved) {
    if (ns) {
      // Newton-Schulz (the sweep for any segment it cannot solve).
      // ||I - A' X||_F bounds the relative error of the inverse: 1e-4 is far
      // below the bf16 rounding of M', fp32 storage asks for the fp32 floor
      // (fp32 storage: a stall above 1e-5 goes to the fp64 sweep, so an
      // ill-conditioned G still gives an fp32-accurate inverse)
      const float tol = BF ? kNsTolBf16 : 2e-6f, accept = BF ? kNsAcceptBf16 : 1e-5f;
      hipLaunchKernelGGL(ns_inverse_kernel, dim3((unsigned)B), dim3(512), 0, st, G, Gi, Gi32, stat, prec, r, eps,
                         kNsMaxit, tol, accept, nullptr, 0, (int64_t)0, sg);
    } else if (solver == DYRA_SOLVER_CHOL) {
      launch_chol(G, Gi, Gi32, stat, prec, r, eps, B, st);
    } else {
      launch_sweep(G, Gi, Gi32, stat, prec, r, eps, B, st);
    }
  }
  launch_apply_inverse<T>(Gi, Gi32, M, Mp, B, r, c1, stat, prec, st);
  E.mark(3, st);
  // S5: R^T (c2 x B r) = W_res^T (c2 x c1) . M' (B r x c1)^T; bf16: split
  // over K when the output has few tiles, else the persistent output kernel
  // with one segment, no residual part and no bias
  if constexpr (BF) {
    const S5Split sp = s5_split(c2, B * r, c1);
    if (sp.slices > 1) {
      typedef CfgB Cs;
      float* Pk = reinterpret_cast<float*>(ws + WL.Pk);
      const int tiles_n = (int)cdiv(B * r, Cs::BN);
      const int tiles = (int)(cdiv(c2, Cs::BM) * tiles_n);
      hipLaunchKernelGGL(gemm_tn_splitk_kernel<Cs>, dim3((unsigned)(tiles * sp.slices)), dim3(Cs::NT), 0, st,
                         reinterpret_cast<const char*>(Wrt), c1 * 2, reinterpret_cast<const char*>(Mp), c1 * 2, Pk,
                         c2, B * r, c1, sp.kslice, tiles_n, tiles);
      const int64_t mn = c2 * B * r;
      hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)cdiv(mn, 256 * 8)), dim3(256), 0, st, Pk,
                         reinterpret_cast<bf16_t*>(Rt), mn, sp.slices);
      return;
    }
    if (s6_ws_fits(c2, B * r, (int)c1, 0, 1) && device_cus() >= 8) {
      launch_s6_ws(Wrt, c1, 0, nullptr, 0, Mp, nullptr, nullptr, Rt, c2, B * r, (int)c1, 0, SegMap{nullptr, c2, 1, c2},
                   1, st);
      return;
    }
  }
  launch_gemm_tn<C>(Wrt, c1, Mp, c1, Rt, B * r, c2, B * r, c1, nullptr, st);
}

typedef GemmCfg<bf16_t, 128, 64, 2, 2> CfgL;   // left ALS step: L_b = X_b Z_b (r <= 64 columns per tile)

// One left ALS half-step on the bf16 workspace: R^T -> R; K_b = R_b R_b^T and
// Q_b^T = R_b W_res^T (fp32) with (K_b + lambda_b I)^-1 by the sweep; Z_b^T;
// then L_b = X_b Z_b overwrites L (and L^T) in the workspace.  The step does
// not involve the static branch: only where L sits in the first-stage output
// depends on the structure (column lcol of rows of pitch ldo: k / k + r
// low-rank, c / c + r Monarch, nb rb / nb rb + r BLAST).
void left_step_bf16(const dyra_spec& s, const char* plan, const bf16_t* X, const SegInfo& si, float eps,
                    char* ws, hipStream_t st, int half_steps, int lcol, int64_t ldo) {
  const PlanLayout PL = plan_layout(s, DYRA_BF16);
  const WsLayout WL = si.layout(s, DYRA_BF16, half_steps);
  const int64_t B = si.B, n = si.n, c1 = s.c1, c2 = s.c2;
  const int r = s.r;
  const bf16_t* Rt = reinterpret_cast<const bf16_t*>(ws + WL.Rt);
  bf16_t* R = reinterpret_cast<bf16_t*>(ws + WL.R);
  float* K = reinterpret_cast<float*>(ws + WL.K);
  double* Kinv = reinterpret_cast<double*>(ws + WL.Kinv);
  float* Ki32 = reinterpret_cast<float*>(ws + WL.Ki32);
  float* Qt = reinterpret_cast<float*>(ws + WL.Qt);
  bf16_t* Zt = reinterpret_cast<bf16_t*>(ws + WL.Zt);
  int32_t* kst = reinterpret_cast<int32_t*>(ws + WL.kstatus);
  int32_t* kpr = reinterpret_cast<int32_t*>(ws + WL.kprec);
  const bf16_t* Wrt = reinterpret_cast<const bf16_t*>(plan + PL.Wrt);
  // R [B r x c2] = (R^T [c2 x B r])^T
  hipLaunchKernelGGL(transpose_b16_kernel, dim3((unsigned)(cdiv(c2, 64) * cdiv(B * r, 64))), dim3(256), 0, st, Rt, R,
                     c2, B * r);
  // K_b, Q_b^T, (K_b + lambda I)^-1: c2 is the reduction ("token") axis
  const int64_t nn = B * c2;
  if (r <= 16) launch_s3_bf16<1, 1>(R, c2, Wrt, c1, r, SegMap{nullptr, c2, B, nn}, nn, B, Qt, K, Kinv, Ki32, kst, kpr, eps, 1, st, r, true);
  else if (r <= 32) launch_s3_bf16<2, 1>(R, c2, Wrt, c1, r, SegMap{nullptr, c2, B, nn}, nn, B, Qt, K, Kinv, Ki32, kst, kpr, eps, 1, st, r, true);
  else if (r <= 64) launch_s3_bf16<4, 2>(R, c2, Wrt, c1, r, SegMap{nullptr, c2, B, nn}, nn, B, Qt, K, Kinv, Ki32, kst, kpr, eps, 1, st, r, true);
  else launch_s3_bf16<8, 4>(R, c2, Wrt, c1, r, SegMap{nullptr, c2, B, nn}, nn, B, Qt, K, Kinv, Ki32, kst, kpr, eps, 1, st, r, true);
  launch_apply_inverse<bf16_t>(Kinv, Ki32, Qt, Zt, B, r, c1, kst, kpr, st);
  // L_b = X_b Z_b into [T | L] and L^T
  const int tiles_n = (int)cdiv(r, CfgL::BN);
  hipLaunchKernelGGL(s1_left_kernel<CfgL>, dim3((unsigned)(cdiv(n, CfgL::BM) * tiles_n)), dim3(CfgL::NT), 0, st, X,
                     Zt, reinterpret_cast<bf16_t*>(ws + WL.A), reinterpret_cast<bf16_t*>(ws + WL.Lt), n, c1, lcol, r,
                     si.map(), lt_pitch(n), tiles_n, ldo);
}

// One left ALS half-step on the fp32 workspace (low-rank; fp32 storage
// exists for no other structure): R = (R^T)^T; K_b = R_b R_b^T and
// Q_b^T = R_b W_res^T by the fp32 token reduction with c2 as its token axis
// (one launch per segment: that kernel addresses tokens absolutely); the
// sweep's (K_b + lambda_b I)^-1; Z_b^T = (K_b + lambda_b I)^-1 Q_b^T; then
// L_b = X_b Z_b by the batched engine GEMM into the L columns of [T | L],
// and L^T again for the next right step.
void left_step_f32(const dyra_spec& s, const char* plan, const float* X, const SegInfo& si, float eps,
                   char* ws, hipStream_t st, int half_steps) {
  const PlanLayout PL = plan_layout(s, DYRA_F32);
  const WsLayout WL = si.layout(s, DYRA_F32, half_steps);
  const int64_t B = si.B, n = si.n, seg = si.seg, c1 = s.c1, c2 = s.c2;
  const int r = s.r, k = s.k;
  const float* Rt = reinterpret_cast<const float*>(ws + WL.Rt);
  float* R = reinterpret_cast<float*>(ws + WL.R);
  float* K = reinterpret_cast<float*>(ws + WL.K);
  double* Kinv = reinterpret_cast<double*>(ws + WL.Kinv);
  float* Ki32 = reinterpret_cast<float*>(ws + WL.Ki32);
  float* Qt = reinterpret_cast<float*>(ws + WL.Qt);
  float* Zt = reinterpret_cast<float*>(ws + WL.Zt);
  int32_t* kst = reinterpret_cast<int32_t*>(ws + WL.kstatus);
  int32_t* kpr = reinterpret_cast<int32_t*>(ws + WL.kprec);
  const float* Wrt = reinterpret_cast<const float*>(plan + PL.Wrt);
  float* TL = reinterpret_cast<float*>(ws + WL.A);
  float* Lt = reinterpret_cast<float*>(ws + WL.Lt);
  // R [B r x c2] = (R^T [c2 x B r])^T
  hipLaunchKernelGGL(transpose_b32_kernel, dim3((unsigned)(cdiv(c2, 64) * cdiv(B * r, 64))), dim3(256), 0, st, Rt,
                     B * r, R, c2, c2, B * r);
  const int tr = (int)cdiv(r, CfgF3::BM), tcm = (int)cdiv(c1, CfgF3::BN), tcg = (int)cdiv(r, CfgF3::BN);
  for (int64_t b = 0; b < B; ++b)
    hipLaunchKernelGGL(s3_gram_kernel<CfgF3>, dim3((unsigned)(tr * (tcm + tcg))), dim3(CfgF3::NT), 0, st,
                       R + b * r * c2, c2, Wrt, c1, r, SegMap{nullptr, c2, 1, c2}, c2, Qt + b * r * c1, K + b * r * r,
                       tr, tcm, tcg);
  launch_sweep(K, Kinv, Ki32, kst, kpr, r, eps, B, st);
  launch_apply_inverse<float>(Kinv, Ki32, Qt, Zt, B, r, c1, kst, kpr, st);
  // L_b [s_b x r] = X_b [s_b x c1] . (Z_b^T [r x c1])^T at column k of [T | L]
  // (one batched launch for uniform segments, one launch per ragged one)
  if (!si.off_host) {
    launch_gemm_tn<CfgF>(X, c1, Zt, c1, TL + k, k + r, seg, r, c1, nullptr, st, (int)B, seg * c1, (int64_t)r * c1,
                         seg * (k + r));
  } else {
    for (int64_t b = 0; b < B; ++b) {
      const int64_t lo = si.off_host[b], len = si.off_host[b + 1] - lo;
      launch_gemm_tn<CfgF>(X + lo * c1, c1, Zt + b * r * c1, c1, TL + lo * (k + r) + k, k + r, len, r, c1, nullptr,
                           st);
    }
  }
  // L^T [r x ldt] = (L [n x r], pitch k + r)^T
  hipLaunchKernelGGL(transpose_b32_kernel, dim3((unsigned)(cdiv(n, 64) * cdiv(r, 64))), dim3(256), 0, st, TL + k,
                     (int64_t)(k + r), Lt, lt_pitch(n), n, (int64_t)r);
}

template <class C, class C3, class C6>
int forward_lowrank(const dyra_spec& s, const char* plan, const void* X, const void* bias, void* Y,
                    const SegInfo& si, float eps, int solver, char* ws, hipStream_t st,
                    const StageEvents& E, int half_steps = 2) {
  typedef typename C::elem T;
  const int dtype = TT<T>::ESZ == 2 ? DYRA_BF16 : DYRA_F32;
  const PlanLayout PL = plan_layout(s, dtype);
  const WsLayout WL = si.layout(s, dtype);
  const int64_t B = si.B, n = si.n, c1 = s.c1, c2 = s.c2;
  const int k = s.k, r = s.r;
  T* TL = reinterpret_cast<T*>(ws + WL.A);
  T* Lt = reinterpret_cast<T*>(ws + WL.Lt);
  T* Rt = reinterpret_cast<T*>(ws + WL.Rt);
  int64_t gram_rows = 0;
  E.mark(0, st);
  {  // S1: [T | L] = X [U | P], L^T
    auto launch = [&](auto cfg) {
      typedef decltype(cfg) C1;
      const int tiles_n = (int)cdiv(k + r, C1::BN);
      const int64_t tiles = cdiv(n, C1::BM) * tiles_n;
      hipLaunchKernelGGL(s1_lowrank_kernel<C1>, dim3((unsigned)tiles), dim3(C1::NT), 0, st,
                         reinterpret_cast<const T*>(X), reinterpret_cast<const T*>(plan + PL.UPt), TL, Lt, n, c1, k,
                         r, lt_pitch(n), tiles_n, (int64_t)(k + r));
    };
    // 128 x 128 tiles leave k + r in (256, 320] as 2.5 column tiles and, at
    // ViT-L sizes, more tiles than two per CU: one 160 x 320 tile per row
    // block instead (a single round, X read once per row block)
    if constexpr (TT<T>::ESZ == 2) {
      if (s1_tile_shape(s, DYRA_BF16)) {
        // Gram partials from the tile epilogue when a tile meets at most two
        // segments and r fills whole 32 x 32 blocks
        const bool gram = (r == 32 || r == 64) && si.min_len >= S1T_BM;
        if (gram) gram_rows = S1T_BM;
        hipLaunchKernelGGL(s1_tile_kernel, dim3((unsigned)cdiv(n, S1T_BM)), dim3(512), 0, st,
                           reinterpret_cast<const bf16_t*>(X), reinterpret_cast<const bf16_t*>(plan + PL.UPt),
                           reinterpret_cast<bf16_t*>(TL), reinterpret_cast<bf16_t*>(Lt), (int)n, (int)c1, k, r,
                           lt_pitch(n), gram ? reinterpret_cast<float*>(ws + WL.Gp) : nullptr, si.map());
      } else if (k + r > 256 && k + r <= 320) launch(CfgB1W());
      else launch(C());
    } else {
      launch(C());
    }
  }
  E.mark(1, st);
  forward_residual<C, C3>(s, plan, X, si, eps, solver, ws, st, E, gram_rows);
  // further ALS half-steps: left (L from R), right (R from L), ...
  for (int h = 2; h < half_steps; ++h) {
    if (h % 2 == 0) {
      if constexpr (TT<T>::ESZ == 2)
        left_step_bf16(s, plan, reinterpret_cast<const bf16_t*>(X), si, eps, ws, st, half_steps, k,
                       (int64_t)(k + r));
      else
        left_step_f32(s, plan, reinterpret_cast<const float*>(X), si, eps, ws, st, half_steps);
    } else {
      forward_residual<C, C3>(s, plan, X, si, eps, solver, ws, st, StageEvents{nullptr, 0});
    }
  }
  E.mark(4, st);
  {  // S6: Y = T V + L R_b + bias
    const int tiles_n = (int)cdiv(c2, C6::BN);
    const int64_t tiles = cdiv(n, C6::BM) * tiles_n;
    constexpr bool BF = TT<T>::ESZ == 2;
    if (BF && s6_ws_fits(n, c2, k, r, B) && device_cus() >= 8)
      launch_s6_ws(reinterpret_cast<const bf16_t*>(TL), k + r, 0, nullptr, 0,
                   reinterpret_cast<const bf16_t*>(plan + PL.Vt), reinterpret_cast<const bf16_t*>(Rt),
                   reinterpret_cast<const bf16_t*>(bias), reinterpret_cast<bf16_t*>(Y), n, c2, k, r, si.map(), B, st);
    else
      hipLaunchKernelGGL((s6_lowrank_kernel<C6, BF, true, BF ? S6_WPE : 1, BF>), dim3((unsigned)tiles), dim3(C6::NT), 0,
                         st, TL, reinterpret_cast<const T*>(plan + PL.Vt), Rt, reinterpret_cast<const T*>(bias),
                         reinterpret_cast<T*>(Y), n, c2, k, r, si.map(), B, tiles_n);
  }
  E.mark(5, st);
  return hipGetLastError() == hipSuccess ? DYRA_OK : DYRA_EHIP;
}

template <int RB>
void launch_monarch(const bf16_t* X, const char* plan, const PlanLayout& PL, bf16_t* A, bf16_t* Lt, int64_t n,
                    int r, int64_t ldt, hipStream_t st) {
  hipLaunchKernelGGL((s1_monarch_kernel<RB>), dim3((unsigned)cdiv(n, 32)), dim3(256), 0, st, X,
                     reinterpret_cast<const bf16_t*>(plan + PL.Pt), A, Lt, n, r, ldt);
}

void launch_monarch6(const bf16_t* X, const bf16_t* A, const char* plan, const PlanLayout& PL, const bf16_t* Rt,
                     const bf16_t* bias, bf16_t* Y, int64_t n, int r, SegMap sg, int64_t B, hipStream_t st) {
  hipLaunchKernelGGL(s6_monarch_fused_kernel, dim3((unsigned)cdiv(n, 32)), dim3(256), 0, st, X,
                     reinterpret_cast<const bf16_t*>(plan + PL.B1t), reinterpret_cast<const bf16_t*>(plan + PL.B2t), A,
                     Rt, bias, Y, n, r, sg, B);
}

int forward_monarch(const dyra_spec& s, const char* plan, const void* X, const void* bias, void* Y,
                    const SegInfo& si, float eps, int solver, char* ws, hipStream_t st, const StageEvents& E,
                    int half_steps = 2) {
  const PlanLayout PL = plan_layout(s, DYRA_BF16);
  const WsLayout WL = si.layout(s, DYRA_BF16);
  const int64_t B = si.B, n = si.n;
  const int r = s.r;
  bf16_t* A = reinterpret_cast<bf16_t*>(ws + WL.A);
  bf16_t* Lt = reinterpret_cast<bf16_t*>(ws + WL.Lt);
  const bf16_t* Xb = reinterpret_cast<const bf16_t*>(X);
  const int64_t ldt = lt_pitch(n);
  E.mark(0, st);
  if (r <= 32) launch_monarch<1>(Xb, plan, PL, A, Lt, n, r, ldt, st);
  else if (r <= 64) launch_monarch<2>(Xb, plan, PL, A, Lt, n, r, ldt, st);
  else launch_monarch<4>(Xb, plan, PL, A, Lt, n, r, ldt, st);
  E.mark(1, st);
  forward_residual<CfgB, CfgB3>(s, plan, X, si, eps, solver, ws, st, E);
  for (int h = 2; h < half_steps; ++h) {   // further ALS half-steps (L sits after the C = m^2 V columns)
    if (h % 2 == 0) left_step_bf16(s, plan, Xb, si, eps, ws, st, half_steps, MO * MO, MO * MO + r);
    else forward_residual<CfgB, CfgB3>(s, plan, X, si, eps, solver, ws, st, StageEvents{nullptr, 0});
  }
  E.mark(4, st);
  const bf16_t* Rt = reinterpret_cast<const bf16_t*>(ws + WL.Rt);
  const bf16_t* bb = reinterpret_cast<const bf16_t*>(bias);
  bf16_t* Yb = reinterpret_cast<bf16_t*>(Y);
  launch_monarch6(Xb, A, plan, PL, Rt, bb, Yb, n, r, si.map(), B, st);
  E.mark(5, st);
  return hipGetLastError() == hipSuccess ? DYRA_OK : DYRA_EHIP;
}

int forward_blast(const dyra_spec& s, const char* plan, const void* X, const void* bias, void* Y,
                  const SegInfo& si, float eps, int solver, char* ws, hipStream_t st, const StageEvents& E,
                  int half_steps = 2) {
  const PlanLayout PL = plan_layout(s, DYRA_BF16);
  const WsLayout WL = si.layout(s, DYRA_BF16);
  const int64_t B = si.B, n = si.n, c1 = s.c1, c2 = s.c2;
  const int r = s.r, nb = s.nb, rb = s.rb;
  const int64_t b1 = c1 / nb, b2 = c2 / nb, NR = (int64_t)nb * rb, ldzl = NR + r;
  bf16_t* ZL = reinterpret_cast<bf16_t*>(ws + WL.A);
  bf16_t* Wp = reinterpret_cast<bf16_t*>(ws + WL.Wp);
  bf16_t* Lt = reinterpret_cast<bf16_t*>(ws + WL.Lt);
  const bf16_t* Xb = reinterpret_cast<const bf16_t*>(X);
  E.mark(0, st);
  // S1: Z_i = X_i U_i for every block row i (batched), and L = X P with L^T
  launch_gemm_tn<CfgB>(Xb, c1, plan + PL.Ubt, b1, ZL, ldzl, n, rb, b1, nullptr, st, nb, b1, (int64_t)rb * b1, rb);
  {
    const int tiles_n = (int)cdiv(r, CfgB::BN);
    const int64_t tiles = cdiv(n, CfgB::BM) * tiles_n;
    // L = X P has r columns only: split over K when its tiles are few
    const S5Split sl = s5_split(n, r, c1);
    if (sl.slices > 1) {
      float* Pk = reinterpret_cast<float*>(ws + WL.Pk);
      hipLaunchKernelGGL(gemm_tn_splitk_kernel<CfgB>, dim3((unsigned)(tiles * sl.slices)), dim3(CfgB::NT), 0, st,
                         reinterpret_cast<const char*>(Xb), c1 * 2, plan + PL.Pt, c1 * 2, Pk, n, (int64_t)r, c1,
                         sl.kslice, tiles_n, (int)tiles);
      hipLaunchKernelGGL(splitk_reduce_lt_kernel, dim3((unsigned)cdiv(lt_pitch(n), SRL_T)), dim3(256), 0, st, Pk,
                         sl.slices, n, r, ZL + NR, ldzl, Lt, lt_pitch(n));
    } else {
      hipLaunchKernelGGL(s1_lowrank_kernel<CfgB>, dim3((unsigned)tiles), dim3(CfgB::NT), 0, st, Xb,
                         reinterpret_cast<const bf16_t*>(plan + PL.Pt), ZL + NR, Lt, n, c1, 0, r, lt_pitch(n),
                         tiles_n, ldzl);
    }
  }
  E.mark(1, st);
  forward_residual<CfgB, CfgB3>(s, plan, X, si, eps, solver, ws, st, E);
  for (int h = 2; h < half_steps; ++h) {   // further ALS half-steps (L sits after the nb rb Z columns)
    if (h % 2 == 0) left_step_bf16(s, plan, Xb, si, eps, ws, st, half_steps, (int)NR, ldzl);
    else forward_residual<CfgB, CfgB3>(s, plan, X, si, eps, solver, ws, st, StageEvents{nullptr, 0});
  }
  if (s.kind == DYRA_BLAST_DIAG) {
    // coupling W'_j = sum_i Z_i diag(s_ij): elementwise over the block grid
    const int zt = (int)std::max<int64_t>(1, std::min<int64_t>(8, (BDC_LDS / 2) / NR));
    const int64_t groups = cdiv(n, zt);
    hipLaunchKernelGGL(blast_diag_coupling_kernel, dim3((unsigned)std::min<int64_t>(groups, 4096)), dim3(256), 0, st,
                       ZL, ldzl, reinterpret_cast<const bf16_t*>(plan + PL.St), Wp, NR, n, nb, rb, zt);
  } else {
    // coupling W' = Z S (dense over the nb x nb grid of rb x rb blocks)
    launch_gemm_tn<CfgB>(ZL, ldzl, plan + PL.St, NR, Wp, NR, n, NR, NR, nullptr, st);
  }
  E.mark(4, st);
  {
    typedef CfgB6 C6;
    const bf16_t* Rt = reinterpret_cast<const bf16_t*>(ws + WL.Rt);
    // the persistent output kernel: part 0 is W'_j V_j^T (W' columns of the
    // tile's block column j, V_j rows = the tile's output columns of Vb read
    // as a [c2 x rb] matrix), part 1 is L R_b
    if (b2 % CfgB6W::BN == 0 && s6_ws_fits(n, c2, rb, r, B, std::max<int64_t>(NR, ldzl)) && device_cus() >= 8) {
      launch_s6_ws(Wp, NR, b2, ZL + NR, ldzl, reinterpret_cast<const bf16_t*>(plan + PL.Vb), Rt,
                   reinterpret_cast<const bf16_t*>(bias), reinterpret_cast<bf16_t*>(Y), n, c2, rb, r, si.map(), B,
                   st);
    } else if (b2 % C6::BN == 0) {
      const int tiles_n = (int)(c2 / C6::BN);
      const int64_t tiles = cdiv(n, C6::BM) * tiles_n;
      hipLaunchKernelGGL(s6_blast_kernel<C6>, dim3((unsigned)tiles), dim3(C6::NT), 0, st, Wp, NR, ZL, ldzl, NR,
                         reinterpret_cast<const bf16_t*>(plan + PL.Vb), Rt, reinterpret_cast<const bf16_t*>(bias),
                         reinterpret_cast<bf16_t*>(Y), n, c2, b2, rb, r, si.map(), B, tiles_n);
    } else {
      const int tiles_n = (int)(c2 / CfgB::BN);
      const int64_t tiles = cdiv(n, CfgB::BM) * tiles_n;
      hipLaunchKernelGGL(s6_blast_kernel<CfgB>, dim3((unsigned)tiles), dim3(CfgB::NT), 0, st, Wp, NR, ZL, ldzl, NR,
                         reinterpret_cast<const bf16_t*>(plan + PL.Vb), Rt, reinterpret_cast<const bf16_t*>(bias),
                         reinterpret_cast<bf16_t*>(Y), n, c2, b2, rb, r, si.map(), B, tiles_n);
    }
  }
  E.mark(5, st);
  return hipGetLastError() == hipSuccess ? DYRA_OK : DYRA_EHIP;
}

// half_steps: 2 t of the ALS (2: t = 1; 3: t = 1.5; 4: t = 2), for every
// structure and storage type the forward takes.
int check_als(const dyra_spec& spec, int32_t dtype, int32_t half_steps) {
  (void)spec;
  (void)dtype;
  if (half_steps < 2 || half_steps > 4) return DYRA_EINVAL;
  return DYRA_OK;
}

int check_forward_args(const dyra_spec* spec, const void* plan, const void* X, void* Y, int64_t B, int64_t s,
                       int32_t dtype, float eps, int32_t solver, void* ws, size_t ws_bytes, int32_t half_steps = 2) {
  if (!spec || !plan || !X || !Y || !ws) return DYRA_EINVAL;
  int rc = validate_spec(spec);
  if (rc) return rc;
  rc = validate_dtype(*spec, dtype);
  if (rc) return rc;
  if (!(eps >= 0.f) || !std::isfinite(eps)) return DYRA_EINVAL;
  if (solver < DYRA_SOLVER_AUTO || solver > DYRA_SOLVER_NS) return DYRA_EINVAL;
  if (B <= 0 || s <= 0 || B >= ((int64_t)1 << 31) || s >= ((int64_t)1 << 31)) return DYRA_ESHAPE;
  if (B * s >= ((int64_t)1 << 31)) return DYRA_ESHAPE;
  if ((reinterpret_cast<uintptr_t>(plan) | reinterpret_cast<uintptr_t>(X) | reinterpret_cast<uintptr_t>(Y) |
       reinterpret_cast<uintptr_t>(ws)) & 15)
    return DYRA_EINVAL;
  rc = check_als(*spec, dtype, half_steps);
  if (rc) return rc;
  if (ws_bytes < ws_layout(*spec, B, s, dtype, half_steps).total) return DYRA_EWORKSPACE;
  return DYRA_OK;
}

}  // namespace

extern "C" int dyra_workspace_size(const dyra_spec* spec, int64_t B, int64_t s, int32_t dtype, size_t* bytes) {
  if (!spec || !bytes) return DYRA_EINVAL;
  int rc = validate_spec(spec);
  if (rc) return rc;
  rc = validate_dtype(*spec, dtype);
  if (rc) return rc;
  if (B <= 0 || s <= 0 || B * s >= ((int64_t)1 << 31)) return DYRA_ESHAPE;
  *bytes = ws_layout(*spec, B, s, dtype).total;
  return DYRA_OK;
}

extern "C" int dyra_workspace_size_als(const dyra_spec* spec, int64_t B, int64_t s, int32_t dtype,
                                       int32_t half_steps, size_t* bytes) {
  if (!spec || !bytes) return DYRA_EINVAL;
  int rc = validate_spec(spec);
  if (rc) return rc;
  rc = validate_dtype(*spec, dtype);
  if (rc) return rc;
  rc = check_als(*spec, dtype, half_steps);
  if (rc) return rc;
  if (B <= 0 || s <= 0 || B * s >= ((int64_t)1 << 31)) return DYRA_ESHAPE;
  *bytes = ws_layout(*spec, B, s, dtype, half_steps).total;
  return DYRA_OK;
}

namespace {
// The forward on validated arguments.
int dispatch(const dyra_spec* spec, const void* plan, const void* X, const void* bias, void* Y, const SegInfo& si,
             int32_t dtype, float ridge_eps, int32_t solver, void* workspace, void* stream, const StageEvents& E,
             int32_t half_steps) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const char* plan_c = reinterpret_cast<const char*>(plan);
  char* ws = reinterpret_cast<char*>(workspace);
  if (spec->kind == DYRA_MONARCH)
    return forward_monarch(*spec, plan_c, X, bias, Y, si, ridge_eps, solver, ws, st, E, half_steps);
  if (is_blast(spec->kind))
    return forward_blast(*spec, plan_c, X, bias, Y, si, ridge_eps, solver, ws, st, E, half_steps);
  if (dtype == DYRA_BF16)
    return forward_lowrank<CfgB, CfgB3, CfgB6>(*spec, plan_c, X, bias, Y, si, ridge_eps, solver, ws, st, E,
                                               half_steps);
  return forward_lowrank<CfgF, CfgF3, CfgF>(*spec, plan_c, X, bias, Y, si, ridge_eps, solver, ws, st, E,
                                            half_steps);
}

int forward_impl(const dyra_spec* spec, const void* plan, const void* X, const void* bias, void* Y, int64_t B,
                 int64_t s, int32_t dtype, float ridge_eps, int32_t solver, void* workspace, size_t ws_bytes,
                 void* stream, const StageEvents& E, int32_t half_steps = 2) {
  int rc = check_forward_args(spec, plan, X, Y, B, s, dtype, ridge_eps, solver, workspace, ws_bytes, half_steps);
  if (rc) return rc;
  if (bias && (reinterpret_cast<uintptr_t>(bias) & 15)) return DYRA_EINVAL;
  return dispatch(spec, plan, X, bias, Y, SegInfo::uniform(B, s), dtype, ridge_eps, solver, workspace, stream, E,
                  half_steps);
}

// Ragged segments from host row offsets off[0 .. B] (off[0] = 0, every
// segment at least one row, off[B] = n < 2^31); off_dev is the caller's
// device copy (may be null when only sizes are wanted).
int varlen_info(int64_t B, const int64_t* off, const int32_t* off_dev, SegInfo& si) {
  if (!off) return DYRA_EINVAL;
  if (B <= 0 || B >= ((int64_t)1 << 31)) return DYRA_ESHAPE;
  if (off[0] != 0) return DYRA_ESHAPE;
  int64_t mx = 0, mn = INT64_MAX;
  for (int64_t b = 0; b < B; ++b) {
    const int64_t len = off[b + 1] - off[b];
    if (len < 1) return DYRA_ESHAPE;
    mx = std::max(mx, len);
    mn = std::min(mn, len);
  }
  if (off[B] >= ((int64_t)1 << 31)) return DYRA_ESHAPE;
  if (off_dev && (reinterpret_cast<uintptr_t>(off_dev) & 3)) return DYRA_EINVAL;
  si = SegInfo{};
  si.B = B;
  si.n = off[B];
  si.seg = 0;
  si.max_len = mx;
  si.min_len = mn;
  si.off_dev = off_dev;
  si.off_host = off;
  return DYRA_OK;
}
}  // namespace

extern "C" int dyra_workspace_size_varlen_als(const dyra_spec* spec, int64_t B, const int64_t* offsets,
                                              int32_t dtype, int32_t half_steps, size_t* bytes) {
  if (!spec || !bytes) return DYRA_EINVAL;
  int rc = validate_spec(spec);
  if (rc) return rc;
  rc = validate_dtype(*spec, dtype);
  if (rc) return rc;
  rc = check_als(*spec, dtype, half_steps);
  if (rc) return rc;
  SegInfo si;
  rc = varlen_info(B, offsets, nullptr, si);
  if (rc) return rc;
  *bytes = si.layout(*spec, dtype, half_steps).total;
  return DYRA_OK;
}

extern "C" int dyra_workspace_size_varlen(const dyra_spec* spec, int64_t B, const int64_t* offsets, int32_t dtype,
                                          size_t* bytes) {
  return dyra_workspace_size_varlen_als(spec, B, offsets, dtype, 2, bytes);
}

extern "C" int dyra_forward_varlen_als(const dyra_spec* spec, const void* plan, const void* X, const void* bias,
                                       void* Y, int64_t B, const int64_t* offsets, const int32_t* offsets_dev,
                                       int32_t dtype, float ridge_eps, int32_t solver, int32_t half_steps,
                                       int32_t* status_out, void* workspace, size_t ws_bytes, void* stream) {
  if (!offsets_dev) return DYRA_EINVAL;
  SegInfo si;
  int rc = varlen_info(B, offsets, offsets_dev, si);
  if (rc) return rc;
  // the uniform checks with one segment of all n rows, then the ragged size
  rc = check_forward_args(spec, plan, X, Y, 1, si.n, dtype, ridge_eps, solver, workspace, (size_t)-1, half_steps);
  if (rc) return rc;
  if (bias && (reinterpret_cast<uintptr_t>(bias) & 15)) return DYRA_EINVAL;
  if (status_out && (reinterpret_cast<uintptr_t>(status_out) & 3)) return DYRA_EINVAL;
  const WsLayout WL = si.layout(*spec, dtype, half_steps);
  if (ws_bytes < WL.total) return DYRA_EWORKSPACE;
  rc = dispatch(spec, plan, X, bias, Y, si, dtype, ridge_eps, solver, workspace, stream, StageEvents{nullptr, 0},
                half_steps);
  if (rc || !status_out) return rc;
  if (hipMemcpyAsync(status_out, reinterpret_cast<const char*>(workspace) + WL.status, (size_t)B * 4,
                     hipMemcpyDeviceToDevice, reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return DYRA_EHIP;
  return DYRA_OK;
}

extern "C" int dyra_forward_varlen(const dyra_spec* spec, const void* plan, const void* X, const void* bias,
                                   void* Y, int64_t B, const int64_t* offsets, const int32_t* offsets_dev,
                                   int32_t dtype, float ridge_eps, int32_t solver, int32_t* status_out,
                                   void* workspace, size_t ws_bytes, void* stream) {
  return dyra_forward_varlen_als(spec, plan, X, bias, Y, B, offsets, offsets_dev, dtype, ridge_eps, solver, 2,
                                 status_out, workspace, ws_bytes, stream);
}

extern "C" int dyra_forward(const dyra_spec* spec, const void* plan, const void* X, const void* bias, void* Y,
                            int64_t B, int64_t s, int32_t dtype, float ridge_eps, int32_t solver,
                            void* workspace, size_t ws_bytes, void* stream) {
  return forward_impl(spec, plan, X, bias, Y, B, s, dtype, ridge_eps, solver, workspace, ws_bytes, stream,
                      StageEvents{nullptr, 0});
}

extern "C" int dyra_forward_als(const dyra_spec* spec, const void* plan, const void* X, const void* bias, void* Y,
                                int64_t B, int64_t s, int32_t dtype, float ridge_eps, int32_t solver,
                                int32_t half_steps, void* workspace, size_t ws_bytes, void* stream) {
  return forward_impl(spec, plan, X, bias, Y, B, s, dtype, ridge_eps, solver, workspace, ws_bytes, stream,
                      StageEvents{nullptr, 0}, half_steps);
}

extern "C" int dyra_forward_events(const dyra_spec* spec, const void* plan, const void* X, const void* bias,
                                   void* Y, int64_t B, int64_t s, int32_t dtype, float ridge_eps,
                                   int32_t solver, void* workspace, size_t ws_bytes, void* stream,
                                   void* const* events, int32_t nevents) {
  if (nevents < 0 || (nevents > 0 && !events)) return DYRA_EINVAL;
  return forward_impl(spec, plan, X, bias, Y, B, s, dtype, ridge_eps, solver, workspace, ws_bytes, stream,
                      StageEvents{events, nevents});
}

// ---------------------------------------------------------------------------
// Allocation-free forward: the workspace is this file-scope device array,
// one copy per GPU the library runs on, held until the process ends.  Host
// code never passes the array's name to a kernel or copy (on the host it is
// a stand-in, not a device address): each device's address comes from
// hipGetSymbolAddress, taken once per device on the first call made with
// that device current, and only that address is used.
// ---------------------------------------------------------------------------
static __device__ __align__(256) char scratch[DYRA_NOALLOC_MAX_WORKSPACE];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {nullptr};

int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DYRA_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DYRA_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DYRA_OK;
}
}  // namespace

extern "C" int dyra_forward_noalloc(const dyra_spec* spec, const void* plan, const void* X, const void* bias,
                                    void* Y, int64_t B, int64_t s, int32_t dtype, float ridge_eps, int32_t solver,
                                    int32_t* status_out, void* stream) {
  // every argument and the size limit are checked before any HIP call
  const void* not_null = plan;
  int rc = check_forward_args(spec, plan, X, Y, B, s, dtype, ridge_eps, solver, const_cast<void*>(not_null),
                              (size_t)DYRA_NOALLOC_MAX_WORKSPACE);
  if (rc) return rc;
  if (bias && (reinterpret_cast<uintptr_t>(bias) & 15)) return DYRA_EINVAL;
  if (status_out && (reinterpret_cast<uintptr_t>(status_out) & 3)) return DYRA_EINVAL;
  void* ws = nullptr;
  rc = scratch_address(&ws);
  if (rc) return rc;
  rc = forward_impl(spec, plan, X, bias, Y, B, s, dtype, ridge_eps, solver, ws, (size_t)DYRA_NOALLOC_MAX_WORKSPACE,
                    stream, StageEvents{nullptr, 0, false});
  if (rc || !status_out) return rc;
  const WsLayout WL = ws_layout(*spec, B, s, dtype);
  if (hipMemcpyAsync(status_out, reinterpret_cast<const char*>(ws) + WL.status, (size_t)B * 4,
                     hipMemcpyDeviceToDevice, reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return DYRA_EHIP;
  return DYRA_OK;
}

extern "C" int dyra_solver_status(const dyra_spec* spec, const void* workspace, int64_t B, int64_t s,
                                  int32_t dtype, int32_t* host_out, void* stream) {
  if (!spec || !workspace || !host_out) return DYRA_EINVAL;
  int rc = validate_spec(spec);
  if (rc) return rc;
  rc = validate_dtype(*spec, dtype);
  if (rc) return rc;
  if (B <= 0 || s <= 0) return DYRA_ESHAPE;
  const WsLayout WL = ws_layout(*spec, B, s, dtype);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(host_out, reinterpret_cast<const char*>(workspace) + WL.status, (size_t)B * 4,
                     hipMemcpyDeviceToHost, st) != hipSuccess)
    return DYRA_EHIP;
  if (hipStreamSynchronize(st) != hipSuccess) return DYRA_EHIP;
  return DYRA_OK;
}

extern "C" int dyra_dense_ref(const void* X, const void* Wt, const void* bias, void* Y, int64_t n, int64_t c1,
                              int64_t c2, int32_t dtype, void* stream) {
  if (!X || !Wt || !Y) return DYRA_EINVAL;
  if (dtype != DYRA_F32 && dtype != DYRA_BF16) return DYRA_EINVAL;
  if (n <= 0 || c1 <= 0 || c2 <= 0 || c1 % 8 || c2 % 8 || n >= ((int64_t)1 << 31)) return DYRA_ESHAPE;
  if ((reinterpret_cast<uintptr_t>(X) | reinterpret_cast<uintptr_t>(Wt) | reinterpret_cast<uintptr_t>(Y) |
       reinterpret_cast<uintptr_t>(bias)) & 15)
    return DYRA_EINVAL;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (dtype == DYRA_BF16) launch_gemm_tn<CfgB>(X, c1, Wt, c1, Y, c2, n, c2, c1, bias, st);
  else launch_gemm_tn<CfgF>(X, c1, Wt, c1, Y, c2, n, c2, c1, bias, st);
  return hipGetLastError() == hipSuccess ? DYRA_OK : DYRA_EHIP;
}
