// Shared host-side helpers: spec validation and the byte layouts of the
// packed device plan and of the forward workspace.
#pragma once

#include <algorithm>
#include <cstddef>
#include <cstdint>

#include "../../include/dyra.h"

namespace dyra_spec_util {

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
inline size_t elem_bytes(int dtype) { return dtype == DYRA_BF16 ? 2 : 4; }

// Validates a spec (and optionally a dtype).  Returns DYRA_OK or an error.
inline int validate_spec(const dyra_spec* sp) {
  if (!sp) return DYRA_EINVAL;
  const dyra_spec& s = *sp;
  if (s.c1 <= 0 || s.c2 <= 0 || s.r <= 0) return DYRA_ESHAPE;
  if (s.c1 % 8 || s.c2 % 8 || s.r % 8) return DYRA_ESHAPE;
  if (s.r > 128) return DYRA_ESHAPE;
  const int64_t mn = s.c1 < s.c2 ? s.c1 : s.c2;
  if (s.r > mn) return DYRA_ESHAPE;
  if (s.c1 > (int64_t)1 << 24 || s.c2 > (int64_t)1 << 24) return DYRA_ESHAPE;
  switch (s.kind) {
    case DYRA_LOWRANK:
      if (s.k <= 0 || s.k % 8 || s.k + s.r > mn) return DYRA_ESHAPE;
      break;
    case DYRA_MONARCH:
      if (s.mblk <= 0 || s.c1 != s.c2 || s.c1 != (int64_t)s.mblk * s.mblk) return DYRA_ESHAPE;
      break;
    case DYRA_BLAST:
    case DYRA_BLAST_DIAG:
      if (s.nb <= 0 || s.rb <= 0 || s.c1 % s.nb || s.c2 % s.nb) return DYRA_ESHAPE;
      if (s.rb > s.c1 / s.nb || s.rb > s.c2 / s.nb) return DYRA_ESHAPE;
      break;
    default:
      return DYRA_EINVAL;
  }
  return DYRA_OK;
}

inline bool is_blast(int kind) { return kind == DYRA_BLAST || kind == DYRA_BLAST_DIAG; }

// Structures / dtypes the device path implements.
inline int validate_dtype(const dyra_spec& s, int dtype) {
  if (dtype != DYRA_F32 && dtype != DYRA_BF16) return DYRA_EINVAL;
  if (s.kind == DYRA_MONARCH) {
    if (dtype != DYRA_BF16 || s.mblk != 32) return DYRA_EDTYPE;
  }
  if (is_blast(s.kind)) {
    if (dtype != DYRA_BF16 || s.rb % 8 || (s.c1 / s.nb) % 8 || (s.c2 / s.nb) % 128) return DYRA_EDTYPE;
    if (s.kind == DYRA_BLAST_DIAG && (int64_t)s.nb * s.rb > 32768) return DYRA_EDTYPE;
  }
  return DYRA_OK;
}

// ---- packed device plan --------------------------------------------------
// low-rank : UPt [(k+r) x c1] ([U | P]^T), Vt [c2 x k] (V^T), Wrt [c2 x c1] (W_res^T)
//            For the 160 x 320 first-stage tile (bf16, k + r = 320, c1 a
//            multiple of 64) UPt is stored k-tile-major instead: 32-column
//            k-tiles, each a contiguous [(k+r) x 32] block.
// Monarch  : B1t and Pt in MFMA fragment order (each 16-byte run one lane's
//            operand of one 32x32x16 step, the 64 lanes of a step one 1 KB
//            run): B1t[((a 2 + s) 64 + l + 32 g) 8 + e] = B1[a][16 s + 8 g + e][l],
//            Pt[(((q 32 + a) 2 + s) 64 + l + 32 g) 8 + e] = P[32 a + 16 s + 8 g + e][32 q + l]
//            (zero for 32 q + l >= r; r rounded up to a multiple of 32 rows);
//            B2t [m][m][m] (B2t[j][l][a] = B2[j][a][l]), Wrt [c x c]
// BLAST    : Ubt [nb][rb][c1/nb] (U_i^T), Pt [r x c1],
//            St [(nb rb) x (nb rb)] (St[j rb + q][i rb + p] = S[i][j][p][q]);
//            BLAST_DIAG: St [nb][nb][rb] (St[j][i][p] = S[i][j][p]),
//            Vb [nb][c2/nb][rb] (as prepared), Wrt [c2 x c1]
// Shape of the first-stage tile kernel: 160 token rows x 320 = k + r output
// columns per workgroup, 32-column k-tiles.
constexpr int S1T_BM = 160, S1T_BN = 320, S1T_BK = 32;
inline bool s1_tile_shape(const dyra_spec& s, int dtype) {
  return s.kind == DYRA_LOWRANK && dtype == DYRA_BF16 && s.k + s.r == S1T_BN && s.c1 % (2 * S1T_BK) == 0 &&
         (int64_t)S1T_BN * s.c1 * 2 < ((int64_t)1 << 31) && (int64_t)S1T_BM * s.c1 * 2 < ((int64_t)1 << 31);
}
// Element index of UPt[q][i] (row q of [U | P]^T, input column i).
inline size_t upt_index(const dyra_spec& s, int dtype, int64_t q, int64_t i) {
  if (s1_tile_shape(s, dtype))
    return (size_t)((i / S1T_BK) * S1T_BN * S1T_BK + q * S1T_BK + i % S1T_BK);
  return (size_t)(q * s.c1 + i);
}

struct PlanLayout {
  size_t UPt = 0, Vt = 0, B1t = 0, B2t = 0, Pt = 0, Ubt = 0, St = 0, Vb = 0, Wrt = 0;
  size_t total = 0;
};

inline PlanLayout plan_layout(const dyra_spec& s, int dtype) {
  PlanLayout L;
  const size_t e = elem_bytes(dtype);
  size_t off = 0;
  auto take = [&](size_t elems) {
    size_t o = off;
    off = align256(off + elems * e);
    return o;
  };
  const size_t c1 = (size_t)s.c1, c2 = (size_t)s.c2, r = (size_t)s.r;
  if (s.kind == DYRA_LOWRANK) {
    L.UPt = take(((size_t)s.k + r) * c1);
    L.Vt = take(c2 * (size_t)s.k);
  } else if (s.kind == DYRA_MONARCH) {
    const size_t m = (size_t)s.mblk;
    L.B1t = take(m * m * m);
    L.Pt = take((r + 31) / 32 * 32 * c1);
    L.B2t = take(m * m * m);
  } else {
    const size_t nb = (size_t)s.nb, rb = (size_t)s.rb;
    L.Ubt = take(nb * rb * (c1 / nb));
    L.Pt = take(r * c1);
    L.St = take(s.kind == DYRA_BLAST_DIAG ? nb * nb * rb : nb * rb * nb * rb);
    L.Vb = take(nb * (c2 / nb) * rb);
  }
  L.Wrt = take(c2 * c1);
  L.total = off;
  return L;
}

// Right-factor GEMM R^T [c2 x nr] (nr = B r, reduction over K = c1) in bf16:
// when even 128 x 128 output tiles would leave most of a 256-CU chip idle,
// K is cut into `slices` runs of `kslice` (a multiple of 64) whose fp32
// partial products are summed afterwards.  slices == 1: a single pass.
struct S5Split {
  int slices = 1;
  int64_t kslice = 0;
};
inline S5Split s5_split(int64_t c2, int64_t nr, int64_t K) {
  S5Split sp;
  sp.kslice = K;
  const int64_t wide = ((c2 + 255) / 256) * ((nr + 127) / 128);
  const int64_t tiles = ((c2 + 127) / 128) * ((nr + 127) / 128);
  if (wide >= 256 || tiles >= 256) return sp;
  // about two workgroups per CU; at least 256 of K per slice; the fp32
  // partials (slices x nr x 4 bytes per output row) at most four times the
  // W_res^T bytes (K x 2 per row).  Measured on MI355X: a 1024 x 2048
  // output with K = 4096 gains with 4 slices (54 -> 42 us); a 1024 x 2048
  // output with K = 1024, whose partials would be 16 times W_res^T, loses.
  int64_t want = std::min<int64_t>((512 + tiles - 1) / tiles, 16);
  want = std::min<int64_t>(want, std::max<int64_t>(1, K / 256));
  want = std::min<int64_t>(want, 2 * K / std::max<int64_t>(nr, 1));
  if (want <= 1) return sp;
  sp.kslice = ((K + want - 1) / want + 63) / 64 * 64;
  sp.slices = (int)((K + sp.kslice - 1) / sp.kslice);
  if (sp.slices <= 1) sp.kslice = K;
  return sp;
}

// ---- forward workspace -----------------------------------------------------
// A    [n x wa]   stage-1 output: low-rank [T | L] (wa = k + r); Monarch
//                 [V | L] (wa = c + r, V the permuted stage-1 output);
//                 BLAST [Z | L] (wa = nb rb + r)
// Wp   [n x nb rb] BLAST coupled output Z S (BLAST only)
// Lt   [r x n256] L transposed (token-contiguous, pitch n rounded up to 256)
// G    [B x r x r] fp32        Gram matrices L_b^T L_b
// M    [B x r x c1] fp32       L_b^T X_b
// Ginv [B x r x r] fp64        (G_b + lambda_b I)^-1 (fp64: near-singular G_b
//                              put 1 / lambda_b-sized entries in it that
//                              cancel in Ginv M; fp32 rounding would not)
// Gi32 [B x r x r] fp32        the same inverse rounded to fp32 (read by the
//                              fp32 apply of well-conditioned segments)
// Mp   [B x r x c1] dtype      M'_b = Ginv_b M_b
// Rt   [c2 x B r] dtype        R_b^T for every segment, R_b = M'_b W_res
// status [B] int32
// Pk   [slices x c2 x B r] fp32  right-factor split-K partials (bf16 only);
//      BLAST also [slices x n x r] for L = X P split over K
struct WsLayout {
  int64_t wa = 0;
  size_t A = 0, Wp = 0, Lt = 0, G = 0, M = 0, Ginv = 0, Mp = 0, Rt = 0, status = 0, Pk = 0;
  // per-segment precision of M' = Ginv M (0 fp32, 1 fp64), set by the solve
  size_t prec = 0, kprec = 0, Gi32 = 0, Ki32 = 0;
  // token-split partials of M [msplit][B x r x c1] fp32 (msplit > 1 only)
  size_t Mpart = 0;
  int msplit = 1;
  // Gram partials [B][gchunks][r x r] fp32 over token chunks of gchunk tokens
  size_t Gp = 0;
  int64_t gchunk = 0, gchunks = 0;
  // left ALS steps (half_steps > 2): R [B r x c2], K [B x r x r] fp32 and
  // Kinv fp64, Q^T [B x r x c1] fp32, Z^T [B x r x c1], their status words [B]
  size_t R = 0, K = 0, Kinv = 0, Qt = 0, Zt = 0, kstatus = 0;
  size_t total = 0;
};

// Token split of the M_b = L_b^T X_b strips: with few (segment, 128-column
// strip) pairs the reduction runs on too few workgroups to stream X at the
// chip's rate, so each strip's tokens are cut into parts whose fp32 partials
// a second launch adds in a fixed order.  At least 512 tokens per part.
inline int s3_token_split(int64_t B, int64_t c1, int64_t max_len) {
  const int64_t pairs = B * ((c1 + 127) / 128);
  if (pairs >= 128) return 1;
  int64_t ts = (256 + pairs - 1) / pairs;
  if (ts > 8) ts = 8;
  if (ts > max_len / 512) ts = max_len / 512;
  return ts < 1 ? 1 : (int)ts;
}

// B segments of n rows in all, the longest max_len rows.
inline WsLayout ws_layout_n(const dyra_spec& s, int64_t B, int64_t n_rows, int64_t max_len, int dtype,
                            int half_steps = 2) {
  WsLayout W;
  const size_t e = elem_bytes(dtype);
  const int64_t seg = max_len;
  const size_t n = (size_t)n_rows, r = (size_t)s.r, c1 = (size_t)s.c1, c2 = (size_t)s.c2;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  int64_t stat = 0;
  if (s.kind == DYRA_LOWRANK) stat = s.k;
  else if (s.kind == DYRA_MONARCH) stat = s.c2;
  else stat = (int64_t)s.nb * s.rb;
  W.wa = stat + s.r;
  W.A = take(n * (size_t)W.wa * e);
  if (is_blast(s.kind)) W.Wp = take(n * (size_t)stat * e);
  W.Lt = take(r * ((n + 255) / 256 * 256) * e);   // token pitch padded to 256
  W.G = take((size_t)B * r * r * 4);
  W.M = take((size_t)B * r * c1 * 4);
  W.Ginv = take((size_t)B * r * r * 8);
  W.Gi32 = take((size_t)B * r * r * 4);
  W.Mp = take((size_t)B * r * c1 * e);
  W.Rt = take(c2 * (size_t)B * r * e);
  W.status = take((size_t)B * 4);
  W.prec = take((size_t)B * 4);
  W.msplit = s3_token_split(B, s.c1, seg);
  if (W.msplit > 1) W.Mpart = take((size_t)W.msplit * B * r * c1 * 4);
  W.gchunk = s.r > 64 ? 256 : 128;
  W.gchunks = (seg + W.gchunk - 1) / W.gchunk;
  // token-chunk partials, or two per 160-token first-stage tile
  W.Gp = take(std::max((size_t)B * (size_t)W.gchunks, ((n + 159) / 160) * 2) * r * r * 4);
  if (dtype == DYRA_BF16) {
    // shared by the right factor and (BLAST) L = X P, which never overlap
    const S5Split sp = s5_split((int64_t)c2, B * (int64_t)r, (int64_t)c1);
    size_t pk = sp.slices > 1 ? (size_t)sp.slices * c2 * (size_t)B * r * 4 : 0;
    if (is_blast(s.kind)) {
      const S5Split sl = s5_split((int64_t)n, (int64_t)r, (int64_t)c1);
      if (sl.slices > 1) pk = std::max(pk, (size_t)sl.slices * n * r * 4);
    }
    if (pk) W.Pk = take(pk);
  }
  if (half_steps > 2) {
    W.R = take((size_t)B * r * c2 * e);
    W.K = take((size_t)B * r * r * 4);
    W.Kinv = take((size_t)B * r * r * 8);
    W.Ki32 = take((size_t)B * r * r * 4);
    W.Qt = take((size_t)B * r * c1 * 4);
    W.Zt = take((size_t)B * r * c1 * e);
    W.kstatus = take((size_t)B * 4);
    W.kprec = take((size_t)B * 4);
  }
  W.total = off;
  return W;
}

// B segments of seg rows each.
inline WsLayout ws_layout(const dyra_spec& s, int64_t B, int64_t seg, int dtype, int half_steps = 2) {
  return ws_layout_n(s, B, B * seg, seg, dtype, half_steps);
}

}  // namespace dyra_spec_util
