// Offline DyRA preparation on the host (float64) and packing of the device
// plan.  Follows the offline stage of the method: fit the structured
// approximation W_hat, form the dense residual W_res = W - W_hat, fix the
// initial right factor R0 (top-r right singular vectors of W_res) and
// precompute the thin projection P = W_res R0^T.
// Sources: nanless.github.io DyRA digest ("overall DyRA flow", "offline
// preparation and online computation", structured-matrix section);
// paperlayer.ai App. A and App. B.
#include <cmath>
#include <cstring>
#include <vector>

#include "host_linalg.h"
#include "spec.h"

using dyra_host::Mat;
using dyra_host::Pool;
using namespace dyra_spec_util;

extern "C" const char* dyra_status_string(int code) {
  switch (code) {
    case DYRA_OK: return "ok";
    case DYRA_EINVAL: return "invalid argument";
    case DYRA_ESHAPE: return "invalid shape";
    case DYRA_EWORKSPACE: return "workspace too small";
    case DYRA_EHIP: return "HIP error";
    case DYRA_ENOCONV: return "eigensolver did not converge";
    case DYRA_EDTYPE: return "dtype not supported for this structure";
    default: return "unknown status";
  }
}

extern "C" int dyra_prepare_sizes(const dyra_spec* spec, dyra_sizes* out) {
  if (!spec || !out) return DYRA_EINVAL;
  int rc = validate_spec(spec);
  if (rc) return rc;
  const dyra_spec& s = *spec;
  std::memset(out, 0, sizeof(*out));
  if (s.kind == DYRA_LOWRANK) {
    out->U = s.c1 * s.k;
    out->V = (int64_t)s.k * s.c2;
  } else if (s.kind == DYRA_MONARCH) {
    out->B1 = (int64_t)s.mblk * s.mblk * s.mblk;
    out->B2 = out->B1;
  } else {
    out->Ub = s.c1 * s.rb;                       // nb * (c1/nb) * rb
    out->S = (int64_t)s.nb * s.nb * s.rb * (s.kind == DYRA_BLAST_DIAG ? 1 : s.rb);
    out->Vb = s.c2 * s.rb;
  }
  out->P = s.c1 * s.r;
  out->R0 = (int64_t)s.r * s.c2;
  out->Wres = s.c1 * s.c2;
  out->res_sv = s.r;
  return DYRA_OK;
}

namespace {

// Low-rank: truncated SVD, sqrt(sigma) on each side.
bool fit_lowrank(Pool& pool, const Mat& W, int k, Mat& Uf, Mat& Vf, Mat& What) {
  Mat U, V;
  std::vector<double> s;
  if (!dyra_host::svd_top(pool, W, k, U, s, V)) return false;
  Uf = Mat(W.rows, k);
  Vf = Mat(k, W.cols);
  for (int q = 0; q < k; ++q) {
    const double rs = std::sqrt(s[(size_t)q]);
    for (int64_t i = 0; i < W.rows; ++i) Uf(i, q) = U(i, q) * rs;
    for (int64_t j = 0; j < W.cols; ++j) Vf(q, j) = rs * V(j, q);
  }
  What = dyra_host::matmul(pool, Uf, Vf);
  return true;
}

// Monarch: rank-1 truncated SVD of every m x m block (a, j):
// block = sigma u v^T -> B1[a][:, j] = sqrt(sigma) u, B2[j][a, :] = sqrt(sigma) v.
bool fit_monarch(Pool& pool, const Mat& W, int m, std::vector<double>& B1, std::vector<double>& B2,
                 Mat& What) {
  const int64_t M = m;
  B1.assign((size_t)(M * M * M), 0.0);
  B2.assign((size_t)(M * M * M), 0.0);
  What = Mat(W.rows, W.cols);
  bool ok = true;
  pool.parallel_for(M * M, [&](int64_t b0, int64_t b1) {
    Pool serial(1);
    for (int64_t b = b0; b < b1; ++b) {
      const int64_t a = b / M, j = b % M;
      Mat blk(M, M);
      for (int64_t i = 0; i < M; ++i)
        for (int64_t l = 0; l < M; ++l) blk(i, l) = W(a * M + i, j * M + l);
      Mat U, V;
      std::vector<double> s;
      if (!dyra_host::svd_top(serial, blk, 1, U, s, V)) {
        ok = false;
        continue;
      }
      const double rs = std::sqrt(s[0]);
      for (int64_t i = 0; i < M; ++i) B1[(size_t)((a * M + i) * M + j)] = rs * U(i, 0);
      for (int64_t l = 0; l < M; ++l) B2[(size_t)((j * M + a) * M + l)] = rs * V(l, 0);
      for (int64_t i = 0; i < M; ++i)
        for (int64_t l = 0; l < M; ++l)
          What(a * M + i, j * M + l) = B1[(size_t)((a * M + i) * M + j)] * B2[(size_t)((j * M + a) * M + l)];
    }
  });
  return ok;
}

// BLAST: U_i = top-rb left singular vectors of block row i, V_j = top-rb
// right singular vectors of block column j, S_ij = U_i^T W_ij V_j; with
// diagonal couplings only diag(U_i^T W_ij V_j) (S holds [nb][nb][rb]).
bool fit_blast(Pool& pool, const Mat& W, int nb, int rb, bool diag, std::vector<double>& Ub,
               std::vector<double>& S, std::vector<double>& Vb, Mat& What) {
  const int64_t b1 = W.rows / nb, b2 = W.cols / nb;
  std::vector<Mat> U((size_t)nb), V((size_t)nb);
  for (int i = 0; i < nb; ++i) {
    Mat Wi(b1, W.cols);
    std::memcpy(Wi.a.data(), W.row(i * b1), sizeof(double) * (size_t)(b1 * W.cols));
    Mat Vd;
    std::vector<double> s;
    if (!dyra_host::svd_top(pool, Wi, rb, U[(size_t)i], s, Vd, true, false)) return false;
  }
  for (int j = 0; j < nb; ++j) {
    Mat Wj(W.rows, b2);
    for (int64_t i = 0; i < W.rows; ++i)
      std::memcpy(Wj.row(i), W.row(i) + j * b2, sizeof(double) * (size_t)b2);
    Mat Ud;
    std::vector<double> s;
    if (!dyra_host::svd_top(pool, Wj, rb, Ud, s, V[(size_t)j], false, true)) return false;
  }
  Ub.assign((size_t)(nb * b1 * rb), 0.0);
  Vb.assign((size_t)(nb * b2 * rb), 0.0);
  S.assign((size_t)nb * nb * rb * (diag ? 1 : rb), 0.0);
  for (int i = 0; i < nb; ++i)
    std::memcpy(Ub.data() + (size_t)i * b1 * rb, U[(size_t)i].a.data(), sizeof(double) * (size_t)(b1 * rb));
  for (int j = 0; j < nb; ++j)
    std::memcpy(Vb.data() + (size_t)j * b2 * rb, V[(size_t)j].a.data(), sizeof(double) * (size_t)(b2 * rb));
  What = Mat(W.rows, W.cols);
  Pool serial(1);
  pool.parallel_for((int64_t)nb * nb, [&](int64_t t0, int64_t t1) {
    Pool one(1);
    for (int64_t t = t0; t < t1; ++t) {
      const int64_t i = t / nb, j = t % nb;
      Mat Wij(b1, b2);
      for (int64_t a = 0; a < b1; ++a)
        std::memcpy(Wij.row(a), W.row(i * b1 + a) + j * b2, sizeof(double) * (size_t)b2);
      Mat T = dyra_host::matmul_tn(one, U[(size_t)i], Wij);      // rb x b2
      Mat Sij = dyra_host::matmul(one, T, V[(size_t)j]);          // rb x rb
      if (diag) {
        for (int p = 0; p < rb; ++p) {
          S[(size_t)t * rb + p] = Sij(p, p);
          for (int q = 0; q < rb; ++q)
            if (q != p) Sij(p, q) = 0.0;
        }
      } else {
        std::memcpy(S.data() + (size_t)t * rb * rb, Sij.a.data(), sizeof(double) * (size_t)(rb * rb));
      }
      Mat US = dyra_host::matmul(one, U[(size_t)i], Sij);        // b1 x rb
      Mat Wh = dyra_host::matmul_nt(one, US, V[(size_t)j]);      // b1 x b2
      for (int64_t a = 0; a < b1; ++a)
        std::memcpy(What.row(i * b1 + a) + j * b2, Wh.row(a), sizeof(double) * (size_t)b2);
    }
  });
  (void)serial;
  return true;
}

inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

inline void put(void* base, size_t byte_off, size_t idx, double v, int dtype) {
  const float f = (float)v;
  if (dtype == DYRA_BF16) {
    reinterpret_cast<uint16_t*>(static_cast<char*>(base) + byte_off)[idx] = f32_to_bf16_rne(f);
  } else {
    reinterpret_cast<float*>(static_cast<char*>(base) + byte_off)[idx] = f;
  }
}

// W_res = W - W_hat; R0 = top-r right singular vectors of W_res and
// P = W_res R0^T, written to out (with res_sv).
int finish_residual(Pool& pool, const dyra_spec& s, const Mat& Wm, const Mat& What, dyra_host_factors* out) {
  Mat Wres(s.c1, s.c2);
  for (size_t i = 0; i < Wres.a.size(); ++i) Wres.a[i] = Wm.a[i] - What.a[i];
  Mat Ud, V;
  std::vector<double> rho;
  if (!dyra_host::svd_top(pool, Wres, s.r, Ud, rho, V, false, true)) return DYRA_ENOCONV;
  Mat P = dyra_host::matmul(pool, Wres, V);     // c1 x r
  for (int q = 0; q < s.r; ++q) {
    for (int64_t j = 0; j < s.c2; ++j) out->R0[(size_t)q * s.c2 + j] = V(j, q);
    out->res_sv[q] = rho[(size_t)q];
  }
  std::memcpy(out->P, P.a.data(), sizeof(double) * P.a.size());
  std::memcpy(out->Wres, Wres.a.data(), sizeof(double) * Wres.a.size());
  return DYRA_OK;
}

// Lower Cholesky factor of a symmetric positive definite K (n x n), column
// by column; the rows below each pivot run in parallel.  False if a pivot is
// not positive.
bool cholesky_lower(Pool& pool, const Mat& K, Mat& C) {
  const int64_t n = K.rows;
  C = K;
  for (int64_t j = 0; j < n; ++j) {
    const double* cj = C.row(j);
    double d = C(j, j);
    for (int64_t q = 0; q < j; ++q) d -= cj[q] * cj[q];
    if (!(d > 0.0) || !std::isfinite(d)) return false;
    const double piv = std::sqrt(d);
    C(j, j) = piv;
    pool.parallel_for(n - j - 1, [&](int64_t a, int64_t b) {
      for (int64_t i = j + 1 + a; i < j + 1 + b; ++i) {
        double* ci = C.row(i);
        double v = ci[j];
        for (int64_t q = 0; q < j; ++q) v -= ci[q] * cj[q];
        ci[j] = v / piv;
      }
    });
  }
  for (int64_t i = 0; i < n; ++i)
    for (int64_t j = i + 1; j < n; ++j) C(i, j) = 0.0;
  return true;
}

}  // namespace

extern "C" int dyra_prepare_input_aware(const dyra_spec* spec, const double* W, const double* X_cal,
                                        int64_t n_cal, int32_t mode, dyra_host_factors* out, int32_t nthreads) {
  if (!spec || !W || !X_cal || !out) return DYRA_EINVAL;
  int rc = validate_spec(spec);
  if (rc) return rc;
  const dyra_spec& s = *spec;
  if (s.kind != DYRA_LOWRANK) return DYRA_EINVAL;
  if (mode != DYRA_INPUT_AWARE_DIAG && mode != DYRA_INPUT_AWARE_CHOL) return DYRA_EINVAL;
  if (n_cal <= 0) return DYRA_ESHAPE;
  if (!out->U || !out->V || !out->P || !out->R0 || !out->Wres || !out->res_sv) return DYRA_EINVAL;
  try {
    Pool pool(nthreads);
    const int64_t c1 = s.c1, c2 = s.c2;
    Mat Wm(c1, c2);
    std::memcpy(Wm.a.data(), W, sizeof(double) * (size_t)(c1 * c2));
    Mat Xc(n_cal, c1);
    std::memcpy(Xc.a.data(), X_cal, sizeof(double) * (size_t)(n_cal * c1));
    for (double v : Xc.a)
      if (!std::isfinite(v)) return DYRA_EINVAL;
    // S W, and later U_f = S^-1 (U_k sqrt(sigma))
    Mat SW(c1, c2), Ct;
    std::vector<double> sdiag;
    if (mode == DYRA_INPUT_AWARE_DIAG) {
      sdiag.assign((size_t)c1, 0.0);
      for (int64_t t = 0; t < n_cal; ++t)
        for (int64_t i = 0; i < c1; ++i) sdiag[(size_t)i] += Xc(t, i) * Xc(t, i);
      double mx = 0.0;
      for (auto& v : sdiag) {
        v = std::sqrt(v / (double)n_cal);
        mx = std::max(mx, v);
      }
      if (!(mx > 0.0)) return DYRA_EINVAL;
      for (auto& v : sdiag) v = std::max(v, 1e-6 * mx);
      for (int64_t i = 0; i < c1; ++i)
        for (int64_t j = 0; j < c2; ++j) SW(i, j) = sdiag[(size_t)i] * Wm(i, j);
    } else {
      Mat K = dyra_host::gram_cols(pool, Xc);    // X^T X
      double tr = 0.0;
      for (int64_t i = 0; i < c1; ++i) tr += K(i, i);
      if (!(tr > 0.0)) return DYRA_EINVAL;
      for (auto& v : K.a) v /= (double)n_cal;
      for (int64_t i = 0; i < c1; ++i) K(i, i) += 1e-6 * tr / (double)n_cal / (double)c1;
      Mat C;
      if (!cholesky_lower(pool, K, C)) return DYRA_ENOCONV;
      SW = dyra_host::matmul_tn(pool, C, Wm);     // C^T W
      Ct = dyra_host::transpose(pool, C);          // S = C^T, upper triangular
    }
    Mat U, V;
    std::vector<double> sv;
    if (!dyra_host::svd_top(pool, SW, s.k, U, sv, V)) return DYRA_ENOCONV;
    const int k = s.k;
    Mat Uf(c1, k), Vf(k, c2);
    for (int q = 0; q < k; ++q) {
      const double rs = std::sqrt(sv[(size_t)q]);
      for (int64_t i = 0; i < c1; ++i) Uf(i, q) = U(i, q) * rs;
      for (int64_t j = 0; j < c2; ++j) Vf(q, j) = rs * V(j, q);
    }
    if (mode == DYRA_INPUT_AWARE_DIAG) {
      for (int64_t i = 0; i < c1; ++i)
        for (int q = 0; q < k; ++q) Uf(i, q) /= sdiag[(size_t)i];
    } else {
      // back substitution C^T x = b for each of the k columns
      pool.parallel_for(k, [&](int64_t q0, int64_t q1) {
        for (int64_t q = q0; q < q1; ++q)
          for (int64_t i = c1 - 1; i >= 0; --i) {
            const double* ct = Ct.row(i);
            double v = Uf(i, q);
            for (int64_t j = i + 1; j < c1; ++j) v -= ct[j] * Uf(j, q);
            Uf(i, q) = v / ct[i];
          }
      });
    }
    Mat What = dyra_host::matmul(pool, Uf, Vf);
    std::memcpy(out->U, Uf.a.data(), sizeof(double) * Uf.a.size());
    std::memcpy(out->V, Vf.a.data(), sizeof(double) * Vf.a.size());
    rc = finish_residual(pool, s, Wm, What, out);
    if (rc) return rc;
  } catch (...) {
    return DYRA_EINVAL;
  }
  return DYRA_OK;
}

extern "C" int dyra_prepare(const dyra_spec* spec, const double* W, dyra_host_factors* out,
                            int32_t nthreads) {
  if (!spec || !W || !out) return DYRA_EINVAL;
  int rc = validate_spec(spec);
  if (rc) return rc;
  const dyra_spec& s = *spec;
  if (!out->P || !out->R0 || !out->Wres || !out->res_sv) return DYRA_EINVAL;
  if (s.kind == DYRA_LOWRANK && (!out->U || !out->V)) return DYRA_EINVAL;
  if (s.kind == DYRA_MONARCH && (!out->B1 || !out->B2)) return DYRA_EINVAL;
  if (is_blast(s.kind) && (!out->Ub || !out->S || !out->Vb)) return DYRA_EINVAL;
  try {
    Pool pool(nthreads);
    Mat Wm(s.c1, s.c2);
    std::memcpy(Wm.a.data(), W, sizeof(double) * (size_t)(s.c1 * s.c2));
    Mat What;
    if (s.kind == DYRA_LOWRANK) {
      Mat Uf, Vf;
      if (!fit_lowrank(pool, Wm, s.k, Uf, Vf, What)) return DYRA_ENOCONV;
      std::memcpy(out->U, Uf.a.data(), sizeof(double) * Uf.a.size());
      std::memcpy(out->V, Vf.a.data(), sizeof(double) * Vf.a.size());
    } else if (s.kind == DYRA_MONARCH) {
      std::vector<double> B1, B2;
      if (!fit_monarch(pool, Wm, s.mblk, B1, B2, What)) return DYRA_ENOCONV;
      std::memcpy(out->B1, B1.data(), sizeof(double) * B1.size());
      std::memcpy(out->B2, B2.data(), sizeof(double) * B2.size());
    } else {
      std::vector<double> Ub, S, Vb;
      if (!fit_blast(pool, Wm, s.nb, s.rb, s.kind == DYRA_BLAST_DIAG, Ub, S, Vb, What)) return DYRA_ENOCONV;
      std::memcpy(out->Ub, Ub.data(), sizeof(double) * Ub.size());
      std::memcpy(out->S, S.data(), sizeof(double) * S.size());
      std::memcpy(out->Vb, Vb.data(), sizeof(double) * Vb.size());
    }
    rc = finish_residual(pool, s, Wm, What, out);
    if (rc) return rc;
  } catch (...) {
    return DYRA_EINVAL;
  }
  return DYRA_OK;
}

extern "C" int dyra_plan_size(const dyra_spec* spec, int32_t dtype, size_t* bytes) {
  if (!spec || !bytes) return DYRA_EINVAL;
  int rc = validate_spec(spec);
  if (rc) return rc;
  rc = validate_dtype(*spec, dtype);
  if (rc) return rc;
  *bytes = plan_layout(*spec, dtype).total;
  return DYRA_OK;
}

extern "C" int dyra_plan_pack(const dyra_spec* spec, const dyra_host_factors* f, int32_t dtype,
                              void* host_plan) {
  if (!spec || !f || !host_plan) return DYRA_EINVAL;
  int rc = validate_spec(spec);
  if (rc) return rc;
  rc = validate_dtype(*spec, dtype);
  if (rc) return rc;
  const dyra_spec& s = *spec;
  if (!f->P || !f->Wres) return DYRA_EINVAL;
  const PlanLayout L = plan_layout(s, dtype);
  std::memset(host_plan, 0, L.total);
  const int64_t c1 = s.c1, c2 = s.c2, r = s.r;
  if (s.kind == DYRA_LOWRANK) {
    if (!f->U || !f->V) return DYRA_EINVAL;
    const int64_t k = s.k;
    for (int64_t q = 0; q < k; ++q)
      for (int64_t i = 0; i < c1; ++i) put(host_plan, L.UPt, upt_index(s, dtype, q, i), f->U[i * k + q], dtype);
    for (int64_t p = 0; p < r; ++p)
      for (int64_t i = 0; i < c1; ++i) put(host_plan, L.UPt, upt_index(s, dtype, k + p, i), f->P[i * r + p], dtype);
    for (int64_t j = 0; j < c2; ++j)
      for (int64_t q = 0; q < k; ++q) put(host_plan, L.Vt, (size_t)(j * k + q), f->V[q * c2 + j], dtype);
  } else if (s.kind == DYRA_MONARCH) {
    if (!f->B1 || !f->B2) return DYRA_EINVAL;
    const int64_t m = s.mblk;
    // fragment order (m = 32): element k = 16 s + 8 g + e of the reduction,
    // output column l, lane l + 32 g of 32x32x16 step s
    auto frag = [](int64_t blk, int64_t k, int64_t l) {
      return (size_t)(((blk * 2 + k / 16) * 64 + l + 32 * ((k / 8) % 2)) * 8 + k % 8);
    };
    for (int64_t a = 0; a < m; ++a)
      for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < m; ++j) {
          put(host_plan, L.B1t, frag(a, i, j), f->B1[(a * m + i) * m + j], dtype);
          // B2 block a plays the role of j here: B2t[a][l=j][row=i] = B2[a][i][j]
          put(host_plan, L.B2t, (size_t)((a * m + j) * m + i), f->B2[(a * m + i) * m + j], dtype);
        }
    for (int64_t p = 0; p < r; ++p)
      for (int64_t i = 0; i < c1; ++i)
        put(host_plan, L.Pt, frag((p / 32) * m + i / m, i % m, p % 32), f->P[i * r + p], dtype);
  } else {
    if (!f->Ub || !f->S || !f->Vb) return DYRA_EINVAL;
    const int64_t nb = s.nb, rb = s.rb, b1 = c1 / nb, b2 = c2 / nb;
    for (int64_t i = 0; i < nb; ++i)
      for (int64_t q = 0; q < b1; ++q)
        for (int64_t p = 0; p < rb; ++p)
          put(host_plan, L.Ubt, (size_t)((i * rb + p) * b1 + q), f->Ub[(i * b1 + q) * rb + p], dtype);
    for (int64_t p = 0; p < r; ++p)
      for (int64_t i = 0; i < c1; ++i) put(host_plan, L.Pt, (size_t)(p * c1 + i), f->P[i * r + p], dtype);
    const int64_t NR = nb * rb;
    if (s.kind == DYRA_BLAST_DIAG) {
      for (int64_t i = 0; i < nb; ++i)
        for (int64_t j = 0; j < nb; ++j)
          for (int64_t p = 0; p < rb; ++p)
            put(host_plan, L.St, (size_t)((j * nb + i) * rb + p), f->S[(i * nb + j) * rb + p], dtype);
    } else {
      for (int64_t i = 0; i < nb; ++i)
        for (int64_t j = 0; j < nb; ++j)
          for (int64_t p = 0; p < rb; ++p)
            for (int64_t q = 0; q < rb; ++q)
              put(host_plan, L.St, (size_t)((j * rb + q) * NR + i * rb + p),
                  f->S[((i * nb + j) * rb + p) * rb + q], dtype);
    }
    for (int64_t t = 0; t < nb * b2 * rb; ++t) put(host_plan, L.Vb, (size_t)t, f->Vb[t], dtype);
  }
  for (int64_t i = 0; i < c1; ++i)
    for (int64_t j = 0; j < c2; ++j) put(host_plan, L.Wrt, (size_t)(j * c1 + i), f->Wres[i * c2 + j], dtype);
  return DYRA_OK;
}

extern "C" int dyra_workspace_offsets(const dyra_spec* spec, int64_t B, int64_t s, int32_t dtype,
                                      dyra_ws_offsets* out) {
  if (!spec || !out) return DYRA_EINVAL;
  int rc = validate_spec(spec);
  if (rc) return rc;
  rc = validate_dtype(*spec, dtype);
  if (rc) return rc;
  if (B <= 0 || s <= 0 || B * s >= ((int64_t)1 << 31)) return DYRA_ESHAPE;
  const WsLayout W = ws_layout(*spec, B, s, dtype);
  out->A = (int64_t)W.A;
  out->Wp = (int64_t)W.Wp;
  out->Lt = (int64_t)W.Lt;
  out->G = (int64_t)W.G;
  out->M = (int64_t)W.M;
  out->Ginv = (int64_t)W.Ginv;
  out->Mp = (int64_t)W.Mp;
  out->Rt = (int64_t)W.Rt;
  out->status = (int64_t)W.status;
  out->total = (int64_t)W.total;
  out->wa = W.wa;
  out->lt_pitch = (B * s + 255) / 256 * 256;
  out->prec = (int64_t)W.prec;
  return DYRA_OK;
}
