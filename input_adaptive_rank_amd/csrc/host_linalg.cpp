// Host float64 linear algebra for the offline DyRA preparation.
//
// Symmetric top-k eigenpairs: Householder reduction to tridiagonal form
// (Golub & Van Loan, "Matrix Computations", sec. 8.3.1), eigenvalues by
// Sturm-sequence bisection (sec. 8.4.1), eigenvectors by inverse iteration on
// the tridiagonal matrix with Gaussian elimination and partial pivoting
// (sec. 8.2.2 / 7.6.1), re-orthogonalised inside clusters, then mapped back
// through the Householder reflectors.  Written for this library; no LAPACK.
#include "host_linalg.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <condition_variable>
#include <cstring>
#include <limits>
#include <mutex>
#include <thread>

namespace dyra_host {

// ---------------------------------------------------------------------------
// worker pool
// ---------------------------------------------------------------------------

struct Pool::Impl {
  std::vector<std::thread> th;
  std::mutex mu;
  std::condition_variable cv_job, cv_done;
  const std::function<void(int64_t, int64_t)>* fn = nullptr;
  int64_t n = 0, chunk = 1;
  std::atomic<int64_t> next{0};
  int busy = 0;
  uint64_t gen = 0;
  bool stop = false;

  void run_chunks() {
    for (;;) {
      int64_t b = next.fetch_add(chunk);
      if (b >= n) break;
      (*fn)(b, std::min(n, b + chunk));
    }
  }
};

Pool::Pool(int nthreads) : impl_(new Impl), nthreads_(nthreads) {
  if (nthreads_ < 1) {
    unsigned hc = std::thread::hardware_concurrency();
    nthreads_ = hc ? (int)hc : 1;
  }
  for (int t = 1; t < nthreads_; ++t) {
    impl_->th.emplace_back([this] {
      Impl* p = impl_;
      uint64_t seen = 0;
      for (;;) {
        {
          std::unique_lock<std::mutex> lk(p->mu);
          p->cv_job.wait(lk, [&] { return p->stop || p->gen != seen; });
          if (p->stop) return;
          seen = p->gen;
        }
        p->run_chunks();
        {
          std::lock_guard<std::mutex> lk(p->mu);
          if (--p->busy == 0) p->cv_done.notify_all();
        }
      }
    });
  }
}

Pool::~Pool() {
  {
    std::lock_guard<std::mutex> lk(impl_->mu);
    impl_->stop = true;
  }
  impl_->cv_job.notify_all();
  for (auto& t : impl_->th) t.join();
  delete impl_;
}

void Pool::parallel_for(int64_t n, const std::function<void(int64_t, int64_t)>& fn) {
  if (n <= 0) return;
  if (nthreads_ == 1 || n == 1) {
    fn(0, n);
    return;
  }
  Impl* p = impl_;
  {
    std::lock_guard<std::mutex> lk(p->mu);
    p->fn = &fn;
    p->n = n;
    p->chunk = std::max<int64_t>(1, n / (4 * (int64_t)nthreads_));
    p->next.store(0);
    p->busy = nthreads_ - 1;
    ++p->gen;
  }
  p->cv_job.notify_all();
  p->run_chunks();
  std::unique_lock<std::mutex> lk(p->mu);
  p->cv_done.wait(lk, [&] { return p->busy == 0; });
  p->fn = nullptr;
}

// ---------------------------------------------------------------------------
// dense kernels
// ---------------------------------------------------------------------------

typedef double v4d __attribute__((vector_size(32)));

static inline v4d load4(const double* p) {
  v4d v;
  std::memcpy(&v, p, sizeof(v));
  return v;
}
static inline double hsum(v4d v) { return (v[0] + v[1]) + (v[2] + v[3]); }

// acc[ii][jj] += dot(A[ii][k0:k1], B[jj][k0:k1]) for a 4 x 4 block of rows.
static void dot4x4(const double* const* ar, const double* const* br, int na, int nbr, int64_t k0,
                   int64_t k1, double acc[4][4]) {
  v4d s[4][4];
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j) s[i][j] = v4d{0, 0, 0, 0};
  int64_t k = k0;
  if (na == 4 && nbr == 4) {
    for (; k + 4 <= k1; k += 4) {
      v4d a0 = load4(ar[0] + k), a1 = load4(ar[1] + k), a2 = load4(ar[2] + k), a3 = load4(ar[3] + k);
      v4d b0 = load4(br[0] + k), b1 = load4(br[1] + k), b2 = load4(br[2] + k), b3 = load4(br[3] + k);
      s[0][0] += a0 * b0; s[0][1] += a0 * b1; s[0][2] += a0 * b2; s[0][3] += a0 * b3;
      s[1][0] += a1 * b0; s[1][1] += a1 * b1; s[1][2] += a1 * b2; s[1][3] += a1 * b3;
      s[2][0] += a2 * b0; s[2][1] += a2 * b1; s[2][2] += a2 * b2; s[2][3] += a2 * b3;
      s[3][0] += a3 * b0; s[3][1] += a3 * b1; s[3][2] += a3 * b2; s[3][3] += a3 * b3;
    }
  }
  for (int i = 0; i < na; ++i)
    for (int j = 0; j < nbr; ++j) {
      double t = hsum(s[i][j]);
      for (int64_t kk = k; kk < k1; ++kk) t += ar[i][kk] * br[j][kk];
      acc[i][j] += t;
    }
}

// C[i][j] = dot(A_i, B_j) over rows of A (m x K) and B (n x K); if sym, A == B
// and only j >= i tiles are computed then mirrored.
static Mat rowdots(Pool& pool, const Mat& A, const Mat& B, bool sym) {
  const int64_t m = A.rows, n = B.rows, K = A.cols;
  Mat C(m, n);
  const int64_t T = 64, KC = 256;
  const int64_t mt = (m + T - 1) / T, nt = (n + T - 1) / T;
  std::vector<std::pair<int64_t, int64_t>> tiles;
  for (int64_t it = 0; it < mt; ++it)
    for (int64_t jt = sym ? it : 0; jt < nt; ++jt) tiles.emplace_back(it, jt);
  pool.parallel_for((int64_t)tiles.size(), [&](int64_t t0, int64_t t1) {
    std::vector<double> ct((size_t)(T * T));
    for (int64_t t = t0; t < t1; ++t) {
      const int64_t i0 = tiles[t].first * T, j0 = tiles[t].second * T;
      const int64_t i1 = std::min(m, i0 + T), j1 = std::min(n, j0 + T);
      std::fill(ct.begin(), ct.end(), 0.0);
      for (int64_t k0 = 0; k0 < K; k0 += KC) {
        const int64_t k1 = std::min(K, k0 + KC);
        for (int64_t i = i0; i < i1; i += 4) {
          const double* ar[4];
          int na = (int)std::min<int64_t>(4, i1 - i);
          for (int q = 0; q < 4; ++q) ar[q] = A.row(std::min(i + q, m - 1));
          for (int64_t j = j0; j < j1; j += 4) {
            const double* br[4];
            int nbr = (int)std::min<int64_t>(4, j1 - j);
            for (int q = 0; q < 4; ++q) br[q] = B.row(std::min(j + q, n - 1));
            double acc[4][4] = {};
            dot4x4(ar, br, na, nbr, k0, k1, acc);
            for (int a = 0; a < na; ++a)
              for (int b = 0; b < nbr; ++b) ct[(size_t)((i - i0 + a) * T + (j - j0 + b))] += acc[a][b];
          }
        }
      }
      for (int64_t i = i0; i < i1; ++i)
        for (int64_t j = j0; j < j1; ++j) {
          double v = ct[(size_t)((i - i0) * T + (j - j0))];
          C(i, j) = v;
          if (sym) C(j, i) = v;
        }
    }
  });
  return C;
}

Mat gram_rows(Pool& pool, const Mat& A) { return rowdots(pool, A, A, true); }

Mat transpose(Pool& pool, const Mat& A) {
  Mat T(A.cols, A.rows);
  const int64_t B = 64;
  const int64_t nb = (A.cols + B - 1) / B;
  pool.parallel_for(nb, [&](int64_t b0, int64_t b1) {
    for (int64_t bj = b0; bj < b1; ++bj) {
      const int64_t j0 = bj * B, j1 = std::min(A.cols, j0 + B);
      for (int64_t i0 = 0; i0 < A.rows; i0 += B) {
        const int64_t i1 = std::min(A.rows, i0 + B);
        for (int64_t j = j0; j < j1; ++j)
          for (int64_t i = i0; i < i1; ++i) T(j, i) = A(i, j);
      }
    }
  });
  return T;
}

Mat gram_cols(Pool& pool, const Mat& A) {
  Mat T = transpose(pool, A);
  return rowdots(pool, T, T, true);
}

Mat matmul_nt(Pool& pool, const Mat& A, const Mat& B) { return rowdots(pool, A, B, false); }

Mat matmul(Pool& pool, const Mat& A, const Mat& B) {
  Mat Bt = transpose(pool, B);
  return rowdots(pool, A, Bt, false);
}

Mat matmul_tn(Pool& pool, const Mat& A, const Mat& B) {
  Mat At = transpose(pool, A);
  Mat Bt = transpose(pool, B);
  return rowdots(pool, At, Bt, false);
}

// ---------------------------------------------------------------------------
// symmetric eigenproblem, top-k
// ---------------------------------------------------------------------------

// Householder tridiagonalisation in place.  On return d (diagonal), e
// (e[i] couples i and i+1), beta[k] and the reflector v_k stored in
// A.row(k)[k+1 .. n-1] define T = Q^T A Q, Q = H_0 H_1 ... H_{n-3},
// H_k = I - beta_k v_k v_k^T acting on indices k+1 .. n-1.
static void tridiagonalize(Pool& pool, Mat& A, std::vector<double>& d, std::vector<double>& e,
                           std::vector<double>& beta) {
  const int64_t n = A.rows;
  d.assign((size_t)n, 0.0);
  e.assign((size_t)std::max<int64_t>(n, 1), 0.0);
  beta.assign((size_t)std::max<int64_t>(n, 1), 0.0);
  std::vector<double> p((size_t)n), w((size_t)n);
  for (int64_t k = 0; k + 2 < n; ++k) {
    const int64_t len = n - k - 1;
    double* x = A.row(k) + k + 1;
    double nrm2 = 0.0;
    for (int64_t i = 0; i < len; ++i) nrm2 += x[i] * x[i];
    d[(size_t)k] = A(k, k);
    double tail2 = nrm2 - x[0] * x[0];
    if (tail2 == 0.0) {                     // already tridiagonal in this column
      e[(size_t)k] = x[0];
      beta[(size_t)k] = 0.0;
      continue;
    }
    const double nrm = std::sqrt(nrm2);
    const double alpha = x[0] >= 0 ? -nrm : nrm;
    x[0] -= alpha;                          // v = x - alpha e1 (stored in place)
    const double vtv = x[0] * x[0] + tail2;
    const double b = 2.0 / vtv;
    beta[(size_t)k] = b;
    e[(size_t)k] = alpha;
    const int64_t off = k + 1;
    auto symv = [&](int64_t r0, int64_t r1) {
      for (int64_t i = r0; i < r1; ++i) {
        const double* ai = A.row(off + i) + off;
        double s = 0.0;
        for (int64_t j = 0; j < len; ++j) s += ai[j] * x[j];
        p[(size_t)i] = b * s;
      }
    };
    if (len >= 256) pool.parallel_for(len, symv); else symv(0, len);
    double pv = 0.0;
    for (int64_t i = 0; i < len; ++i) pv += p[(size_t)i] * x[i];
    const double K = 0.5 * b * pv;
    for (int64_t i = 0; i < len; ++i) w[(size_t)i] = p[(size_t)i] - K * x[i];
    auto upd = [&](int64_t r0, int64_t r1) {
      for (int64_t i = r0; i < r1; ++i) {
        double* ai = A.row(off + i) + off;
        const double vi = x[i], wi = w[(size_t)i];
        for (int64_t j = 0; j < len; ++j) ai[j] -= vi * w[(size_t)j] + wi * x[j];
      }
    };
    if (len >= 256) pool.parallel_for(len, upd); else upd(0, len);
  }
  if (n >= 2) {
    d[(size_t)(n - 2)] = A(n - 2, n - 2);
    e[(size_t)(n - 2)] = A(n - 2, n - 1);
  }
  if (n >= 1) d[(size_t)(n - 1)] = A(n - 1, n - 1);
  if (n >= 1) e[(size_t)(n - 1)] = 0.0;
}

// Number of eigenvalues of T strictly below x (Sturm sequence via the LDL^T
// pivots of T - x I).
static int64_t sturm_count(const std::vector<double>& d, const std::vector<double>& e2, double x,
                           double pivmin) {
  const int64_t n = (int64_t)d.size();
  int64_t cnt = 0;
  double q = d[0] - x;
  if (std::fabs(q) < pivmin) q = -pivmin;
  if (q < 0) ++cnt;
  for (int64_t i = 1; i < n; ++i) {
    q = d[(size_t)i] - x - e2[(size_t)(i - 1)] / q;
    if (std::fabs(q) < pivmin) q = -pivmin;
    if (q < 0) ++cnt;
  }
  return cnt;
}

// Solve (T - lam I) x = b in place on b, T tridiagonal (d, e), by Gaussian
// elimination with partial pivoting; zero pivots are replaced by `tiny`.
static void tri_shift_solve(const std::vector<double>& d, const std::vector<double>& e, double lam,
                            double tiny, std::vector<double>& b) {
  const int64_t n = (int64_t)d.size();
  std::vector<double> D((size_t)n), U1((size_t)n, 0.0), U2((size_t)n, 0.0), mult((size_t)n, 0.0);
  std::vector<char> sw((size_t)n, 0);
  for (int64_t i = 0; i < n; ++i) {
    D[(size_t)i] = d[(size_t)i] - lam;
    if (i + 1 < n) U1[(size_t)i] = e[(size_t)i];
  }
  for (int64_t i = 0; i + 1 < n; ++i) {
    const double sub = e[(size_t)i];
    if (std::fabs(D[(size_t)i]) >= std::fabs(sub)) {
      if (D[(size_t)i] == 0.0) D[(size_t)i] = tiny;
      const double m = sub / D[(size_t)i];
      mult[(size_t)i] = m;
      D[(size_t)(i + 1)] -= m * U1[(size_t)i];
      // U1[i+1] unchanged (row i has no entry at column i+2)
    } else {
      const double m = D[(size_t)i] / sub;
      mult[(size_t)i] = m;
      sw[(size_t)i] = 1;
      const double oldU1i = U1[(size_t)i], oldDi1 = D[(size_t)(i + 1)];
      const double oldU1i1 = (i + 1 < n - 1) ? U1[(size_t)(i + 1)] : 0.0;
      D[(size_t)i] = sub;
      U1[(size_t)i] = oldDi1;
      U2[(size_t)i] = oldU1i1;
      D[(size_t)(i + 1)] = oldU1i - m * oldDi1;
      if (i + 1 < n - 1) U1[(size_t)(i + 1)] = -m * oldU1i1;
    }
  }
  if (D[(size_t)(n - 1)] == 0.0) D[(size_t)(n - 1)] = tiny;
  for (int64_t i = 0; i + 1 < n; ++i) {
    if (sw[(size_t)i]) std::swap(b[(size_t)i], b[(size_t)(i + 1)]);
    b[(size_t)(i + 1)] -= mult[(size_t)i] * b[(size_t)i];
  }
  for (int64_t i = n - 1; i >= 0; --i) {
    double s = b[(size_t)i];
    if (i + 1 < n) s -= U1[(size_t)i] * b[(size_t)(i + 1)];
    if (i + 2 < n) s -= U2[(size_t)i] * b[(size_t)(i + 2)];
    b[(size_t)i] = s / D[(size_t)i];
  }
}

static uint64_t splitmix(uint64_t& s) {
  uint64_t z = (s += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
static double urand(uint64_t& s) { return (double)(splitmix(s) >> 11) * (1.0 / 9007199254740992.0) - 0.5; }

static void normalize(std::vector<double>& x) {
  double s = 0.0;
  for (double v : x) s += v * v;
  s = std::sqrt(s);
  if (s > 0)
    for (double& v : x) v /= s;
}

bool sym_eig_top(Pool& pool, Mat& A, int k, std::vector<double>& w, Mat& V) {
  const int64_t n = A.rows;
  if (k <= 0 || k > n) return false;
  std::vector<double> d, e, beta;
  tridiagonalize(pool, A, d, e, beta);

  // Gershgorin bounds and pivot floor
  double lo = std::numeric_limits<double>::infinity(), hi = -lo, tnorm = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    double r = (i > 0 ? std::fabs(e[(size_t)(i - 1)]) : 0.0) + (i + 1 < n ? std::fabs(e[(size_t)i]) : 0.0);
    lo = std::min(lo, d[(size_t)i] - r);
    hi = std::max(hi, d[(size_t)i] + r);
    tnorm = std::max(tnorm, std::fabs(d[(size_t)i]) + r);
  }
  if (tnorm == 0.0) tnorm = 1.0;
  const double eps = std::numeric_limits<double>::epsilon();
  const double pivmin = std::numeric_limits<double>::min() * 1e4 + tnorm * 1e-300;
  std::vector<double> e2((size_t)n, 0.0);
  for (int64_t i = 0; i + 1 < n; ++i) e2[(size_t)i] = e[(size_t)i] * e[(size_t)i];

  // k largest eigenvalues by bisection (ascending index n-1-j)
  w.assign((size_t)k, 0.0);
  bool ok = true;
  pool.parallel_for(k, [&](int64_t j0, int64_t j1) {
    for (int64_t j = j0; j < j1; ++j) {
      const int64_t idx = n - 1 - j;
      double a = lo - eps * tnorm, b = hi + eps * tnorm;
      for (int it = 0; it < 300; ++it) {
        const double mid = 0.5 * (a + b);
        if (mid <= a || mid >= b) break;
        if (b - a <= 2.0 * eps * std::max(std::fabs(a), std::fabs(b)) + pivmin) break;
        if (sturm_count(d, e2, mid, pivmin) > idx) b = mid; else a = mid;
      }
      w[(size_t)j] = 0.5 * (a + b);
    }
  });

  // eigenvectors of T by inverse iteration, clusters re-orthogonalised
  const double tiny = eps * tnorm;
  const double clus = 1e-3 * tnorm;
  std::vector<std::vector<double>> Y((size_t)k, std::vector<double>((size_t)n));
  int64_t cstart = 0;
  for (int64_t j = 0; j < k; ++j) {
    if (j > 0 && std::fabs(w[(size_t)j] - w[(size_t)(j - 1)]) > clus) cstart = j;
    uint64_t seed = 0x243F6A8885A308D3ull ^ (uint64_t)(j * 7919 + 17);
    std::vector<double>& y = Y[(size_t)j];
    for (int64_t i = 0; i < n; ++i) y[(size_t)i] = urand(seed);
    normalize(y);
    for (int it = 0; it < 4; ++it) {
      tri_shift_solve(d, e, w[(size_t)j], tiny, y);
      normalize(y);
      for (int pass = 0; pass < 2; ++pass)
        for (int64_t q = cstart; q < j; ++q) {
          const std::vector<double>& z = Y[(size_t)q];
          double s = 0.0;
          for (int64_t i = 0; i < n; ++i) s += z[(size_t)i] * y[(size_t)i];
          for (int64_t i = 0; i < n; ++i) y[(size_t)i] -= s * z[(size_t)i];
        }
      normalize(y);
    }
    for (double v : y)
      if (!std::isfinite(v)) ok = false;
  }

  // back-transform x = H_0 H_1 ... H_{n-3} y, groups of vectors per pass
  V = Mat(n, k);
  const int64_t G = 8;
  const int64_t ng = (k + G - 1) / G;
  pool.parallel_for(ng, [&](int64_t g0, int64_t g1) {
    for (int64_t g = g0; g < g1; ++g) {
      const int64_t q0 = g * G, q1 = std::min<int64_t>(k, q0 + G);
      for (int64_t kk = n - 3; kk >= 0; --kk) {
        const double b = beta[(size_t)kk];
        if (b == 0.0) continue;
        const double* v = A.row(kk) + kk + 1;
        const int64_t len = n - kk - 1;
        for (int64_t q = q0; q < q1; ++q) {
          double* y = Y[(size_t)q].data() + kk + 1;
          double s = 0.0;
          for (int64_t i = 0; i < len; ++i) s += v[i] * y[i];
          s *= b;
          for (int64_t i = 0; i < len; ++i) y[i] -= s * v[i];
        }
      }
    }
  });
  for (int64_t q = 0; q < k; ++q)
    for (int64_t i = 0; i < n; ++i) V(i, q) = Y[(size_t)q][(size_t)i];
  return ok;
}

// Make the columns of Q (n x k) orthonormal by two passes of modified
// Gram-Schmidt; columns whose norm collapses are replaced by deterministic
// pseudo-random vectors orthogonalised against the others.
static void orthonormalize_columns(Mat& Q) {
  const int64_t n = Q.rows, k = Q.cols;
  std::vector<double> c((size_t)n);
  uint64_t seed = 0x13198A2E03707344ull;
  for (int64_t j = 0; j < k; ++j) {
    for (int64_t i = 0; i < n; ++i) c[(size_t)i] = Q(i, j);
    double n0 = 0.0;
    for (double v : c) n0 += v * v;
    n0 = std::sqrt(n0);
    for (int attempt = 0; attempt < 4; ++attempt) {
      for (int pass = 0; pass < 2; ++pass)
        for (int64_t q = 0; q < j; ++q) {
          double s = 0.0;
          for (int64_t i = 0; i < n; ++i) s += Q(i, q) * c[(size_t)i];
          for (int64_t i = 0; i < n; ++i) c[(size_t)i] -= s * Q(i, q);
        }
      double nn = 0.0;
      for (double v : c) nn += v * v;
      nn = std::sqrt(nn);
      if (nn > 1e-8 * std::max(n0, 1e-300) && nn > 1e-280) {
        for (int64_t i = 0; i < n; ++i) Q(i, j) = c[(size_t)i] / nn;
        break;
      }
      for (int64_t i = 0; i < n; ++i) c[(size_t)i] = urand(seed);
      n0 = 1.0;
    }
  }
}

bool svd_top(Pool& pool, const Mat& A, int k, Mat& U, std::vector<double>& s, Mat& V, bool want_u,
             bool want_v) {
  const int64_t m = A.rows, n = A.cols;
  if (k <= 0 || k > std::min(m, n)) return false;
  std::vector<double> lam;
  Mat E;
  s.assign((size_t)k, 0.0);
  if (m <= n) {
    Mat C = gram_rows(pool, A);
    if (!sym_eig_top(pool, C, k, lam, E)) return false;
    for (int q = 0; q < k; ++q) s[(size_t)q] = std::sqrt(std::max(lam[(size_t)q], 0.0));
    if (want_v) {
      Mat Vt = matmul_tn(pool, E, A);   // k x n = E^T A
      V = Mat(n, k);
      for (int q = 0; q < k; ++q) {
        const double inv = s[(size_t)q] > 0 ? 1.0 / s[(size_t)q] : 0.0;
        for (int64_t i = 0; i < n; ++i) V(i, q) = Vt(q, i) * inv;
      }
      orthonormalize_columns(V);
    }
    if (want_u) U = std::move(E);
  } else {
    Mat C = gram_cols(pool, A);
    if (!sym_eig_top(pool, C, k, lam, E)) return false;
    for (int q = 0; q < k; ++q) s[(size_t)q] = std::sqrt(std::max(lam[(size_t)q], 0.0));
    if (want_u) {
      U = matmul(pool, A, E);           // m x k
      for (int q = 0; q < k; ++q) {
        const double inv = s[(size_t)q] > 0 ? 1.0 / s[(size_t)q] : 0.0;
        for (int64_t i = 0; i < m; ++i) U(i, q) *= inv;
      }
      orthonormalize_columns(U);
    }
    if (want_v) V = std::move(E);
  }
  return true;
}

}  // namespace dyra_host
