// Host float64 linear algebra for the offline DyRA preparation:
// threaded Gram products, Householder tridiagonalisation, Sturm bisection,
// inverse iteration and back-transformation -> top-k symmetric eigenpairs,
// and top-k singular triplets built on them.  No LAPACK is used.
#pragma once

#include <cstdint>
#include <functional>
#include <vector>

namespace dyra_host {

struct Mat {
  int64_t rows = 0, cols = 0;
  std::vector<double> a;
  Mat() = default;
  Mat(int64_t r, int64_t c) : rows(r), cols(c), a((size_t)(r * c), 0.0) {}
  double* row(int64_t i) { return a.data() + i * cols; }
  const double* row(int64_t i) const { return a.data() + i * cols; }
  double& operator()(int64_t i, int64_t j) { return a[(size_t)(i * cols + j)]; }
  double operator()(int64_t i, int64_t j) const { return a[(size_t)(i * cols + j)]; }
};

// Fixed-size worker pool; parallel_for splits [0, n) into contiguous chunks.
class Pool {
 public:
  explicit Pool(int nthreads);
  ~Pool();
  int size() const { return nthreads_; }
  void parallel_for(int64_t n, const std::function<void(int64_t, int64_t)>& fn);

 private:
  struct Impl;
  Impl* impl_;
  int nthreads_;
};

// C = A A^T (A: m x n) -> m x m symmetric.
Mat gram_rows(Pool& pool, const Mat& A);
// C = A^T A via a transposed copy.
Mat gram_cols(Pool& pool, const Mat& A);
Mat transpose(Pool& pool, const Mat& A);
// C = A B (A: m x k, B: k x n).
Mat matmul(Pool& pool, const Mat& A, const Mat& B);
// C = A B^T (A: m x k, B: n x k).
Mat matmul_nt(Pool& pool, const Mat& A, const Mat& B);
// C = A^T B (A: k x m, B: k x n).
Mat matmul_tn(Pool& pool, const Mat& A, const Mat& B);

// Top-k eigenpairs of a symmetric matrix (A is overwritten).  Eigenvalues
// descending in `w`, eigenvectors as the COLUMNS of the returned n x k matrix.
// Returns false if the iteration failed to converge.
bool sym_eig_top(Pool& pool, Mat& A, int k, std::vector<double>& w, Mat& V);

// Top-k singular triplets of A (m x n) through the Gram matrix of the smaller
// side: U (m x k, columns), s (k, descending), V (n x k, columns).  Singular
// vectors of (numerically) zero singular values are completed to an
// orthonormal set.
bool svd_top(Pool& pool, const Mat& A, int k, Mat& U, std::vector<double>& s, Mat& V,
             bool want_u = true, bool want_v = true);

}  // namespace dyra_host
