// Drives every host-side entry point of the library (preparation, input-aware
// preparation, plan packing, size and offset queries, error paths) on small
// specs of every structure.  Built with AddressSanitizer and
// UndefinedBehaviorSanitizer from the host sources alone (no HIP), so an
// out-of-bounds index, a use after free, a leak or undefined arithmetic in
// the host code ends the run with a report.  Exit status 0 = every check
// passed and the sanitizers stayed silent.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "dyra.h"

namespace {

int failures = 0;

#define CHECK(cond)                                                          \
  do {                                                                       \
    if (!(cond)) {                                                           \
      std::fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                            \
    }                                                                        \
  } while (0)

// xorshift64* normal deviates (Box-Muller); test data only
struct Rng {
  uint64_t s;
  explicit Rng(uint64_t seed) : s(seed * 0x9E3779B97F4A7C15ull + 1) {}
  double uniform() {
    s ^= s >> 12;
    s ^= s << 25;
    s ^= s >> 27;
    return ((s * 0x2545F4914F6CDD1Dull) >> 11) * (1.0 / 9007199254740992.0);
  }
  double normal() {
    double u = uniform(), v = uniform();
    if (u < 1e-300) u = 1e-300;
    return std::sqrt(-2.0 * std::log(u)) * std::cos(6.283185307179586 * v);
  }
};

std::vector<double> randn(size_t n, uint64_t seed) {
  Rng g(seed);
  std::vector<double> x(n);
  for (auto& v : x) v = g.normal();
  return x;
}

dyra_spec make(int32_t kind, int64_t c1, int64_t c2, int32_t r, int32_t k = 0, int32_t mblk = 0,
               int32_t nb = 0, int32_t rb = 0) {
  dyra_spec s;
  std::memset(&s, 0, sizeof s);
  s.kind = kind;
  s.k = k;
  s.mblk = mblk;
  s.nb = nb;
  s.rb = rb;
  s.r = r;
  s.c1 = c1;
  s.c2 = c2;
  return s;
}

// Caller-side storage of one set of host factors, sized by the library.
struct Factors {
  dyra_sizes n{};
  std::vector<double> U, V, B1, B2, Ub, S, Vb, P, R0, Wres, sv;
  dyra_host_factors f{};
  explicit Factors(const dyra_spec& s) {
    CHECK(dyra_prepare_sizes(&s, &n) == DYRA_OK);
    auto take = [](std::vector<double>& v, int64_t count) -> double* {
      v.assign((size_t)count, NAN);
      return count ? v.data() : nullptr;
    };
    f.U = take(U, n.U);
    f.V = take(V, n.V);
    f.B1 = take(B1, n.B1);
    f.B2 = take(B2, n.B2);
    f.Ub = take(Ub, n.Ub);
    f.S = take(S, n.S);
    f.Vb = take(Vb, n.Vb);
    f.P = take(P, n.P);
    f.R0 = take(R0, n.R0);
    f.Wres = take(Wres, n.Wres);
    f.res_sv = take(sv, n.res_sv);
  }
  bool finite() const {
    for (const auto* v : {&U, &V, &B1, &B2, &Ub, &S, &Vb, &P, &R0, &Wres, &sv})
      for (double x : *v)
        if (!std::isfinite(x)) return false;
    return true;
  }
};

void pack_both(const dyra_spec& s, const Factors& F, bool bf16_ok, bool f32_ok) {
  for (int32_t dt : {DYRA_F32, DYRA_BF16}) {
    const bool ok = dt == DYRA_BF16 ? bf16_ok : f32_ok;
    size_t bytes = 0;
    const int rc = dyra_plan_size(&s, dt, &bytes);
    if (!ok) {
      CHECK(rc == DYRA_EDTYPE);
      continue;
    }
    CHECK(rc == DYRA_OK && bytes > 0);
    std::vector<unsigned char> plan(bytes, 0xA5);
    CHECK(dyra_plan_pack(&s, &F.f, dt, plan.data()) == DYRA_OK);
    dyra_ws_offsets o;
    CHECK(dyra_workspace_offsets(&s, 3, 77, dt, &o) == DYRA_OK);
    CHECK(o.total > o.status && o.total > o.prec && o.lt_pitch >= 3 * 77);
  }
}

void lowrank(int64_t c1, int64_t c2, int32_t k, int32_t r, uint64_t seed) {
  const dyra_spec s = make(DYRA_LOWRANK, c1, c2, r, k);
  const auto W = randn((size_t)(c1 * c2), seed);
  Factors F(s);
  CHECK(dyra_prepare(&s, W.data(), &F.f, 3) == DYRA_OK);
  CHECK(F.finite());
  pack_both(s, F, true, true);
  // input-aware starts
  const int64_t n_cal = 2 * c1 + 5;
  auto X = randn((size_t)(n_cal * c1), seed + 7);
  for (int64_t t = 0; t < n_cal; ++t)
    for (int64_t i = 0; i < c1; ++i) X[(size_t)(t * c1 + i)] *= 1.0 + (double)(i % 5);
  for (int32_t mode : {DYRA_INPUT_AWARE_DIAG, DYRA_INPUT_AWARE_CHOL}) {
    Factors G(s);
    CHECK(dyra_prepare_input_aware(&s, W.data(), X.data(), n_cal, mode, &G.f, 2) == DYRA_OK);
    CHECK(G.finite());
    pack_both(s, G, true, true);
  }
  // fewer calibration rows than channels (the Cholesky transform leans on its ridge)
  Factors H(s);
  CHECK(dyra_prepare_input_aware(&s, W.data(), X.data(), 3, DYRA_INPUT_AWARE_CHOL, &H.f, 1) == DYRA_OK);
  CHECK(H.finite());
  // error paths
  Factors E(s);
  CHECK(dyra_prepare_input_aware(&s, W.data(), X.data(), 0, DYRA_INPUT_AWARE_DIAG, &E.f, 1) == DYRA_ESHAPE);
  CHECK(dyra_prepare_input_aware(&s, W.data(), X.data(), n_cal, 7, &E.f, 1) == DYRA_EINVAL);
  X[5] = NAN;
  CHECK(dyra_prepare_input_aware(&s, W.data(), X.data(), n_cal, DYRA_INPUT_AWARE_DIAG, &E.f, 1) == DYRA_EINVAL);
  std::vector<double> Z((size_t)(n_cal * c1), 0.0);
  CHECK(dyra_prepare_input_aware(&s, W.data(), Z.data(), n_cal, DYRA_INPUT_AWARE_DIAG, &E.f, 1) == DYRA_EINVAL);
}

void monarch(int32_t m, int32_t r, uint64_t seed) {
  const int64_t c = (int64_t)m * m;
  const dyra_spec s = make(DYRA_MONARCH, c, c, r, 0, m);
  const auto W = randn((size_t)(c * c), seed);
  Factors F(s);
  CHECK(dyra_prepare(&s, W.data(), &F.f, 4) == DYRA_OK);
  CHECK(F.finite());
  pack_both(s, F, m == 32, false);
}

void blast(int32_t kind, int64_t c1, int64_t c2, int32_t nb, int32_t rb, int32_t r, uint64_t seed) {
  const dyra_spec s = make(kind, c1, c2, r, 0, 0, nb, rb);
  const auto W = randn((size_t)(c1 * c2), seed);
  Factors F(s);
  CHECK(dyra_prepare(&s, W.data(), &F.f, 2) == DYRA_OK);
  CHECK(F.finite());
  pack_both(s, F, true, false);
}

void error_paths() {
  const dyra_spec good = make(DYRA_LOWRANK, 64, 96, 8, 16);
  dyra_sizes n;
  CHECK(dyra_prepare_sizes(nullptr, &n) == DYRA_EINVAL);
  CHECK(dyra_prepare_sizes(&good, nullptr) == DYRA_EINVAL);
  dyra_spec bad = good;
  bad.r = 12;   // not a multiple of 8
  CHECK(dyra_prepare_sizes(&bad, &n) == DYRA_ESHAPE);
  bad = good;
  bad.k = 96;   // k + r > min(c1, c2)
  CHECK(dyra_prepare_sizes(&bad, &n) == DYRA_ESHAPE);
  bad = good;
  bad.kind = 9;
  CHECK(dyra_prepare_sizes(&bad, &n) == DYRA_EINVAL);
  Factors F(good);
  CHECK(dyra_prepare(&good, nullptr, &F.f, 1) == DYRA_EINVAL);
  size_t bytes = 0;
  CHECK(dyra_plan_size(&good, 5, &bytes) == DYRA_EINVAL);
  dyra_ws_offsets o;
  CHECK(dyra_workspace_offsets(&good, 0, 10, DYRA_BF16, &o) == DYRA_ESHAPE);
  CHECK(dyra_workspace_offsets(&good, 1 << 20, 1 << 12, DYRA_BF16, &o) == DYRA_ESHAPE);
  for (int code = -6; code <= 0; ++code) CHECK(dyra_status_string(code) != nullptr);
}

}  // namespace

// argument "small": skip the two largest specs (for the slower ThreadSanitizer build)
int main(int argc, char** argv) {
  const bool small = argc > 1 && std::strcmp(argv[1], "small") == 0;
  error_paths();
  lowrank(64, 96, 16, 8, 1);
  if (!small) lowrank(384, 384, 256, 64, 2);   // k + r = 320: the first-stage tile layout of the plan
  monarch(8, 8, 3);
  if (!small) monarch(32, 32, 4);
  blast(DYRA_BLAST, 64, 256, 2, 8, 8, 5);
  blast(DYRA_BLAST_DIAG, 64, 256, 2, 8, 8, 6);
  blast(DYRA_BLAST, 96, 128, 1, 16, 16, 7);
  if (failures) {
    std::fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  std::printf("host entry points: all checks passed\n");
  return 0;
}
