// Offline float64 linear algebra: Gram matrix and a top-r symmetric
// eigensolver (Householder tridiagonalisation + bisection + inverse
// iteration), used for the top-r SVD of the smoothed weight.  The methods
// are the textbook ones for the symmetric eigenproblem (G. H. Golub and
// C. F. Van Loan, "Matrix Computations", the chapter on the symmetric
// eigenvalue problem: Householder tridiagonalisation, Sturm-sequence
// bisection, inverse iteration), written here from their mathematics.
#include "host_linalg.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <limits>
#include <vector>

#include "host_threads.h"

namespace svdq {

typedef double v4d __attribute__((vector_size(32)));

static inline v4d load4(const double *p) {
  v4d v;
  std::memcpy(&v, p, sizeof(v));
  return v;
}

static inline double hsum(v4d v) { return (v[0] + v[1]) + (v[2] + v[3]); }

// ------------------------------------------------------------------ Gram
void gram_rows(const double *B, int64_t n, int64_t len, double *G) {
  const int64_t TB = 64;    // tile of rows on each side
  const int64_t CH = 256;   // chunk along the reduction
  const int64_t nt = (n + TB - 1) / TB;
  // lower-triangle tile pairs (ti >= tj), enumerated in one index
  std::vector<std::pair<int64_t, int64_t>> tiles;
  for (int64_t ti = 0; ti < nt; ++ti)
    for (int64_t tj = 0; tj <= ti; ++tj) tiles.emplace_back(ti, tj);
  parallel_for((int64_t)tiles.size(), 1, [&](int64_t t0, int64_t t1) {
    std::vector<double> acc(TB * TB);
    for (int64_t t = t0; t < t1; ++t) {
      const int64_t i0 = tiles[t].first * TB, j0 = tiles[t].second * TB;
      const int64_t ni = std::min(TB, n - i0), nj = std::min(TB, n - j0);
      std::fill(acc.begin(), acc.end(), 0.0);
      for (int64_t c0 = 0; c0 < len; c0 += CH) {
        const int64_t cl = std::min(CH, len - c0);
        const int64_t cv = cl & ~int64_t(3);
        for (int64_t a = 0; a < ni; a += 4) {
          const int64_t na = std::min<int64_t>(4, ni - a);
          const double *x[4];
          for (int q = 0; q < 4; ++q) x[q] = B + (i0 + a + std::min<int64_t>(q, na - 1)) * len + c0;
          for (int64_t b = 0; b < nj; b += 4) {
            const int64_t nb = std::min<int64_t>(4, nj - b);
            const double *y[4];
            for (int q = 0; q < 4; ++q) y[q] = B + (j0 + b + std::min<int64_t>(q, nb - 1)) * len + c0;
            v4d s[4][4];
            for (int p = 0; p < 4; ++p)
              for (int q = 0; q < 4; ++q) s[p][q] = v4d{0, 0, 0, 0};
            for (int64_t k = 0; k < cv; k += 4) {
              v4d xv[4], yv[4];
              for (int p = 0; p < 4; ++p) xv[p] = load4(x[p] + k);
              for (int q = 0; q < 4; ++q) yv[q] = load4(y[q] + k);
              for (int p = 0; p < 4; ++p)
                for (int q = 0; q < 4; ++q) s[p][q] += xv[p] * yv[q];
            }
            for (int p = 0; p < na; ++p)
              for (int q = 0; q < nb; ++q) {
                double t2 = hsum(s[p][q]);
                for (int64_t k = cv; k < cl; ++k) t2 += x[p][k] * y[q][k];
                acc[(a + p) * TB + (b + q)] += t2;
              }
          }
        }
      }
      for (int64_t a = 0; a < ni; ++a)
        for (int64_t b = 0; b < nj; ++b) {
          G[(i0 + a) * n + (j0 + b)] = acc[a * TB + b];
          G[(j0 + b) * n + (i0 + a)] = acc[a * TB + b];
        }
    }
  });
}

// ------------------------------------------------ tridiagonalisation
// Householder reduction of symmetric A to tridiagonal T = Q^T A Q.
// Reflector k acts on indices k+1..n-1: H_k = I - beta_k v_k v_k^T, with
// v_k stored in column k of A below the subdiagonal position.
static void tridiagonalize(double *A, int64_t n, double *d, double *e, double *beta) {
  std::vector<double> v(n), p(n);
  for (int64_t k = 0; k + 2 < n; ++k) {
    const int64_t m = n - k - 1;
    double scale = 0.0;
    for (int64_t i = 0; i < m; ++i) scale = std::max(scale, std::fabs(A[(k + 1 + i) * n + k]));
    d[k] = A[k * n + k];
    if (scale == 0.0) {
      e[k] = 0.0;
      beta[k] = 0.0;
      for (int64_t i = 0; i < m; ++i) A[(k + 1 + i) * n + k] = 0.0;
      continue;
    }
    double ss = 0.0;
    for (int64_t i = 0; i < m; ++i) {
      v[i] = A[(k + 1 + i) * n + k];
      double t = v[i] / scale;
      ss += t * t;
    }
    const double xnorm = scale * std::sqrt(ss);
    const double alpha = v[0] > 0 ? -xnorm : xnorm;
    const double vtv = 2.0 * xnorm * (xnorm + std::fabs(v[0]));  // ||x - alpha e1||^2
    v[0] -= alpha;
    const double b = 2.0 / vtv;
    // p = b * A_sub v
    double *Asub = A + (k + 1) * n + (k + 1);
    const double *vp = v.data();
    double *pp = p.data();
    parallel_for(m, 64, [&](int64_t r0, int64_t r1) {
      for (int64_t i = r0; i < r1; ++i) {
        const double *row = Asub + i * n;
        double s = 0.0;
        for (int64_t j = 0; j < m; ++j) s += row[j] * vp[j];
        pp[i] = b * s;
      }
    });
    double pv = 0.0;
    for (int64_t i = 0; i < m; ++i) pv += p[i] * v[i];
    const double K = 0.5 * b * pv;
    for (int64_t i = 0; i < m; ++i) p[i] -= K * v[i];   // w
    // A_sub -= v w^T + w v^T
    parallel_for(m, 64, [&](int64_t r0, int64_t r1) {
      for (int64_t i = r0; i < r1; ++i) {
        double *row = Asub + i * n;
        const double vi = vp[i], wi = pp[i];
        for (int64_t j = 0; j < m; ++j) row[j] -= vi * pp[j] + wi * vp[j];
      }
    });
    e[k] = alpha;
    beta[k] = b;
    for (int64_t i = 0; i < m; ++i) A[(k + 1 + i) * n + k] = v[i];
  }
  if (n >= 2) {
    d[n - 2] = A[(n - 2) * n + (n - 2)];
    e[n - 2] = A[(n - 1) * n + (n - 2)];
    beta[n - 2] = 0.0;
  }
  d[n - 1] = A[(n - 1) * n + (n - 1)];
}

// Number of eigenvalues of the tridiagonal (d, e) that are < x (Sturm count).
static int64_t sturm_less(const double *d, const double *e2, int64_t n, double x, double pivmin) {
  int64_t c = 0;
  double q = d[0] - x;
  if (std::fabs(q) < pivmin) q = -pivmin;
  if (q < 0) ++c;
  for (int64_t i = 1; i < n; ++i) {
    q = d[i] - x - e2[i - 1] / q;
    if (std::fabs(q) < pivmin) q = -pivmin;
    if (q < 0) ++c;
  }
  return c;
}

// Solves (T - lambda I) y = y in place by Gaussian elimination with partial
// pivoting on the tridiagonal matrix.
static void tri_shift_solve(const double *d, const double *e, int64_t n, double lambda,
                            double tiny, double *y, std::vector<double> &u0,
                            std::vector<double> &u1, std::vector<double> &u2,
                            std::vector<double> &L, std::vector<char> &P) {
  double c0 = d[0] - lambda, c1 = n > 1 ? e[0] : 0.0, c2 = 0.0;
  for (int64_t i = 0; i + 1 < n; ++i) {
    const double r0 = e[i], r1 = d[i + 1] - lambda, r2 = (i + 2 < n) ? e[i + 1] : 0.0;
    if (std::fabs(c0) >= std::fabs(r0)) {
      if (c0 == 0.0) c0 = tiny;
      const double l = r0 / c0;
      u0[i] = c0; u1[i] = c1; u2[i] = c2; L[i] = l; P[i] = 0;
      c0 = r1 - l * c1;
      c1 = r2 - l * c2;
      c2 = 0.0;
    } else {
      const double l = c0 / r0;
      u0[i] = r0; u1[i] = r1; u2[i] = r2; L[i] = l; P[i] = 1;
      c0 = c1 - l * r1;
      c1 = c2 - l * r2;
      c2 = 0.0;
    }
  }
  if (c0 == 0.0) c0 = tiny;
  u0[n - 1] = c0;
  for (int64_t i = 0; i + 1 < n; ++i) {
    if (P[i]) std::swap(y[i], y[i + 1]);
    y[i + 1] -= L[i] * y[i];
  }
  y[n - 1] /= u0[n - 1];
  if (n >= 2) y[n - 2] = (y[n - 2] - u1[n - 2] * y[n - 1]) / u0[n - 2];
  for (int64_t i = n - 3; i >= 0; --i)
    y[i] = (y[i] - u1[i] * y[i + 1] - u2[i] * y[i + 2]) / u0[i];
}

static void normalize(double *y, int64_t n) {
  double mx = 0.0;
  for (int64_t i = 0; i < n; ++i) mx = std::max(mx, std::fabs(y[i]));
  if (mx == 0.0) return;
  double s = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    y[i] /= mx;
    s += y[i] * y[i];
  }
  s = 1.0 / std::sqrt(s);
  for (int64_t i = 0; i < n; ++i) y[i] *= s;
}

int sym_top_eigs(double *A, int64_t n, int64_t r, double *w, double *Z) {
  if (r <= 0) return 0;
  for (int64_t i = 0; i < n * n; ++i)
    if (!std::isfinite(A[i])) return 1;
  std::vector<double> d(n), e(std::max<int64_t>(n, 1)), beta(std::max<int64_t>(n, 1));
  if (n == 1) {
    w[0] = A[0];
    Z[0] = 1.0;
    return 0;
  }
  tridiagonalize(A, n, d.data(), e.data(), beta.data());
  std::vector<double> e2(n);
  double tnorm = 0.0, emax2 = 0.0;
  double glo = std::numeric_limits<double>::infinity(), ghi = -glo;
  for (int64_t i = 0; i < n; ++i) {
    const double el = i > 0 ? std::fabs(e[i - 1]) : 0.0;
    const double er = i + 1 < n ? std::fabs(e[i]) : 0.0;
    glo = std::min(glo, d[i] - el - er);
    ghi = std::max(ghi, d[i] + el + er);
    tnorm = std::max(tnorm, std::fabs(d[i]) + el + er);
    if (i + 1 < n) {
      e2[i] = e[i] * e[i];
      emax2 = std::max(emax2, e2[i]);
    }
  }
  const double eps = std::numeric_limits<double>::epsilon();
  const double safemin = std::numeric_limits<double>::min();
  const double pivmin = std::max(safemin, safemin * emax2);
  if (tnorm == 0.0) tnorm = 1.0;
  glo -= 2.0 * eps * tnorm + pivmin;
  ghi += 2.0 * eps * tnorm + pivmin;
  // bisection for the r largest eigenvalues (ascending index n-1-j)
  parallel_for(r, 1, [&](int64_t j0, int64_t j1) {
    for (int64_t j = j0; j < j1; ++j) {
      const int64_t idx = n - 1 - j;
      double lo = glo, hi = ghi;
      for (int it = 0; it < 400; ++it) {
        const double mid = 0.5 * (lo + hi);
        if (hi - lo <= 2.0 * eps * std::max(std::fabs(lo), std::fabs(hi)) + pivmin) break;
        if (sturm_less(d.data(), e2.data(), n, mid, pivmin) > idx) hi = mid;
        else lo = mid;
      }
      w[j] = 0.5 * (lo + hi);
    }
  });
  // inverse iteration, descending order, re-orthogonalising within clusters
  std::vector<double> Y(n * r);
  std::vector<double> u0(n), u1(n), u2(n), L(n);
  std::vector<char> P(n);
  const double ortol = 1e-3 * tnorm;
  const double tiny = eps * tnorm;
  int64_t cluster_start = 0;
  for (int64_t j = 0; j < r; ++j) {
    if (j > 0 && w[j - 1] - w[j] > ortol) cluster_start = j;
    double *y = &Y[j * n];
    // deterministic start vector
    uint64_t s = 0x9E3779B97F4A7C15ull * (uint64_t)(j + 1);
    for (int64_t i = 0; i < n; ++i) {
      s ^= s << 13; s ^= s >> 7; s ^= s << 17;
      y[i] = (double)(s >> 11) * (1.0 / 9007199254740992.0) - 0.5;
    }
    // a tiny separation keeps equal eigenvalues from producing equal vectors
    const double shift = w[j] + (double)(j - cluster_start) * 1e-2 * tiny;
    for (int it = 0; it < 5; ++it) {
      normalize(y, n);
      tri_shift_solve(d.data(), e.data(), n, shift, tiny, y, u0, u1, u2, L, P);
      normalize(y, n);
      for (int64_t c = cluster_start; c < j; ++c) {
        const double *yc = &Y[c * n];
        double dot = 0.0;
        for (int64_t i = 0; i < n; ++i) dot += yc[i] * y[i];
        for (int64_t i = 0; i < n; ++i) y[i] -= dot * yc[i];
      }
    }
    normalize(y, n);
  }
  // back-transform: z = H_0 H_1 ... H_{n-3} y
  parallel_for(r, 1, [&](int64_t j0, int64_t j1) {
    for (int64_t j = j0; j < j1; ++j) {
      double *z = &Y[j * n];
      for (int64_t k = n - 3; k >= 0; --k) {
        if (beta[k] == 0.0) continue;
        const int64_t m = n - k - 1;
        double dot = 0.0;
        for (int64_t i = 0; i < m; ++i) dot += A[(k + 1 + i) * n + k] * z[k + 1 + i];
        dot *= beta[k];
        for (int64_t i = 0; i < m; ++i) z[k + 1 + i] -= dot * A[(k + 1 + i) * n + k];
      }
    }
  });
  for (int64_t i = 0; i < n; ++i)
    for (int64_t j = 0; j < r; ++j) Z[i * r + j] = Y[j * n + i];
  for (int64_t j = 0; j < r; ++j)
    if (!std::isfinite(w[j])) return 2;
  return 0;
}

// ---------------------------------------------------------------- SVD
int svd_top(const double *A, int64_t N, int64_t K, int64_t r, double *U, double *sigma,
            double *V) {
  if (r <= 0) return 0;
  const bool rows_side = N <= K;   // Gram of the smaller side
  const int64_t n = rows_side ? N : K, len = rows_side ? K : N;
  std::vector<double> Bt;
  const double *B = A;
  if (!rows_side) {
    Bt.resize((size_t)K * N);
    parallel_for(K, 16, [&](int64_t k0, int64_t k1) {
      for (int64_t k = k0; k < k1; ++k)
        for (int64_t i = 0; i < N; ++i) Bt[k * N + i] = A[i * K + k];
    });
    B = Bt.data();
  }
  std::vector<double> G((size_t)n * n), lam(r), E((size_t)n * r);
  gram_rows(B, n, len, G.data());
  int rc = sym_top_eigs(G.data(), n, r, lam.data(), E.data());
  if (rc) return rc;
  for (int64_t t = 0; t < r; ++t) sigma[t] = std::sqrt(std::max(lam[t], 0.0));
  // the other side: F = B^T E diag(1/sigma), F is [len][r]
  std::vector<double> F((size_t)len * r, 0.0);
  parallel_for(len, 64, [&](int64_t c0, int64_t c1) {
    for (int64_t c = c0; c < c1; ++c) {
      double *f = &F[c * r];
      for (int64_t i = 0; i < n; ++i) {
        const double b = B[i * len + c];
        const double *ei = &E[i * r];
        for (int64_t t = 0; t < r; ++t) f[t] += b * ei[t];
      }
      for (int64_t t = 0; t < r; ++t) f[t] = sigma[t] > 0.0 ? f[t] / sigma[t] : 0.0;
    }
  });
  if (rows_side) {   // E = U [N][r], F = V [K][r]
    std::memcpy(U, E.data(), sizeof(double) * N * r);
    std::memcpy(V, F.data(), sizeof(double) * K * r);
  } else {           // E = V [K][r], F = U [N][r]
    std::memcpy(V, E.data(), sizeof(double) * K * r);
    std::memcpy(U, F.data(), sizeof(double) * N * r);
  }
  return 0;
}

}  // namespace svdq
