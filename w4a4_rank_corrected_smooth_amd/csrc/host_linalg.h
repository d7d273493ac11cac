// Dense float64 linear algebra for the offline preparation: the top-r
// singular triplets of the smoothed weight, computed from the Gram matrix of
// its smaller side with a symmetric eigensolver.
#pragma once

#include <cstdint>

namespace svdq {

// G[i][j] = <B[i,:], B[j,:]> for B [n][len] row-major; G is [n][n], full.
void gram_rows(const double *B, int64_t n, int64_t len, double *G);

// Top-r eigenpairs of the symmetric n x n matrix A (row-major, full storage;
// destroyed).  Eigenvalues in descending order go to w[r]; the matching
// orthonormal eigenvectors to Z [n][r] (column t is eigenvector t).
// Method (Golub & Van Loan, "Matrix Computations", ch. 8): Householder
// tridiagonalisation, Sturm-sequence bisection for the r largest
// eigenvalues, inverse iteration on the tridiagonal matrix with
// re-orthogonalisation inside clusters, then back-transformation.
// Returns 0 on success, nonzero if a non-finite value appeared.
int sym_top_eigs(double *A, int64_t n, int64_t r, double *w, double *Z);

// Top-r SVD of A [N][K] (row-major): U [N][r], sigma [r] (descending),
// V [K][r], with A ~ U diag(sigma) V^T.  Returns nonzero on failure.
int svd_top(const double *A, int64_t N, int64_t K, int64_t r, double *U,
            double *sigma, double *V);

}  // namespace svdq
