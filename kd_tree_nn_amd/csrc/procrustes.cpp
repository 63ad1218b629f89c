// Host rigid solve (CUDA-KDTree ICP article, §2.1): centroids, the 3x3
// cross-covariance H, its SVD, R = V diag(1, 1, d) U^T, t from the centroids.
// The article writes R = U V^T for H taken target-first; with H taken
// source-first, H = sum (s - mu_s)(m - mu_m)^T, the same rotation is V U^T.
// The sign d = sign det(V U^T) keeps R a proper rotation when the best
// orthogonal fit is a reflection (e.g. planar data).
//
// SVD: one-sided Jacobi (Hestenes) on the columns of H, in fp64: plane
// rotations V make the columns of H V mutually orthogonal, then
// H V = U S with S the column norms.
#include <cmath>

#include "kdnn_internal.hpp"

namespace kdnn {

namespace {

double det3(const double M[3][3])
{
    return M[0][0] * (M[1][1] * M[2][2] - M[1][2] * M[2][1]) -
           M[0][1] * (M[1][0] * M[2][2] - M[1][2] * M[2][0]) +
           M[0][2] * (M[1][0] * M[2][1] - M[1][1] * M[2][0]);
}

// H = U diag(s) V^T with s sorted descending.  Columns of U for zero singular
// values are left as zero; the caller completes them.
void jacobi_svd3(const double H[3][3], double U[3][3], double s[3], double V[3][3])
{
    double A[3][3];
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j) {
            A[i][j] = H[i][j];
            V[i][j] = i == j ? 1.0 : 0.0;
        }
    static const int pairs[3][2] = {{0, 1}, {0, 2}, {1, 2}};
    for (int sweep = 0; sweep < 60; ++sweep) {
        double off = 0.0;
        for (const auto &pq : pairs) {
            const int p = pq[0], q = pq[1];
            double alpha = 0, beta = 0, gamma = 0;
            for (int i = 0; i < 3; ++i) {
                alpha += A[i][p] * A[i][p];
                beta += A[i][q] * A[i][q];
                gamma += A[i][p] * A[i][q];
            }
            if (gamma == 0.0) continue;
            const double scale = std::sqrt(alpha * beta);
            if (scale == 0.0 || std::fabs(gamma) <= 1e-16 * scale) continue;
            off = std::fmax(off, std::fabs(gamma) / scale);
            const double zeta = (beta - alpha) / (2.0 * gamma);
            const double tt = (zeta >= 0 ? 1.0 : -1.0) / (std::fabs(zeta) + std::sqrt(1.0 + zeta * zeta));
            const double c = 1.0 / std::sqrt(1.0 + tt * tt), sn = c * tt;
            for (int i = 0; i < 3; ++i) {
                const double ap = A[i][p], aq = A[i][q];
                A[i][p] = c * ap - sn * aq;
                A[i][q] = sn * ap + c * aq;
                const double vp = V[i][p], vq = V[i][q];
                V[i][p] = c * vp - sn * vq;
                V[i][q] = sn * vp + c * vq;
            }
        }
        if (off < 1e-15) break;
    }
    for (int j = 0; j < 3; ++j)
        s[j] = std::sqrt(A[0][j] * A[0][j] + A[1][j] * A[1][j] + A[2][j] * A[2][j]);
    // sort columns by singular value, descending
    int order[3] = {0, 1, 2};
    for (int a = 0; a < 3; ++a)
        for (int b = a + 1; b < 3; ++b)
            if (s[order[b]] > s[order[a]]) {
                const int tmp = order[a];
                order[a] = order[b];
                order[b] = tmp;
            }
    double s2[3], A2[3][3], V2[3][3];
    for (int j = 0; j < 3; ++j) {
        s2[j] = s[order[j]];
        for (int i = 0; i < 3; ++i) {
            A2[i][j] = A[i][order[j]];
            V2[i][j] = V[i][order[j]];
        }
    }
    for (int j = 0; j < 3; ++j) {
        s[j] = s2[j];
        for (int i = 0; i < 3; ++i) {
            V[i][j] = V2[i][j];
            U[i][j] = s2[j] > 0 ? A2[i][j] / s2[j] : 0.0;
        }
    }
}

}  // namespace

kdnn_status procrustes_from_sums(const kdnn_icp_sums &S, double R[9], double t[3], std::string &err)
{
    if (S.n < 3) {
        err = "procrustes: fewer than 3 pairs";
        return KDNN_EDEGENERATE;
    }
    const double n = double(S.n);
    double ms[3], mm[3], H[3][3];
    for (int a = 0; a < 3; ++a) {
        ms[a] = S.sum_s[a] / n;
        mm[a] = S.sum_m[a] / n;
    }
    for (int a = 0; a < 3; ++a)
        for (int b = 0; b < 3; ++b) H[a][b] = S.sum_sm[3 * a + b] - S.sum_s[a] * S.sum_m[b] / n;
    double U[3][3], V[3][3], sv[3];
    jacobi_svd3(H, U, sv, V);
    if (!(sv[0] > 0.0) || !std::isfinite(sv[0]) || sv[1] <= 1e-12 * sv[0]) {
        err = "procrustes: cross-covariance of rank < 2, rotation undetermined";
        return KDNN_EDEGENERATE;
    }
    if (sv[2] <= 1e-12 * sv[0]) {
        // rank 2 (e.g. planar pairs): complete U with u3 = u1 x u2
        U[0][2] = U[1][0] * U[2][1] - U[2][0] * U[1][1];
        U[1][2] = U[2][0] * U[0][1] - U[0][0] * U[2][1];
        U[2][2] = U[0][0] * U[1][1] - U[1][0] * U[0][1];
    }
    const double d = (det3(U) * det3(V)) < 0 ? -1.0 : 1.0;
    // R = V diag(1, 1, d) U^T
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j)
            R[3 * i + j] = V[i][0] * U[j][0] + V[i][1] * U[j][1] + d * V[i][2] * U[j][2];
    double mus[3], mum[3];
    for (int a = 0; a < 3; ++a) {
        mus[a] = S.c[a] + ms[a];
        mum[a] = S.c[a] + mm[a];
    }
    for (int i = 0; i < 3; ++i)
        t[i] = mum[i] - (R[3 * i] * mus[0] + R[3 * i + 1] * mus[1] + R[3 * i + 2] * mus[2]);
    return KDNN_OK;
}

}  // namespace kdnn
