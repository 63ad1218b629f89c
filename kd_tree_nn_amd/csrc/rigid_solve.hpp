// Rigid solve of one ICP step from the shifted correspondence sums
// (CUDA-KDTree ICP article, §2.1: the rotation that best maps the centred
// source points onto their centred matches, then the translation between the
// centroids).  Compiled for the host (kdnn_procrustes, the host-driven loops)
// and for the device (the loop that keeps every ICP iteration on the GPU).
// The host takes the article's route: the 3x3 SVD of H with the det sign fix
// (rigid_rotation_svd).  One GPU lane takes the quaternion form below, which
// reaches the same rotation with far fewer dependent operations.
//
// Method on the device: Horn's closed form with unit quaternions (B. K. P. Horn, "Closed-form
// solution of absolute orientation using unit quaternions", JOSA A 4(4), 1987):
// the optimal rotation is the quaternion of the largest eigenvalue of a
// symmetric, trace-free 4x4 matrix N built from the cross-covariance H.  A
// proper rotation comes out by construction, so the reflection case of the
// SVD form needs no sign fix.  On one GPU lane an iterative eigensolver or a
// Jacobi SVD costs microseconds of dependent fp64 operations; here instead
//   * the largest eigenvalue is the largest root of the characteristic
//     polynomial x^4 + c2 x^2 + c1 x + c0 of N, with c2 = -2 |H|_F^2,
//     c1 = -8 det H, c0 = det N (the quaternion characteristic polynomial of
//     D. L. Theobald, Acta Cryst. A61, 2005), found by Newton's method from
//     sqrt(3) |H|_F, an upper bound of it (it is the sum of the singular
//     values of H, up to the sign of the smallest), where Newton descends
//     monotonically onto the largest root of a polynomial whose roots are
//     all real;
//   * the eigenvector is a column of the adjugate of N - x I, which for a
//     simple eigenvalue x has rank one and spans it: the column with the
//     largest diagonal entry.
// When the two largest eigenvalues are close (sigma2 ~ sigma3 with det H < 0,
// H nearly a reflection) the root and vector lose accuracy as the inverse
// square of the gap; there the solve takes the article's SVD route instead
// (one-sided Jacobi, slower but accurate to the problem's own conditioning).
// Degenerate (an error): fewer than 3 pairs; rank(H) < 2, tested as
// |cof H|_F <= 1e-12 |H|_F^2 (about sigma2 <= 1e-12 sigma1: every 2x2 minor
// vanishes).
#pragma once

#include <cmath>
#include <cstdint>

#if defined(__HIP__)
#define KDNN_HD __host__ __device__
#else
#define KDNN_HD
#endif

namespace kdnn {

enum RigidStatus : int32_t {
    kRigidOk = 0,
    kRigidFewPairs = 1,   // fewer than 3 pairs
    kRigidRankLow = 2,    // rank(H) < 2 (or H zero / not finite)
};

// 2x2 minors of rows (0, 1) and (2, 3) of a row-major 4x4 matrix (Laplace
// expansion along the first two rows).
struct Minors4 {
    double s[6], c[6];
};

KDNN_HD inline Minors4 minors4(const double a[16])
{
    Minors4 m;
    m.s[0] = a[0] * a[5] - a[4] * a[1];
    m.s[1] = a[0] * a[6] - a[4] * a[2];
    m.s[2] = a[0] * a[7] - a[4] * a[3];
    m.s[3] = a[1] * a[6] - a[5] * a[2];
    m.s[4] = a[1] * a[7] - a[5] * a[3];
    m.s[5] = a[2] * a[7] - a[6] * a[3];
    m.c[5] = a[10] * a[15] - a[14] * a[11];
    m.c[4] = a[9] * a[15] - a[13] * a[11];
    m.c[3] = a[9] * a[14] - a[13] * a[10];
    m.c[2] = a[8] * a[15] - a[12] * a[11];
    m.c[1] = a[8] * a[14] - a[12] * a[10];
    m.c[0] = a[8] * a[13] - a[12] * a[9];
    return m;
}

KDNN_HD inline double det4(const Minors4 &m)
{
    return ((m.s[0] * m.c[5] - m.s[1] * m.c[4]) + (m.s[2] * m.c[3] + m.s[3] * m.c[2])) -
           (m.s[4] * m.c[1] - m.s[5] * m.c[0]);
}

// adj (row-major) of the 4x4 matrix a: adj a = det(a) a^-1.
KDNN_HD inline void adjugate4(const double a[16], const Minors4 &m, double adj[16])
{
    const double *s = m.s, *c = m.c;
    adj[0] = (a[5] * c[5] - a[6] * c[4]) + a[7] * c[3];
    adj[1] = (-a[1] * c[5] + a[2] * c[4]) - a[3] * c[3];
    adj[2] = (a[13] * s[5] - a[14] * s[4]) + a[15] * s[3];
    adj[3] = (-a[9] * s[5] + a[10] * s[4]) - a[11] * s[3];
    adj[4] = (-a[4] * c[5] + a[6] * c[2]) - a[7] * c[1];
    adj[5] = (a[0] * c[5] - a[2] * c[2]) + a[3] * c[1];
    adj[6] = (-a[12] * s[5] + a[14] * s[2]) - a[15] * s[1];
    adj[7] = (a[8] * s[5] - a[10] * s[2]) + a[11] * s[1];
    adj[8] = (a[4] * c[4] - a[5] * c[2]) + a[7] * c[0];
    adj[9] = (-a[0] * c[4] + a[1] * c[2]) - a[3] * c[0];
    adj[10] = (a[12] * s[4] - a[13] * s[2]) + a[15] * s[0];
    adj[11] = (-a[8] * s[4] + a[9] * s[2]) - a[11] * s[0];
    adj[12] = (-a[4] * c[3] + a[5] * c[1]) - a[6] * c[0];
    adj[13] = (a[0] * c[3] - a[1] * c[1]) + a[2] * c[0];
    adj[14] = (-a[12] * s[3] + a[13] * s[1]) - a[14] * s[0];
    adj[15] = (a[8] * s[3] - a[9] * s[1]) + a[10] * s[0];
}

// The column of adj(N - x I) (N symmetric 4x4) with the largest diagonal
// entry, into q; returns that entry's magnitude.  For a simple eigenvalue x
// of N, adj(N - x I) = prod_{j != i}(l_j - x) q q^T: every column is along
// its eigenvector, and the largest diagonal entry is >= prod / 4.
KDNN_HD inline double adj_column(const double N[16], double x, double q[4])
{
    double A[16], adj[16];
    for (int k = 0; k < 16; ++k) A[k] = N[k];
    for (int k = 0; k < 4; ++k) A[5 * k] -= x;
    adjugate4(A, minors4(A), adj);
    int j = 0;
    double best = std::fabs(adj[0]);
    for (int k = 1; k < 4; ++k) {
        const double d = std::fabs(adj[5 * k]);
        if (d > best) {
            best = d;
            j = k;
        }
    }
    for (int i = 0; i < 4; ++i) q[i] = adj[4 * i + j];
    return best;
}

// H = U diag(sv) V^T (3x3, row-major in and out), sv descending: one-sided
// Jacobi (Hestenes) in fp64 -- plane rotations V make the columns of H V
// mutually orthogonal, then H V = U diag(sv).  Columns of U for zero singular
// values are left zero.
KDNN_HD inline void jacobi_svd3(const double H[9], double U[9], double sv[3], double V[9])
{
    double A[9];
    for (int k = 0; k < 9; ++k) {
        A[k] = H[k];
        V[k] = (k % 4 == 0) ? 1.0 : 0.0;
    }
    for (int sweep = 0; sweep < 60; ++sweep) {
        double off = 0.0;
        for (int pq = 0; pq < 3; ++pq) {
            const int p = pq == 2 ? 1 : 0, q = pq == 0 ? 1 : 2;
            double alpha = 0.0, beta = 0.0, gamma = 0.0;
            for (int i = 0; i < 3; ++i) {
                alpha += A[3 * i + p] * A[3 * i + p];
                beta += A[3 * i + q] * A[3 * i + q];
                gamma += A[3 * i + p] * A[3 * i + q];
            }
            if (gamma == 0.0) continue;
            const double scale = std::sqrt(alpha * beta);
            if (scale == 0.0 || std::fabs(gamma) <= 1e-16 * scale) continue;
            off = std::fmax(off, std::fabs(gamma) / scale);
            const double zeta = (beta - alpha) / (2.0 * gamma);
            const double tt = (zeta >= 0 ? 1.0 : -1.0) / (std::fabs(zeta) + std::sqrt(1.0 + zeta * zeta));
            const double c = 1.0 / std::sqrt(1.0 + tt * tt), sn = c * tt;
            for (int i = 0; i < 3; ++i) {
                const double ap = A[3 * i + p], aq = A[3 * i + q];
                A[3 * i + p] = c * ap - sn * aq;
                A[3 * i + q] = sn * ap + c * aq;
                const double vp = V[3 * i + p], vq = V[3 * i + q];
                V[3 * i + p] = c * vp - sn * vq;
                V[3 * i + q] = sn * vp + c * vq;
            }
        }
        if (off < 1e-15) break;
    }
    double s[3];
    for (int j = 0; j < 3; ++j)
        s[j] = std::sqrt((A[j] * A[j] + A[3 + j] * A[3 + j]) + A[6 + j] * A[6 + j]);
    int o[3] = {0, 1, 2};  // columns by singular value, descending
    for (int a = 0; a < 3; ++a)
        for (int b = a + 1; b < 3; ++b)
            if (s[o[b]] > s[o[a]]) {
                const int tmp = o[a];
                o[a] = o[b];
                o[b] = tmp;
            }
    double V2[9];
    for (int j = 0; j < 3; ++j) {
        sv[j] = s[o[j]];
        for (int i = 0; i < 3; ++i) {
            V2[3 * i + j] = V[3 * i + o[j]];
            U[3 * i + j] = sv[j] > 0.0 ? A[3 * i + o[j]] / sv[j] : 0.0;
        }
    }
    for (int k = 0; k < 9; ++k) V[k] = V2[k];
}

KDNN_HD inline double det3(const double M[9])
{
    return (M[0] * (M[4] * M[8] - M[5] * M[7]) - M[1] * (M[3] * M[8] - M[5] * M[6])) +
           M[2] * (M[3] * M[7] - M[4] * M[6]);
}

// The SVD route of the article (§2.1): R = V diag(1, 1, d) U^T with
// d = sign det(V U^T), so that R is a proper rotation.
KDNN_HD inline int32_t rotation_by_svd(const double H[9], double R[9])
{
    double U[9], V[9], sv[3];
    jacobi_svd3(H, U, sv, V);
    if (!(sv[0] > 0.0) || !(sv[0] < INFINITY) || sv[1] <= 1e-12 * sv[0]) return kRigidRankLow;
    if (sv[2] <= 1e-12 * sv[0]) {  // rank 2 (planar pairs): u3 = u1 x u2
        U[2] = U[3] * U[7] - U[6] * U[4];
        U[5] = U[6] * U[1] - U[0] * U[7];
        U[8] = U[0] * U[4] - U[3] * U[1];
    }
    const double d = det3(U) * det3(V) < 0.0 ? -1.0 : 1.0;
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j)
            R[3 * i + j] = (V[3 * i] * U[3 * j] + V[3 * i + 1] * U[3 * j + 1]) + d * V[3 * i + 2] * U[3 * j + 2];
    return kRigidOk;
}

// The rotation R (row-major) minimising sum |R (s - mu_s) - (m - mu_m)|^2 for
// the cross-covariance H[3a + b] = sum (s - mu_s)_a (m - mu_m)_b.
KDNN_HD inline int32_t rigid_rotation(const double H[9], double R[9])
{
    // sums as balanced trees: short dependency chains on one GPU lane
    const double F = (((H[0] * H[0] + H[1] * H[1]) + (H[2] * H[2] + H[3] * H[3])) +
                      ((H[4] * H[4] + H[5] * H[5]) + (H[6] * H[6] + H[7] * H[7]))) +
                     H[8] * H[8];
    if (!(F > 0.0) || !(F < INFINITY)) return kRigidRankLow;
    // cofactors of H (the 2x2 minors, signed)
    const double C[9] = {H[4] * H[8] - H[5] * H[7], H[5] * H[6] - H[3] * H[8],
                         H[3] * H[7] - H[4] * H[6], H[2] * H[7] - H[1] * H[8],
                         H[0] * H[8] - H[2] * H[6], H[1] * H[6] - H[0] * H[7],
                         H[1] * H[5] - H[2] * H[4], H[2] * H[3] - H[0] * H[5],
                         H[0] * H[4] - H[1] * H[3]};
    const double K = (((C[0] * C[0] + C[1] * C[1]) + (C[2] * C[2] + C[3] * C[3])) +
                      ((C[4] * C[4] + C[5] * C[5]) + (C[6] * C[6] + C[7] * C[7]))) +
                     C[8] * C[8];
    if (!(K > 1e-24 * (F * F))) return kRigidRankLow;
    const double detH = (H[0] * C[0] + H[1] * C[1]) + H[2] * C[2];
    const double Sxx = H[0], Sxy = H[1], Sxz = H[2], Syx = H[3], Syy = H[4], Syz = H[5],
                 Szx = H[6], Szy = H[7], Szz = H[8];
    const double N[16] = {(Sxx + Syy) + Szz, Syz - Szy,         Szx - Sxz,          Sxy - Syx,
                          Syz - Szy,         (Sxx - Syy) - Szz, Sxy + Syx,          Szx + Sxz,
                          Szx - Sxz,         Sxy + Syx,         (Syy - Sxx) - Szz,  Syz + Szy,
                          Sxy - Syx,         Szx + Sxz,         Syz + Szy,          (Szz - Sxx) - Syy};
    const double c2 = -2.0 * F, c1 = -8.0 * detH, c0 = det4(minors4(N));
    // start: the smaller of two upper bounds of the largest eigenvalue,
    // sqrt(3) |H|_F and Gershgorin's max_i (N_ii + sum_j!=i |N_ij|) -- the
    // latter is within a fraction of a percent of it when the rotation is
    // small (N is then nearly diagonal in its first row), which saves about
    // half of the Newton steps
    double gersh = -INFINITY;
    for (int i = 0; i < 4; ++i) {
        const double r = N[5 * i] + ((std::fabs(N[4 * i + (i + 1) % 4]) +
                                      std::fabs(N[4 * i + (i + 2) % 4])) +
                                     std::fabs(N[4 * i + (i + 3) % 4]));
        gersh = r > gersh ? r : gersh;
    }
    const double root3F = std::sqrt(3.0 * F);
    double x = gersh < root3F ? gersh : root3F;
    for (int it = 0; it < 100; ++it) {
        const double x2 = x * x;
        const double p = ((x2 + c2) * x2 + c1 * x) + c0;
        const double dp = (4.0 * x2 + 2.0 * c2) * x + c1;
        if (!(dp > 0.0)) break;
        const double nx = x - p / dp;
        if (!(nx < x)) break;  // no further descent: converged to rounding
        x = nx;
    }
    double q[4];
    const double best = adj_column(N, x, q);
    // Close largest eigenvalues (sigma2 ~ sigma3 with det H < 0): the Newton
    // root's error, and with it the vector's, grows as the inverse square of
    // the gap, so take the SVD route there (rare in registration: H is then
    // nearly a reflection).
    if (!(best > 1e-2 * (F * std::sqrt(F)))) return rotation_by_svd(H, R);
    const double q0 = q[0], q1 = q[1], q2 = q[2], q3 = q[3];
    const double nq = ((q0 * q0 + q1 * q1) + q2 * q2) + q3 * q3;
    if (!(nq > 0.0) || !(nq < INFINITY)) return kRigidRankLow;
    const double inv = 1.0 / std::sqrt(nq);
    const double w = q0 * inv, qx = q1 * inv, qy = q2 * inv, qz = q3 * inv;
    R[0] = ((w * w + qx * qx) - qy * qy) - qz * qz;
    R[1] = 2.0 * (qx * qy - w * qz);
    R[2] = 2.0 * (qx * qz + w * qy);
    R[3] = 2.0 * (qy * qx + w * qz);
    R[4] = ((w * w - qx * qx) + qy * qy) - qz * qz;
    R[5] = 2.0 * (qy * qz - w * qx);
    R[6] = 2.0 * (qz * qx - w * qy);
    R[7] = 2.0 * (qz * qy + w * qx);
    R[8] = ((w * w - qx * qx) - qy * qy) + qz * qz;
    return kRigidOk;
}

// The same rotation by the article's SVD route for every H: H = U S V^T by
// one-sided Jacobi, R = V diag(1, 1, d) U^T with d = sign det(V U^T).  Same
// degeneracy test as rigid_rotation, so both report the same cases.
KDNN_HD inline int32_t rigid_rotation_svd(const double H[9], double R[9])
{
    double F = 0.0, K = 0.0;
    for (int k = 0; k < 9; ++k) F += H[k] * H[k];
    if (!(F > 0.0) || !(F < INFINITY)) return kRigidRankLow;
    const double C[9] = {H[4] * H[8] - H[5] * H[7], H[5] * H[6] - H[3] * H[8],
                         H[3] * H[7] - H[4] * H[6], H[2] * H[7] - H[1] * H[8],
                         H[0] * H[8] - H[2] * H[6], H[1] * H[6] - H[0] * H[7],
                         H[1] * H[5] - H[2] * H[4], H[2] * H[3] - H[0] * H[5],
                         H[0] * H[4] - H[1] * H[3]};
    for (int k = 0; k < 9; ++k) K += C[k] * C[k];
    if (!(K > 1e-24 * (F * F))) return kRigidRankLow;
    return rotation_by_svd(H, R);
}

// Centroids and cross-covariance from the sums shifted by c (article §2.1:
// centroids, then de-centred pairs, then H): with S_s = sum (s - c),
// S_m = sum (m - c), S_sm[3a + b] = sum (s - c)_a (m - c)_b over n > 0 pairs,
// mu_s = c + S_s / n, mu_m = c + S_m / n and
// H = sum (s - mu_s)(m - mu_m)^T = S_sm - (S_s / n) S_m^T (the shift cancels).
KDNN_HD inline void moments_from_sums(const double S_s[3], const double S_m[3],
                                      const double S_sm[9], double n, const double c[3],
                                      double mu_s[3], double mu_m[3], double H[9])
{
    const double inv_n = 1.0 / n;  // one division (each costs ~65 cycles on a GPU lane)
    double ms[3], mm[3];
    for (int a = 0; a < 3; ++a) {
        ms[a] = S_s[a] * inv_n;
        mm[a] = S_m[a] * inv_n;
    }
    for (int a = 0; a < 3; ++a)
        for (int b = 0; b < 3; ++b) H[3 * a + b] = S_sm[3 * a + b] - ms[a] * S_m[b];
    for (int a = 0; a < 3; ++a) {
        mu_s[a] = c[a] + ms[a];
        mu_m[a] = c[a] + mm[a];
    }
}

enum RigidMethod : int32_t {
    kRigidHorn = 0,  // quaternion form (one GPU lane: the device-side loop)
    kRigidSvd = 1,   // the article's SVD with the det sign fix (the host)
};

// (R, t) from the shifted sums: the rotation from H (by `method`), then
// t = mu_m - R mu_s.
KDNN_HD inline int32_t rigid_from_sums(const double S_s[3], const double S_m[3],
                                       const double S_sm[9], double n, const double c[3],
                                       double R[9], double t[3], int32_t method = kRigidHorn)
{
    if (!(n >= 3.0)) return kRigidFewPairs;
    double mus[3], mum[3], H[9];
    moments_from_sums(S_s, S_m, S_sm, n, c, mus, mum, H);
    const int32_t st = method == kRigidSvd ? rigid_rotation_svd(H, R) : rigid_rotation(H, R);
    if (st != kRigidOk) return st;
    for (int i = 0; i < 3; ++i)
        t[i] = mum[i] - ((R[3 * i] * mus[0] + R[3 * i + 1] * mus[1]) + R[3 * i + 2] * mus[2]);
    return kRigidOk;
}

}  // namespace kdnn
