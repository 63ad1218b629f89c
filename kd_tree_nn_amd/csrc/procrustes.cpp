// Host rigid solve (CUDA-KDTree ICP article, §2.1): centroids, the 3x3
// cross-covariance H, the rotation that best maps the centred source points
// onto their centred matches, t from the centroids.  The rotation comes from
// the SVD of H with the det sign fix (rigid_solve.hpp), as the article solves
// it on the CPU; the device-side ICP loop reaches the same rotation through
// Horn's quaternion form.
#include "kdnn_internal.hpp"
#include "rigid_solve.hpp"

namespace kdnn {

const char *rigid_status_text(int32_t st)
{
    switch (st) {
    case kRigidFewPairs: return "procrustes: fewer than 3 pairs";
    case kRigidRankLow: return "procrustes: cross-covariance of rank < 2, rotation undetermined";
    default: return "procrustes: ok";
    }
}

kdnn_status procrustes_from_sums(const kdnn_icp_sums &S, double R[9], double t[3], std::string &err)
{
    double Rn[9], tn[3];
    const int32_t st =
        rigid_from_sums(S.sum_s, S.sum_m, S.sum_sm, double(S.n), S.c, Rn, tn, kRigidSvd);
    if (st != kRigidOk) {
        err = rigid_status_text(st);
        return KDNN_EDEGENERATE;
    }
    for (int k = 0; k < 9; ++k) R[k] = Rn[k];
    for (int k = 0; k < 3; ++k) t[k] = tn[k];
    return KDNN_OK;
}

void moments_of_sums(const kdnn_icp_sums &S, kdnn_icp_moments &M)
{
    M = kdnn_icp_moments{};
    M.n = S.n;
    M.E = S.sum_d2;
    if (S.n <= 0) return;
    moments_from_sums(S.sum_s, S.sum_m, S.sum_sm, double(S.n), S.c, M.mu_s, M.mu_m, M.H);
    M.mse = S.sum_d2 / double(S.n);
}

}  // namespace kdnn
