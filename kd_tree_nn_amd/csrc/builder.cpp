// Host KD-tree builder (CUDA-KDTree ICP article, §2.2 and §4.1-§4.2: median
// split on the max-variance axis, leaves of 8-16 points; §2.3: built once on
// the CPU; §3.1: linearised array, parent before child; §5.1: all storage
// reserved up front, in-place std::nth_element; §5.2: optional depth cap).
//
// The tree is complete: every node above depth D is split at a median, so
// the node array is an implicit heap and every leaf sits at depth D.  Node a
// of depth d (a = 0 .. 2^d - 1 from the left) owns the point slots
// [floor(a n / 2^d), floor((a + 1) n / 2^d)) and splits them at
// floor((2a + 1) n / 2^(d+1)), which is the lower or the upper median of its
// points.  Hence leaf j owns [floor(j n / 2^D), floor((j + 1) n / 2^D)):
// floor(n / 2^D) or ceil(n / 2^D) points, and a point range is a function
// of the leaf index alone.  Split values are actual point coordinates: left
// points have coordinate <= split <= right points.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <numeric>
#include <thread>

#include "kdnn_internal.hpp"

namespace kdnn {

static int32_t depth_for(int64_t n, int32_t leaf)
{
    int32_t d = 0;
    while (((n + (int64_t(1) << d) - 1) >> d) > leaf) ++d;  // ceil(n / 2^d) > leaf
    return d;
}

kdnn_status tree_layout(int64_t n, const kdnn_build_params *p, int32_t *depth, int64_t *slots,
                        std::string &err)
{
    kdnn_build_params d{16, 0, 0};
    if (p) d = *p;
    if (d.leaf_size == 0) d.leaf_size = 16;
    if (n < 1 || n >= (int64_t(1) << 31)) {
        err = "kdtree: n must be in [1, 2^31)";
        return KDNN_EINVAL;
    }
    if (d.leaf_size < 1 || d.leaf_size > kMaxLeafSize) {
        err = "kdtree: leaf_size must be in [1, 1024]";
        return KDNN_EINVAL;
    }
    if (d.max_depth < 0 || d.max_depth > kMaxDepth) {
        err = "kdtree: max_depth must be in [0, 28]";
        return KDNN_EINVAL;
    }
    if (d.flags & ~KDNN_BUILD_ROUND_ROBIN) {
        err = "kdtree: unknown build flag";
        return KDNN_EINVAL;
    }
    int32_t D = depth_for(n, d.leaf_size);
    if (d.max_depth > 0) D = std::min(D, d.max_depth);
    if (D > kMaxDepth) {
        err = "kdtree: depth above 28 (n / leaf_size too large)";
        return KDNN_EINVAL;
    }
    *depth = D;
    *slots = int64_t(1) << (D + 1);
    return KDNN_OK;
}

namespace {

struct Builder {
    const float *P;
    int64_t n;
    int32_t D;
    bool round_robin;
    std::vector<int32_t> perm;
    std::vector<int64_t> lo, hi;  // point range of each heap node
    std::vector<float> *nodes;

    int pick_axis(int64_t a, int64_t b, int depth) const
    {
        if (round_robin) return depth % 3;
        const int64_t cnt = b - a;
        if (cnt < 2) return 0;
        double mean[3] = {0, 0, 0};
        for (int64_t k = a; k < b; ++k)
            for (int ax = 0; ax < 3; ++ax) mean[ax] += P[3 * int64_t(perm[k]) + ax];
        for (int ax = 0; ax < 3; ++ax) mean[ax] /= double(cnt);
        double var[3] = {0, 0, 0};
        for (int64_t k = a; k < b; ++k)
            for (int ax = 0; ax < 3; ++ax) {
                const double v = P[3 * int64_t(perm[k]) + ax] - mean[ax];
                var[ax] += v * v;
            }
        int best = 0;  // ties go to the lowest axis
        for (int ax = 1; ax < 3; ++ax)
            if (var[ax] > var[best]) best = ax;
        return best;
    }

    void split_node(int64_t i, int depth)
    {
        const int64_t a = lo[i], b = hi[i];
        const int axis = pick_axis(a, b, depth);
        const int64_t idx_in_level = i - (int64_t(1) << depth);
        const int64_t mid = ((2 * idx_in_level + 1) * n) >> (depth + 1);
        // An empty right child (possible only when the node holds one point)
        // gets split = +inf: every finite query then takes the left side.
        float split = mid < b ? 0.0f : INFINITY;
        if (mid < b) {
            const float *Pp = P;
            auto less = [Pp, axis](int32_t u, int32_t v) {
                const float x = Pp[3 * int64_t(u) + axis], y = Pp[3 * int64_t(v) + axis];
                return x < y || (x == y && u < v);
            };
            std::nth_element(perm.begin() + a, perm.begin() + mid, perm.begin() + b, less);
            split = P[3 * int64_t(perm[mid]) + axis];
        }
        float *w = nodes->data() + i * kNodeWords;
        w[6] = split;
        uint32_t ax32 = uint32_t(axis);
        std::memcpy(&w[7], &ax32, 4);
        lo[2 * i] = a;
        hi[2 * i] = mid;
        lo[2 * i + 1] = mid;
        hi[2 * i + 1] = b;
    }
};

}  // namespace

kdnn_status build_host_tree(const float *xyz, int64_t n, const kdnn_build_params *p, HostTree &out,
                            std::string &err)
{
    int32_t D = 0;
    int64_t slots = 0;
    kdnn_status st = tree_layout(n, p, &D, &slots, err);
    if (st != KDNN_OK) return st;
    if (!xyz) {
        err = "kdtree: null point pointer";
        return KDNN_EINVAL;
    }
    for (int64_t k = 0; k < 3 * n; ++k)
        if (!std::isfinite(xyz[k])) {
            err = "kdtree: non-finite target coordinate at point " + std::to_string(k / 3);
            return KDNN_ENONFINITE;
        }

    out.depth = D;
    out.leaf_size = (p && p->leaf_size) ? p->leaf_size : 16;
    out.n = n;
    try {
        out.nodes.assign(size_t(slots) * kNodeWords, 0.0f);
        out.points.assign(size_t(n) * 4, 0.0f);
    } catch (...) {
        err = "kdtree: host allocation failed";
        return KDNN_ENOMEM;
    }

    Builder b;
    b.P = xyz;
    b.n = n;
    b.D = D;
    b.round_robin = p && (p->flags & KDNN_BUILD_ROUND_ROBIN);
    b.nodes = &out.nodes;
    b.perm.resize(size_t(n));
    std::iota(b.perm.begin(), b.perm.end(), 0);
    b.lo.assign(size_t(slots), 0);
    b.hi.assign(size_t(slots), 0);
    b.lo[1] = 0;
    b.hi[1] = n;

    // Level by level.  Nodes of one level own disjoint ranges of perm, so a
    // wide level is split across threads; results do not depend on that.
    const unsigned hw = std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
    for (int32_t d = 0; d < D; ++d) {
        const int64_t first = int64_t(1) << d, count = first;
        const int64_t per_node = n / count;
        const unsigned nt = (per_node * count >= 200000 && count >= 8) ? hw : 1u;
        if (nt <= 1) {
            for (int64_t i = first; i < first + count; ++i) b.split_node(i, d);
        } else {
            std::vector<std::thread> th;
            for (unsigned w = 0; w < nt; ++w)
                th.emplace_back([&, w] {
                    for (int64_t i = first + w; i < first + count; i += nt) b.split_node(i, d);
                });
            for (auto &x : th) x.join();
        }
    }

    // Leaves: point range and tight boxes; points written in leaf order.
    const int64_t L0 = int64_t(1) << D;
    int32_t mn = INT32_MAX, mx = 0;
    for (int64_t i = L0; i < 2 * L0; ++i) {
        float *w = out.nodes.data() + i * kNodeWords;
        const int64_t a = b.lo[i], e = b.hi[i];
        float lo3[3] = {INFINITY, INFINITY, INFINITY}, hi3[3] = {-INFINITY, -INFINITY, -INFINITY};
        for (int64_t k = a; k < e; ++k) {
            const int32_t j = b.perm[size_t(k)];
            float *q = out.points.data() + 4 * k;
            for (int ax = 0; ax < 3; ++ax) {
                const float v = xyz[3 * int64_t(j) + ax];
                q[ax] = v;
                lo3[ax] = std::min(lo3[ax], v);
                hi3[ax] = std::max(hi3[ax], v);
            }
            std::memcpy(&q[3], &j, 4);
        }
        w[0] = lo3[0]; w[1] = lo3[1]; w[2] = lo3[2];
        w[3] = hi3[0]; w[4] = hi3[1]; w[5] = hi3[2];
        const int32_t begin = int32_t(a), cnt = int32_t(e - a);
        std::memcpy(&w[6], &begin, 4);
        std::memcpy(&w[7], &cnt, 4);
        mn = std::min(mn, cnt);
        mx = std::max(mx, cnt);
    }
    // Internal boxes bottom-up (the union of the children's boxes).
    for (int64_t i = L0 - 1; i >= 1; --i) {
        float *w = out.nodes.data() + i * kNodeWords;
        const float *l = out.nodes.data() + 2 * i * kNodeWords;
        const float *r = out.nodes.data() + (2 * i + 1) * kNodeWords;
        for (int ax = 0; ax < 3; ++ax) {
            w[ax] = std::min(l[ax], r[ax]);
            w[3 + ax] = std::max(l[3 + ax], r[3 + ax]);
        }
    }
    const float *root = out.nodes.data() + kNodeWords;
    for (int ax = 0; ax < 3; ++ax) {
        out.bbox_min[ax] = root[ax];
        out.bbox_max[ax] = root[3 + ax];
        out.center[ax] = 0.5 * (double(root[ax]) + double(root[3 + ax]));
    }
    out.min_leaf = mn;
    out.max_leaf = mx;
    return KDNN_OK;
}

}  // namespace kdnn
