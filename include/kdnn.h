/*
 * kdnn.h -- C ABI of libkdnn.so: exact 3-D nearest-neighbour search on a
 * CPU-built KD-tree and the ICP correspondence step, on one AMD Instinct
 * MI355X (gfx950).
 *
 * The method is the one described by the CUDA-KDTree ICP article
 * (pwwt.cn, "用 CUDA-KDTree 实现 ICP"; cited below as "the article" with its
 * section numbers):
 *   - ICP minimises E(R, t) = sum_i || R s_i + t - m_i ||^2 over rigid
 *     motions, where m_i is the target point nearest to the moved source
 *     point (§2.1);
 *   - each iteration moves the original source by the current (R, t), finds
 *     every nearest neighbour, and solves (R, t) from the centroids and the
 *     3x3 cross-covariance H (§2.1, §3.3);
 *   - the target gets a KD-tree built once on the CPU, linearised into an
 *     array and kept in device memory (§2.2, §2.3, §3.1).
 *
 * Conventions shared by every entry point
 *   - Point clouds are arrays of n points, 3 consecutive fp32 values each
 *     (x, y, z), C-contiguous, 4-byte aligned: the layout of a (n, 3) float32
 *     tensor.  Index arrays are int32 (n < 2^31).
 *   - R is a row-major 3x3 fp64 matrix, t a 3-vector of fp64; a point p is
 *     moved to R p + t.
 *   - "_dev" pointers are device memory of the current HIP device, "_host"
 *     pointers are host memory.  Every buffer is owned by the caller, except
 *     the memory held by a kdnn_tree (freed by kdtree_free).  No entry point
 *     allocates device memory except kdtree_build.
 *   - Nearest neighbour: the target point of least squared distance, the
 *     distance evaluated in fp32 as d = (dx*dx + dy*dy) + dz*dz with no fused
 *     multiply-add and no denormal flushing; ties go to the lowest target
 *     index (the index into the array given to kdtree_build).  A query with a
 *     NaN/Inf coordinate, or with every distance overflowing to +inf, gets
 *     (idx, dist2) = (-1, +inf).
 *   - Functions never throw and never abort.  On failure they return a
 *     non-zero kdnn_status and kdnn_last_error() describes it.  Device faults
 *     of asynchronous work surface as KDNN_EDEVICE from a later synchronising
 *     call.
 */
#ifndef KDNN_H
#define KDNN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDNN_VERSION 5  /* 4: kdnn_moments; icp_align solves on the host unless
                           KDNN_ICP_DEVICE_LOOP; kdnn_procrustes takes the SVD route.
                           5: kdnn_replay_bench */

typedef enum kdnn_status {
    KDNN_OK = 0,
    KDNN_EINVAL = 1,      /* bad argument (size, null pointer, small workspace) */
    KDNN_ENOMEM = 2,      /* host or device allocation failed (kdtree_build only) */
    KDNN_EDEVICE = 3,     /* a HIP call or kernel failed */
    KDNN_ENONFINITE = 4,  /* a target coordinate is NaN or Inf */
    KDNN_EDEGENERATE = 5  /* fewer than 3 pairs, or H of rank < 2: rotation undetermined */
} kdnn_status;

/* Opaque tree handle.  Immutable after kdtree_build; may be shared by
 * concurrent nn_query calls on different streams. */
typedef struct kdnn_tree kdnn_tree;

/* Build flags. */
#define KDNN_BUILD_ROUND_ROBIN 1u /* split axis cycles x, y, z (article §4.2) instead of max variance */

typedef struct kdnn_build_params {
    int32_t leaf_size; /* 1..1024; the article recommends 8..16 (§2.2, §4.1). 0 = 16 */
    int32_t max_depth; /* 0 = none; else the tree stops at this depth and its leaves
                          hold every remaining point (article §5.2) */
    uint32_t flags;    /* KDNN_BUILD_* */
} kdnn_build_params;

typedef struct kdnn_tree_info {
    int64_t n;              /* target points */
    int32_t depth;          /* D: every leaf sits at depth D (root = depth 0) */
    int32_t leaf_size;      /* requested leaf size */
    int64_t node_slots;     /* 2^(D+1): 32-byte node records in device memory */
    int64_t leaves;         /* 2^D */
    int32_t min_leaf;       /* fewest points in a leaf */
    int32_t max_leaf;       /* most points in a leaf */
    float bbox_min[3];      /* tight bounding box of the target */
    float bbox_max[3];
    double center[3];       /* bbox centre; the shift applied in kdnn_icp_sums */
    double build_ms;        /* host build time (excluding the upload) */
    double upload_ms;       /* device allocation + host-to-device copy */
    int64_t device_bytes;   /* device memory held by the tree (node records, child box
                               runs, points, slot map, 64-byte plane record per leaf) */
    int64_t l2_bytes;       /* L2 cache size of the tree's device */
    int32_t auto_sort;      /* 1: nn_query's automatic choice applies the Morton ordering */
    int32_t auto_sort_icp;  /* 1: the ICP entry points' automatic choice applies it */
} kdnn_tree_info;

/* Correspondence sums of one ICP iteration (article §2.1).  Over the pairs
 * (s_i, m_i) -- s_i an ORIGINAL source point, m_i its matched target point --
 * with a fixed shift c (the target's bbox centre, for fp64 conditioning):
 *   n      = number of pairs (source points whose query found a match)
 *   sum_s  = sum (s_i - c),  sum_m = sum (m_i - c)
 *   sum_sm = sum (s_i - c)(m_i - c)^T, row-major: sum_sm[3a + b] = sum (s-c)_a (m-c)_b
 *   sum_d2 = sum of the fp32 squared distances, i.e. E(R, t) at the (R, t) used.
 * Hence mu_s = c + sum_s/n, mu_m = c + sum_m/n and
 * H = sum (s - mu_s)(m - mu_m)^T = sum_sm - sum_s sum_m^T / n.  All fp64. */
typedef struct kdnn_icp_sums {
    int64_t n;
    double c[3];
    double sum_s[3];
    double sum_m[3];
    double sum_sm[9];
    double sum_d2;
} kdnn_icp_sums;

/* What the article's solve takes from one iteration's pairs (§2.1: the
 * centroids, the de-centred pairs' cross-covariance H, and the error E). */
typedef struct kdnn_icp_moments {
    int64_t n;        /* pairs */
    double mu_s[3];   /* source centroid  c + sum_s / n */
    double mu_m[3];   /* matched-target centroid  c + sum_m / n */
    double H[9];      /* sum (s - mu_s)(m - mu_m)^T = sum_sm - sum_s sum_m^T / n, row-major */
    double E;         /* sum of squared distances (sum_d2) */
    double mse;       /* E / n */
} kdnn_icp_moments;

/* Number of doubles icp_correspond_reduce_async writes to sums_dev:
 * [0..2] sum_s, [3..5] sum_m, [6..14] sum_sm, [15] sum_d2, [16] n. */
#define KDNN_SUMS_DOUBLES 17

/* ---------------------------------------------------------------- build */

/* Build the KD-tree of a target cloud on the host and upload it (article
 * §2.2: median split on the max-variance axis, leaves of leaf_size points;
 * §2.3: built once on the CPU, linearised, copied to device memory once;
 * §3.1: nodes in one array, parent before child; §5.1: storage reserved up
 * front, in-place nth_element).
 *   xyz_host : n x 3 fp32, host memory, read only during the call.
 *   params   : NULL = defaults (leaf 16, no depth cap, max-variance axis).
 *   out      : receives the handle; unchanged on failure.
 * Every node above depth D = min{d : ceil(n / 2^d) <= leaf_size} (or
 * max_depth) is split, so all leaves sit at depth D.  Node a of depth d owns
 * the leaf-order slots [floor(a n / 2^d), floor((a+1) n / 2^d)) and splits at
 * slot floor((2a+1) n / 2^(d+1)), a median of its range; leaves hold
 * floor(n/2^D) or ceil(n/2^D) points.
 * Errors: EINVAL (n < 1, n >= 2^31, leaf_size or max_depth out of range,
 * NULL pointers, D > 28), ENONFINITE (NaN/Inf coordinate), ENOMEM, EDEVICE. */
kdnn_status kdtree_build(const float *xyz_host, int64_t n, const kdnn_build_params *params,
                         kdnn_tree **out);

/* Release a tree and its device memory.  NULL is a no-op.  The caller must
 * make sure no work using the tree is still queued. */
void kdtree_free(kdnn_tree *tree);

/* Describe a tree.  Errors: EINVAL on NULL pointers. */
kdnn_status kdtree_info(const kdnn_tree *tree, kdnn_tree_info *out);

/* Host-only build for inspection (no device, no HIP call).  Sizes first:
 * kdtree_layout gives D and the node slot count; kdtree_build_host fills
 *   nodes_out  : node_slots x 8 fp32 words (32-byte records, slot i = heap
 *                node i, root = 1, children 2i and 2i+1, slot 0 unused):
 *                [lo.x lo.y lo.z hi.x hi.y hi.z w6 w7]; internal node: w6 =
 *                split value, w7 = axis (uint32 0/1/2); leaf (i >= 2^D):
 *                w6 = first point slot (int32), w7 = point count (int32).
 *   points_out : n x 4 fp32 words, points in leaf order: x, y, z and the
 *                original index (int32 bit pattern).
 * Same errors as kdtree_build (without ENOMEM/EDEVICE for the device). */
kdnn_status kdtree_layout(int64_t n, const kdnn_build_params *params, int32_t *depth_out,
                          int64_t *node_slots_out);
kdnn_status kdtree_build_host(const float *xyz_host, int64_t n, const kdnn_build_params *params,
                              float *nodes_out, float *points_out);

/* ---------------------------------------------------------------- query */

/* Query flags. */
#define KDNN_QUERY_NO_SORT 1u /* traverse in the given order (skip the Morton ordering) */
#define KDNN_QUERY_SORT 2u    /* always apply the Morton ordering (needs ws_dev) */
/* Neither: the Morton ordering is applied when a workspace is given and the
 * tree's node records and points take more than 4 times the device's L2
 * cache (kdnn_tree_info.auto_sort).  The ordering costs a sort on every
 * call, and the search gains L2 locality from it only for trees well beyond
 * the L2.  The ordering key is the top 8 bits of the queries' 30-bit Morton
 * code in the tree's bounding box (one radix pass; the ICP entry points,
 * which sort once per registration, take 16).  Results never depend on the
 * order. */

/* Search schedule (nn_query, nn_query_stats and the ICP entry points).
 * Default: one lane owns each query, and the 64 lanes of a wavefront share
 * the work (lanes that finish take over pending subtrees of busy ones).
 *   KDNN_LANES(g), g in {2, 4, 8, 16}: g lanes cooperate on each query (g = 1
 *                   is the default).
 *   KDNN_BUDGET(b), b in 1..255: two passes -- one lane
 *                   per query with a budget of b node visits, then groups of
 *                   16 lanes complete the queries left over, starting from
 *                   the first pass's best (nn_query: needs ws_dev).
 *   KDNN_TOP_LDS:   one lane per query, one work-group per CU, with the top
 *                   (up to 12) tree levels copied into LDS first.
 * At most one of the three may be given (else EINVAL).  Results never depend
 * on the schedule. */
#define KDNN_LANES_SHIFT 8
#define KDNN_LANES_MASK (0x1fu << KDNN_LANES_SHIFT)
#define KDNN_LANES(g) ((uint32_t)(g) << KDNN_LANES_SHIFT)
#define KDNN_BUDGET_SHIFT 16
#define KDNN_BUDGET_MASK (0xffu << KDNN_BUDGET_SHIFT)
#define KDNN_BUDGET(b) ((uint32_t)(b) << KDNN_BUDGET_SHIFT)
#define KDNN_TOP_LDS (1u << 24)

/* Bytes of device workspace nn_query needs for m queries (Morton keys,
 * permutation, radix-sort histograms, two-pass list). 0 for m <= 0. */
size_t nn_query_workspace_bytes(int64_t m);

/* Exact nearest neighbour of every query (article §2.2 search with
 * backtracking and split-plane pruning; §3.2 one query per GPU lane;
 * §5.3 queries Morton-ordered so that neighbouring lanes walk the same
 * branches).  Each search first locates the leaf whose cell holds its query
 * by the ancestors' split planes (the top 8 levels' from a copy each
 * work-group keeps in LDS), scans it, and then visits the rest of the
 * tree as far as the best distance requires: the subtrees beside that leaf's
 * path are bounded along their parents' split axes (the leaf's plane record), nodes
 * below them by their boxes.
 *   q_dev      : m x 3 fp32 queries (device).
 *   idx_dev    : m int32 out, original target index of each nearest point.
 *   dist2_dev  : m fp32 out, its squared distance.
 *   flags      : KDNN_QUERY_* and the schedule flags.
 *   ws_dev     : >= nn_query_workspace_bytes(m) bytes of device memory,
 *                256-byte aligned, or NULL (then no Morton ordering and no
 *                two-pass schedule; KDNN_QUERY_SORT with NULL is EINVAL).
 *   stream     : HIP stream (NULL = default stream).  Asynchronous.
 * Results are written in the queries' own order whatever the traversal
 * order.  m == 0 is a no-op.  Errors: EINVAL, EDEVICE (launch failure). */
kdnn_status nn_query(const kdnn_tree *tree, const float *q_dev, int64_t m, int32_t *idx_dev,
                     float *dist2_dev, uint32_t flags, void *ws_dev, size_t ws_bytes,
                     hipStream_t stream);

/* nn_query restricted to target points within max_dist (article §4.4: the
 * distance threshold applied at correspondence time, fused into the search,
 * where it also serves as the initial pruning bound).  The result is the
 * lowest-index nearest point among those whose fp32 squared distance is
 * <= fl32(max_dist * max_dist) (product in fp64, one rounding), else
 * (idx -1, dist2 +inf).  max_dist <= 0 or +inf: no bound (as nn_query).
 * Arguments and errors as nn_query; EINVAL also for a NaN max_dist. */
kdnn_status nn_query_radius(const kdnn_tree *tree, const float *q_dev, int64_t m, double max_dist,
                            int32_t *idx_dev, float *dist2_dev, uint32_t flags, void *ws_dev,
                            size_t ws_bytes, hipStream_t stream);

/* Instrumented nn_query: same results, and per query the number of tree node
 * records loaded and of leaf points scanned (uint32 each, may be NULL).  Node
 * records: one per split plane the point location reads from memory (D - 8
 * when D > 8: the top 8 levels' planes come from the work-group's LDS copy
 * and count none), two for the
 * start leaf's 64-byte plane record, one per sibling box above that record's
 * 14 levels (D - 14 when D > 14), two per child-pair run.  With
 * the default schedule the counts are those of the exact single-lane search
 * of that query (lanes do not share work in this mode, so the counts do not
 * depend on which queries share a wavefront; the balanced search of nn_query
 * loads these plus the extra visits of subtrees handed over).  With
 * KDNN_LANES / KDNN_BUDGET / KDNN_TOP_LDS: the counts of that schedule's
 * traversal.  For measurement only; slower than nn_query. */
kdnn_status nn_query_stats(const kdnn_tree *tree, const float *q_dev, int64_t m, int32_t *idx_dev,
                           float *dist2_dev, uint32_t *nodes_dev, uint32_t *points_dev,
                           uint32_t flags, void *ws_dev, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------ transform */

/* out_i = fl32( ((R_r0 x + R_r1 y) + R_r2 z) + t_r ) per row r, evaluated in
 * fp64 in exactly that order with one round-to-nearest-even cast (article
 * §3.3, step 1 of the main loop).  in_dev == out_dev is allowed (in place);
 * partial overlap is not.  R_host, t_host are read during the call.
 * Asynchronous on stream.  n == 0 is a no-op.  Errors: EINVAL, EDEVICE. */
kdnn_status transform_points(const float *in_dev, float *out_dev, int64_t n, const double *R_host,
                             const double *t_host, hipStream_t stream);

/* ------------------------------------------------------------------ ICP */

/* ICP flags. */
#define KDNN_ICP_REUSE_ORDER 1u /* ws was last used by an ICP call with the same src_dev, n
                                   and ordering choice, stream-ordered before this one: reuse
                                   its traversal order instead of sorting again */
#define KDNN_ICP_NO_SORT 2u     /* traverse source points in their given order */
#define KDNN_ICP_SORT 4u        /* always traverse in Morton order of the transformed points */
#define KDNN_ICP_HOST_LOOP 8u   /* icp_align, icp_align_batch: each iteration's sums come
                                   back to the host, which solves (SVD) and applies the
                                   convergence rule; icp_align's default */
#define KDNN_ICP_DEVICE_LOOP 16u /* icp_align, icp_align_batch: the iterations stay on the
                                    device (a one-group kernel reduces, solves and applies
                                    the convergence rule); icp_align_batch's default */
/* Neither NO_SORT nor SORT: Morton order when the tree's node records and
 * points exceed the device's L2 cache (kdnn_tree_info.auto_sort_icp); the
 * order is computed once per registration. */

/* Correspondence rejection (article §4.4, both ways combined).
 *   max_dist : finite and > 0: a pair takes part only if its fp32 squared
 *              distance is <= fl32(max_dist * max_dist); the search itself is
 *              bounded by it (as nn_query_radius).  Otherwise no threshold.
 *   reject_k : > 0: after the rigid solve (R1, t1) of an iteration, residuals
 *              r_i^2 = ||R1 s_i + t1 - m_i||^2 are taken in fp64 over the
 *              pairs (the moved point not rounded), sigma^2 = mean r_i^2, and
 *              only pairs with r_i^2 <= (k k) sigma^2 enter a second solve
 *              (k = 3: the 3-sigma rule).  0: off.  Must be finite, >= 0.
 * A NULL pointer means neither. */
typedef struct {
    double max_dist;
    double reject_k;
} kdnn_icp_reject;

/* Bytes of device workspace the ICP entry points need for n source points
 * (traversal order, partial sums, rejection state, device-loop state, and
 * each source point's match leaf for icp_align's next iteration). */
size_t icp_workspace_bytes(int64_t n);

/* One ICP correspondence step fused into one kernel (article §2.1, §3.3):
 * move every ORIGINAL source point by (R, t) exactly as transform_points
 * does, find its nearest target point, and reduce the pairs to the sums of
 * kdnn_icp_sums (fp64 accumulation, deterministic order).  The article
 * copies the per-point results back and reduces on the CPU; here only the
 * 17 sums cross to the host.
 *   src_dev    : n x 3 fp32 original source points (device).
 *   R_host, t_host : current transform (host, read during the call).
 *   out_host   : receives the sums.
 *   idx_dev, dist2_dev : optional per-point correspondences (NULL = skip).
 *   reject     : optional; max_dist drops far pairs (idx -1 in idx_dev).  With
 *                reject_k > 0 the matches are also kept in ws for a following
 *                icp_reject_reduce.
 *   ws_dev     : >= icp_workspace_bytes(n) bytes, 256-byte aligned.
 * Synchronises stream.  Calls sharing one ws must not overlap.
 * Errors: EINVAL, EDEVICE. */
kdnn_status icp_correspond_reduce(const kdnn_tree *tree, const float *src_dev, int64_t n,
                                  const double *R_host, const double *t_host,
                                  kdnn_icp_sums *out_host, int32_t *idx_dev, float *dist2_dev,
                                  uint32_t flags, const kdnn_icp_reject *reject, void *ws_dev,
                                  size_t ws_bytes, hipStream_t stream);

/* As icp_correspond_reduce but asynchronous: the KDNN_SUMS_DOUBLES sums are
 * written to sums_dev (device, 8-byte aligned) when the stream reaches the
 * kernel.  For pipelining several registrations and for timing the kernel. */
kdnn_status icp_correspond_reduce_async(const kdnn_tree *tree, const float *src_dev, int64_t n,
                                        const double *R_host, const double *t_host,
                                        double *sums_dev, int32_t *idx_dev, float *dist2_dev,
                                        uint32_t flags, const kdnn_icp_reject *reject,
                                        void *ws_dev, size_t ws_bytes, hipStream_t stream);

/* The residual rejection step of kdnn_icp_reject.reject_k (article §4.4,
 * second way; 3-sigma rule for reject_k = 3) on the matches that the last
 * icp_correspond_reduce(_async) call with reject_k > 0 kept in ws (same src,
 * n, stream-ordered before this call): residuals under (R_host, t_host) --
 * normally the solve of that call's sums -- then the sums of the pairs with
 * r_i^2 <= (reject_k^2) * mean r_i^2.  sum_d2 is the kept pairs' match
 * distances.
 *   out_host   : the kept pairs' sums.   sigma2_out : optional, mean r_i^2.
 *   kept_dev   : optional n uint8 out, 1 where the pair is kept.
 * A ws without such matches gives unspecified sums (the stored slots are
 * bounds-checked, so it is safe).  Synchronises stream.
 * Errors: EINVAL (also reject_k <= 0 or non-finite), EDEVICE. */
kdnn_status icp_reject_reduce(const kdnn_tree *tree, const float *src_dev, int64_t n,
                              const double *R_host, const double *t_host, double reject_k,
                              kdnn_icp_sums *out_host, double *sigma2_out, uint8_t *kept_dev,
                              void *ws_dev, size_t ws_bytes, hipStream_t stream);

/* Centroids, cross-covariance and error of one iteration's pairs from their
 * shifted sums (article §2.1: the centroids, then H over the de-centred
 * pairs, which the SVD of the solve takes).  Host, fp64:
 *   mu_s = c + sum_s / n,  mu_m = c + sum_m / n,
 *   H = sum_sm - sum_s sum_m^T / n  (= sum (s - mu_s)(m - mu_m)^T),
 *   E = sum_d2,  mse = E / n.
 * n <= 0: out->n = n, E copied, every other field zero.
 * Errors: EINVAL (NULL pointer). */
kdnn_status kdnn_moments(const kdnn_icp_sums *sums, kdnn_icp_moments *out);

/* Rigid solve from correspondence sums (article §2.1): centroids and H as
 * kdnn_moments gives them, the SVD H = U S V^T (one-sided Jacobi, fp64),
 * the proper rotation R = V diag(1, 1, d) U^T with d = sign det(V U^T) --
 * the rotation minimising sum |R (s - mu_s) - (m - mu_m)|^2 -- then
 * t = mu_m - R mu_s.  Host.  (The device-side ICP loop reaches the same
 * rotation through Horn's unit-quaternion form.)
 * Errors: EINVAL (NULL), EDEGENERATE (n < 3 or rank(H) < 2; outputs unset). */
kdnn_status kdnn_procrustes(const kdnn_icp_sums *sums, double *R_out, double *t_out);

/* Whole ICP registration (article §2.1 loop, §3.3 main loop, §4.6
 * convergence rule): from (R0, t0) (NULL = identity / zero), repeat
 *   sums_k = correspond-and-reduce at (R_k, t_k);  E_k = sums_k.sum_d2;
 *   (R_{k+1}, t_{k+1}) = kdnn_procrustes(sums_k)
 * for max_iter iterations, or stop early once eps > 0 and the mean squared
 * distance E_k / n_k changed by less than eps on two consecutive iterations.
 *   R_out, t_out : the last solved transform (host).
 *   E_hist       : optional [max_iter] fp64, E_k per iteration done.
 *   Rt_hist      : optional [max_iter][12] fp64, (R_k row-major, t_k) used by
 *                  iteration k.
 *   iters_done   : optional, iterations completed.
 *   flags        : KDNN_ICP_NO_SORT or KDNN_ICP_SORT, and the schedule flags.
 *   reject       : optional correspondence rejection (kdnn_icp_reject): the
 *                  pairs of iteration k are those within max_dist, E_k and
 *                  n_k count them; with reject_k > 0 each iteration solves,
 *                  rejects by residual (icp_reject_reduce) and solves again.
 * The traversal order is computed once, from the source moved by (R0, t0).
 * With one lane per query (no schedule flag or KDNN_LANES(1)) every
 * iteration after the first starts each point's search at the leaf that held
 * its match in the previous iteration (kept in ws), with the rest of the tree
 * still searched as far as the bound requires: the same pairs as a search
 * from the root, in fewer dependent steps.  The subtrees beside that leaf's
 * path are bounded along their parents' split axes by the near faces of
 * their boxes, read from the leaf's 64-byte plane record (kept with the tree:
 * 64 bytes per leaf).
 * Default (and KDNN_ICP_HOST_LOOP): the article's loop (§3.3) -- each
 * iteration's 17 sums come back to the host (a pinned readback), which solves
 * with kdnn_procrustes (SVD, det sign fix) and applies the convergence rule
 * before launching the next iteration.
 * KDNN_ICP_DEVICE_LOOP (one lane per query: no schedule flag or
 * KDNN_LANES(1); max_iter <= 512): the iterations stay on the device -- each
 * one's sums are reduced and solved (Horn's quaternion form) by a one-group
 * kernel that applies the convergence rule and leaves the next transform for
 * the next search (with reject_k > 0: the first solve for the residual pass,
 * then the kept pairs'), so all iterations are enqueued at once (in chunks of
 * 4 when eps > 0, to stop soon after convergence) and the host waits once.
 * KDNN_ICP_DEVICE_LOOP with another schedule or max_iter > 512 is EINVAL.
 * On EDEGENERATE the outputs hold the last good transform.
 * Errors: EINVAL, EDEVICE, EDEGENERATE. */
kdnn_status icp_align(const kdnn_tree *tree, const float *src_dev, int64_t n, const double *R0_host,
                      const double *t0_host, int32_t max_iter, double eps, double *R_out,
                      double *t_out, double *E_hist, double *Rt_hist, int32_t *iters_done,
                      uint32_t flags, const kdnn_icp_reject *reject, void *ws_dev,
                      size_t ws_bytes, hipStream_t stream);

/* icp_align for callers that cannot allocate device memory -- code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation:
 * the same registration, arguments and results as icp_align, with no
 * workspace argument.  Its workspace is a library-owned device array of
 * KDNN_NOALLOC_SCRATCH_BYTES per device (a module global: every device the
 * library runs on holds its copy until the process ends), so the call makes
 * no allocation of any kind.  Limit: n <= KDNN_NOALLOC_MAX_POINTS source
 * points (larger n is EINVAL); the tree must live on the current device.
 * Every call on a device shares that device's array and finds in it what the
 * last call left (no part of it needs to start at zero: each iteration
 * writes every word it reads); the library serialises calls on one device
 * with a lock, since two overlapping calls would race on the array.
 * Synchronises stream.  Errors: EINVAL, EDEVICE, EDEGENERATE (as icp_align). */
#define KDNN_NOALLOC_MAX_POINTS 262144
#define KDNN_NOALLOC_SCRATCH_BYTES (12u << 20)
kdnn_status icp_align_noalloc(const kdnn_tree *tree, const float *src_dev, int64_t n,
                              const double *R0_host, const double *t0_host, int32_t max_iter,
                              double eps, double *R_out, double *t_out, double *E_hist,
                              double *Rt_hist, int32_t *iters_done, uint32_t flags,
                              const kdnn_icp_reject *reject, hipStream_t stream);

/* Bytes of device workspace icp_align_batch needs for B pairs of n[p] source
 * points (partial sums, each pair's loop state and record, ~54 KB, and each
 * point's match leaf, 4 B, for the searches of the next iteration).
 * 0 if B < 1, n is NULL or some n[p] < 1. */
size_t icp_batch_workspace_bytes(int32_t B, const int64_t *n);

/* B independent registrations advanced together (article §3.4: consecutive
 * frames kept in flight at once so the GPU stays busy; here no host round trip
 * per iteration at all, unless KDNN_ICP_HOST_LOOP).  No allocation: every
 * buffer is the caller's workspace or host arrays of this call.  Pair p registers src_dev[p] (n[p]
 * points) onto trees[p] exactly as icp_align does with flags
 * KDNN_ICP_NO_SORT and one lane per query: same iteration, same convergence
 * rule per pair, and the same max_dist bound.  Each launch carries up to 8
 * pairs, each pair on its own XCDs so that its tree stays in their L2.
 *   trees, src_dev, n : [B] (all trees on the current device).
 *   R0_host, t0_host  : optional [B][9] / [B][3] (NULL = identity / zero).
 *   R_out, t_out      : [B][9] / [B][3], the last solved transforms.
 *   E_hist            : optional [B][max_iter], E_k of each pair.
 *   iters_done        : optional [B].      status_out : optional [B].
 *   flags             : 0 or KDNN_ICP_NO_SORT, and one of KDNN_ICP_HOST_LOOP (each
 *                       iteration's sums come back and the host solves) or
 *                       KDNN_ICP_DEVICE_LOOP (the default for max_iter <= 512:
 *                       each pair's reduction group solves and advances its loop
 *                       on the device and the host waits once -- the frames stay
 *                       in flight with no host round trip, §3.4; beyond 512
 *                       iterations the host loop).
 *   reject            : optional; max_dist only (reject_k > 0 is EINVAL).
 *   ws_dev            : >= icp_batch_workspace_bytes(B, n), 256-byte aligned.
 * A pair whose solve degenerates stops with its last good transform and its
 * status_out entry set; the others go on, and the call returns EDEGENERATE.
 * Synchronises stream.  Errors: EINVAL, EDEVICE, EDEGENERATE. */
kdnn_status icp_align_batch(int32_t B, const kdnn_tree *const *trees, const float *const *src_dev,
                            const int64_t *n, const double *R0_host, const double *t0_host,
                            int32_t max_iter, double eps, double *R_out, double *t_out,
                            double *E_hist, int32_t *iters_done, kdnn_status *status_out,
                            uint32_t flags, const kdnn_icp_reject *reject, void *ws_dev,
                            size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------- preprocessing */

/* Bytes of device workspace voxel_downsample needs for n points. */
size_t voxel_downsample_workspace_bytes(int64_t n);

/* Voxel-grid down-sampling (article §4.3: filter the cloud with a voxel grid
 * before building the tree; leaf 0.05-0.1 m indoors, 0.2-0.5 m outdoors).
 * The voxel of p is (floor(p_x / leaf), floor(p_y / leaf), floor(p_z / leaf)),
 * each quotient in fp64.  Every occupied voxel yields one point, the mean of
 * its points (fp64 sums in ascending point index, one round-to-nearest cast
 * to fp32).  Voxels come out by ascending linear key
 * (vx - min vx) + Nx ((vy - min vy) + Ny (vz - min vz)) over the grid spanned
 * by the occupied voxels (x fastest).  Points with a non-finite coordinate
 * belong to no voxel.
 *   xyz_dev    : n x 3 fp32 points (device).
 *   leaf       : voxel side, finite and > 0.
 *   out_dev    : room for n x 3 fp32 (device); the first *m_out rows are set.
 *   m_out      : host, number of voxels.
 *   counts_dev : optional, room for n int32: points per voxel.
 *   ws_dev     : >= voxel_downsample_workspace_bytes(n), 256-byte aligned.
 * Synchronises stream.  n == 0 gives *m_out = 0.
 * Errors: EINVAL (also when the grid over the cloud's extent would need
 * 2^32 cells or more), EDEVICE. */
kdnn_status voxel_downsample(const float *xyz_dev, int64_t n, double leaf, float *out_dev,
                             int64_t *m_out, int32_t *counts_dev, void *ws_dev, size_t ws_bytes,
                             hipStream_t stream);

/* ---------------------------------------------------------------- misc */

/* Text of the last error on the calling thread ("" if none).  Valid until the
 * next kdnn call on that thread. */
const char *kdnn_last_error(void);

/* Kernel timing, a profiling aid.  After kdnn_timing_begin(cap), each of the
 * calling thread's next `cap` search launches (nn_query, nn_query_radius,
 * icp_correspond_reduce, icp_correspond_reduce_async and each iteration of
 * icp_align) has its search kernel's dispatch stamp a pair of HIP events with
 * its start and end time (hipExtLaunchKernel; the traversal-order sort before
 * it and the reduction after it fall outside; the two-pass schedule spans
 * both passes); later launches are not timed.  kdnn_timing_end waits for the recorded events,
 * writes the launch count to *count_out (optional) and, when ms_out is not
 * null, the search kernel's duration in milliseconds of launch k to
 * ms_out[k] (cap_out entries available, at least the count), and ends timing.
 * cap: 1 .. KDNN_TIMING_MAX.  Errors: EINVAL (cap out of range, timing not
 * started, cap_out too small: timing ends anyway), EDEVICE. */
#define KDNN_TIMING_MAX 65536
kdnn_status kdnn_timing_begin(int32_t cap);
kdnn_status kdnn_timing_end(float *ms_out, int32_t cap_out, int32_t *count_out);

/* Roofline micro-benchmarks, a measurement aid: the ceilings of the memory
 * level a working set of a given size lives in (L2, Infinity Cache, HBM) for
 * the access shapes of the search.  Not used by any search.
 *
 * kdnn_gather_bench: `lanes` lanes (a positive multiple of 256) each read
 * `rounds` records (a positive multiple of 4) at pseudo-random indices in
 * [0, n_records), four at a time; a record is `words` consecutive 16-byte
 * words (1: one point; 3: a child-pair box load; 16: a leaf chunk).
 *   buf_dev  : n_records * words * 16 bytes of device memory, 16-byte aligned,
 *              any contents; read only.
 *   sink_dev : one device word the kernel may write (keeps its loads alive).
 *   seed     : varies the index stream.
 *   ms_out   : host; kernel time measured with events on stream (waits).
 * Useful bytes per launch: lanes * rounds * words * 16.
 *
 * kdnn_chase_bench: `waves` waves of 64 lanes each follow a chain of `steps`
 * dependent loads: record i (64 bytes) holds the index of the next record in
 * its first uint32; an index >= n_records is read as n_records - 1.
 *   next_dev : n_records * 64 bytes, 64-byte aligned (e.g. a random cyclic
 *              permutation written by the caller).
 *   ms_out   : host; kernel time (waits).  Latency per hop = ms / steps.
 * Errors (both): EINVAL (arguments out of range, null or misaligned
 * pointers), EDEVICE. */
kdnn_status kdnn_gather_bench(const void *buf_dev, int64_t n_records, int32_t words, int64_t lanes,
                              int32_t rounds, uint32_t seed, uint32_t *sink_dev, float *ms_out,
                              hipStream_t stream);
kdnn_status kdnn_chase_bench(const uint32_t *next_dev, int64_t n_records, int32_t waves,
                             int32_t steps, uint32_t *sink_dev, float *ms_out, hipStream_t stream);

/* Replay ceiling of one search launch, a measurement aid like the two above:
 * the time the memory system takes to deliver exactly the records a search
 * launch's queries visit, in that launch's work-groups, waves and XCDs, with
 * the dependencies between them removed.  A search kernel's time over this
 * time is how far its dependent chains and instruction stream keep it from
 * the memory system's own limit for that access stream.
 *   1. The instrumented single-lane search (the one nn_query_stats counts)
 *      records each query's visits: the split plane of each node on its
 *      point location's path below the top 8 levels (8 B; those come from
 *      LDS), its start leaf's plane record (64 B),
 *      each internal node's run of child boxes (48 B), each leaf (its points,
 *      loaded in chunks as the search loads them); at most KDNN_REPLAY_CAP
 *      per query.
 *      With q_prev_dev (the previous ICP iteration's queries, m points) each
 *      search starts as icp_align's do after the first iteration: at the
 *      leaf of that query's nearest neighbour, with that leaf's plane record
 *      (64 B: the split axes of its deepest 14 ancestors and the near faces
 *      of their off-path children's boxes along them) and, in trees
 *      deeper than 14 levels, the box of each sibling subtree above those
 *      (32 B each) in place of the descent.
 *   2. The rows are laid out per wave in the launch shape of the production
 *      kernel: nn_query's one-lane-per-query kernel, or with KDNN_REPLAY_ICP
 *      the fused ICP kernel's (work-groups, queries per wave, spread of
 *      positions over each XCD's segment, order).
 *   3. A kernel in that shape loads each wave's visits with its 64 lanes,
 *      dealt round-robin, two in flight per lane; timed `reps` times.
 *   q_dev  : m query points (x, y, z fp32, device), already transformed.
 *   flags  : KDNN_QUERY_SORT / KDNN_QUERY_NO_SORT (default: the tree's
 *            automatic choice for nn_query, or for the ICP entry points
 *            with KDNN_REPLAY_ICP), KDNN_REPLAY_ICP.
 *   ws_dev : kdnn_replay_workspace_bytes(tree, m, flags) bytes of device
 *            memory (about 4 KB per query), caller-owned.
 *   ms_out : host, reps floats: each replay's kernel time (events).
 *   info   : host: what was replayed (below).
 * Synchronous (returns after the replays).  Errors: EINVAL (m < 1, reps < 1,
 * null pointers, unknown flag, small workspace), EDEVICE. */
#define KDNN_REPLAY_ICP 4u
#define KDNN_REPLAY_CAP 512
typedef struct kdnn_replay_info {
    int64_t visits;        /* root, box-run and leaf visits replayed */
    int64_t bytes;         /* bytes one replay loads */
    int64_t node_records;  /* node records the visits stand for (cold start: the sum of
                              nn_query_stats' node counts; a warm start's plane record: 2,
                              each sibling box it loads: 1) */
    int64_t leaf_points;   /* leaf points they stand for (sum of nn_query_stats' points) */
    int64_t truncated;     /* queries with more than KDNN_REPLAY_CAP visits (tail not replayed) */
    int64_t blocks;        /* work-groups of the launch shape */
    int32_t queries_per_wave;
    int32_t spread;        /* 1: positions spread over each XCD's segment */
} kdnn_replay_info;
size_t kdnn_replay_workspace_bytes(const kdnn_tree *tree, int64_t m, uint32_t flags);
kdnn_status kdnn_replay_bench(const kdnn_tree *tree, const float *q_dev, const float *q_prev_dev,
                              int64_t m, uint32_t flags, int32_t reps, void *ws_dev,
                              size_t ws_bytes, float *ms_out, kdnn_replay_info *info,
                              hipStream_t stream);

/* KDNN_VERSION of the built library. */
int32_t kdnn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDNN_H */
