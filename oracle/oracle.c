/*
 * ORACLE -- test infrastructure, not product code.
 *
 * Plain, slow, obviously-correct CPU nearest-neighbour search used to check
 * the HIP library.  Only the tests, the smoke check and the benchmark's CPU
 * baseline may load this file's shared object.  It shares no code, header,
 * table or helper with the library under kd_tree_nn_amd/.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fPIC -shared
 * (contraction off so that every product and sum below is rounded to fp32
 * exactly as written; x86-64 evaluates float in SSE, FLT_EVAL_METHOD == 0).
 *
 * What is computed (CUDA-KDTree ICP article, pwwt.cn, §3.2 "nn_kernel"):
 * for a query q the nearest target point under the squared Euclidean
 * distance, reported as (index, squared distance).  The distance is the fp32
 * expression d = (dx*dx + dy*dy) + dz*dz with d? = target - query, each
 * operation rounded to fp32.  Ties are broken towards the lowest target
 * index.  With no candidate strictly closer than +inf the answer is
 * (-1, +inf); that covers a query with a NaN/Inf coordinate.
 *
 * Pinning (see tests/test_oracle_nn.py): hand-built cases with exact
 * answers, a comparison with scipy's exact fp64 KD-tree search, and bit
 * equality between okd_query and oracle_brute_nn on adversarial inputs.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------------- */
/* O1: brute force -- the definition itself.                               */
/* ---------------------------------------------------------------------- */

/* One query against every target point, ascending index, strict '<' so the
 * first (lowest-index) point attaining the minimum is kept. */
static void brute_one(const float *T, int64_t n, float qx, float qy, float qz,
                      int32_t *out_idx, float *out_d2)
{
    float best = INFINITY;
    int32_t bi = -1;
    for (int64_t j = 0; j < n; ++j) {
        const float dx = T[3 * j + 0] - qx;
        const float dy = T[3 * j + 1] - qy;
        const float dz = T[3 * j + 2] - qz;
        const float d = (dx * dx + dy * dy) + dz * dz;
        if (d < best) {
            best = d;
            bi = (int32_t)j;
        }
    }
    *out_idx = bi;
    *out_d2 = best;
}

void oracle_brute_nn(const float *T, int64_t n, const float *Q, int64_t m,
                     int32_t *idx, float *d2)
{
    for (int64_t i = 0; i < m; ++i)
        brute_one(T, n, Q[3 * i], Q[3 * i + 1], Q[3 * i + 2], idx + i, d2 + i);
}

/* ---------------------------------------------------------------------- */
/* O2: an independent, deliberately simple exact KD-tree (an accelerator   */
/* for large inputs; the answer must equal O1 bit for bit).               */
/*                                                                        */
/* Build: recursive, axis cycles x -> y -> z with depth, points of a node */
/* fully sorted on that axis (ties by index), split at the middle element. */
/* A node becomes a leaf once it holds <= leaf_size points.  Every node   */
/* keeps the tight bounding box of its points.                            */
/* Search: recursive, nearer side first; a subtree is skipped when the    */
/* fp32 distance from q to its box exceeds the best distance so far.  The */
/* box distance is a valid lower bound of every fp32 point distance in    */
/* the box because each rounding step is monotone, so nothing that could */
/* tie or beat the current best is ever skipped.                          */
/* ---------------------------------------------------------------------- */

typedef struct {
    float lo[3], hi[3];
    float split;
    int32_t axis;
    int32_t left, right; /* -1 for a leaf */
    int64_t begin, end;  /* range of perm[] held by the node */
} okd_node;

typedef struct {
    int64_t n;
    float *pts;     /* private copy of the target, AoS */
    int64_t *perm;  /* point ids; every node owns a contiguous run */
    okd_node *nodes;
    int64_t n_nodes, cap;
    int32_t leaf;
} okd_tree;

static const float *g_sort_pts; /* qsort has no context argument in C11 */
static int g_sort_axis;

static int cmp_axis(const void *a, const void *b)
{
    const int64_t i = *(const int64_t *)a, j = *(const int64_t *)b;
    const float x = g_sort_pts[3 * i + g_sort_axis], y = g_sort_pts[3 * j + g_sort_axis];
    if (x < y) return -1;
    if (x > y) return 1;
    return (i > j) - (i < j);
}

static int32_t okd_new_node(okd_tree *t)
{
    if (t->n_nodes == t->cap) {
        t->cap = t->cap ? 2 * t->cap : 64;
        t->nodes = (okd_node *)realloc(t->nodes, (size_t)t->cap * sizeof(okd_node));
    }
    return (int32_t)t->n_nodes++;
}

static int32_t okd_build_rec(okd_tree *t, int64_t lo, int64_t hi, int depth)
{
    const int32_t id = okd_new_node(t);
    okd_node nd;
    for (int a = 0; a < 3; ++a) {
        nd.lo[a] = INFINITY;
        nd.hi[a] = -INFINITY;
    }
    for (int64_t k = lo; k < hi; ++k)
        for (int a = 0; a < 3; ++a) {
            const float v = t->pts[3 * t->perm[k] + a];
            if (v < nd.lo[a]) nd.lo[a] = v;
            if (v > nd.hi[a]) nd.hi[a] = v;
        }
    nd.begin = lo;
    nd.end = hi;
    nd.left = nd.right = -1;
    nd.axis = depth % 3;
    nd.split = 0.0f;
    if (hi - lo > t->leaf) {
        g_sort_pts = t->pts;
        g_sort_axis = nd.axis;
        qsort(t->perm + lo, (size_t)(hi - lo), sizeof(int64_t), cmp_axis);
        const int64_t mid = lo + (hi - lo) / 2;
        nd.split = t->pts[3 * t->perm[mid] + nd.axis];
        const int32_t l = okd_build_rec(t, lo, mid, depth + 1);
        const int32_t r = okd_build_rec(t, mid, hi, depth + 1);
        nd.left = l;
        nd.right = r;
    }
    t->nodes[id] = nd; /* after recursion: realloc may have moved the array */
    return id;
}

void *okd_build(const float *pts, int64_t n, int32_t leaf_size)
{
    if (n <= 0 || leaf_size < 1) return NULL;
    okd_tree *t = (okd_tree *)calloc(1, sizeof(okd_tree));
    t->n = n;
    t->leaf = leaf_size;
    t->pts = (float *)malloc((size_t)n * 3 * sizeof(float));
    memcpy(t->pts, pts, (size_t)n * 3 * sizeof(float));
    t->perm = (int64_t *)malloc((size_t)n * sizeof(int64_t));
    for (int64_t i = 0; i < n; ++i) t->perm[i] = i;
    okd_build_rec(t, 0, n, 0);
    return t;
}

void okd_free(void *h)
{
    okd_tree *t = (okd_tree *)h;
    if (!t) return;
    free(t->pts);
    free(t->perm);
    free(t->nodes);
    free(t);
}

int64_t okd_node_count(const void *h) { return ((const okd_tree *)h)->n_nodes; }

static float gap(float q, float lo, float hi)
{
    if (q < lo) return lo - q;
    if (q > hi) return q - hi;
    return 0.0f;
}

typedef struct {
    float best;
    int32_t bi;
    int64_t visits; /* nodes entered, for diagnostics */
} okd_state;

static void okd_search(const okd_tree *t, int32_t id, const float q[3], okd_state *s)
{
    const okd_node *nd = &t->nodes[id];
    const float gx = gap(q[0], nd->lo[0], nd->hi[0]);
    const float gy = gap(q[1], nd->lo[1], nd->hi[1]);
    const float gz = gap(q[2], nd->lo[2], nd->hi[2]);
    const float lb = (gx * gx + gy * gy) + gz * gz;
    /* lb == +inf: every point of the box is at +inf too and cannot win. */
    if (!(lb <= s->best) || lb == INFINITY) return;
    s->visits++;
    if (nd->left < 0) {
        for (int64_t k = nd->begin; k < nd->end; ++k) {
            const int64_t j = t->perm[k];
            const float dx = t->pts[3 * j + 0] - q[0];
            const float dy = t->pts[3 * j + 1] - q[1];
            const float dz = t->pts[3 * j + 2] - q[2];
            const float d = (dx * dx + dy * dy) + dz * dz;
            if (d < s->best || (d == s->best && (int32_t)j < s->bi)) {
                s->best = d;
                s->bi = (int32_t)j;
            }
        }
        return;
    }
    const int go_left = q[nd->axis] < nd->split;
    okd_search(t, go_left ? nd->left : nd->right, q, s);
    okd_search(t, go_left ? nd->right : nd->left, q, s);
}

void okd_query(const void *h, const float *Q, int64_t m, int32_t *idx, float *d2,
               int64_t *visits_or_null)
{
    const okd_tree *t = (const okd_tree *)h;
    for (int64_t i = 0; i < m; ++i) {
        okd_state s = {INFINITY, -1, 0};
        const float q[3] = {Q[3 * i], Q[3 * i + 1], Q[3 * i + 2]};
        okd_search(t, 0, q, &s);
        idx[i] = s.bi;
        d2[i] = s.best;
        if (visits_or_null) visits_or_null[i] = s.visits;
    }
}

/* ---------------------------------------------------------------------- */
/* O9: voxel-grid down-sampling (article §4.3: voxel filter before the     */
/* tree is built).  The plain definition:                                  */
/*   voxel of p = (floor(p_x / leaf), floor(p_y / leaf), floor(p_z / leaf))*/
/*   with each quotient in fp64 (the fp32 coordinate promoted exactly);    */
/*   points with a non-finite coordinate belong to no voxel;               */
/*   every occupied voxel gives one point, the mean of its points: fp64    */
/*   sums taken in ascending original index, divided by the count, one     */
/*   round-to-nearest cast to fp32;                                        */
/*   voxels are listed by ascending linear key                             */
/*   (vx - min vx) + Nx ((vy - min vy) + Ny (vz - min vz)) over the grid   */
/*   spanned by the occupied voxels.                                       */
/* Returns the number of voxels M; out (>= M x 3) and counts (>= M).       */
/* ---------------------------------------------------------------------- */
typedef struct {
    int64_t key;
    int64_t idx;
} vox_item;

static int cmp_vox(const void *a, const void *b)
{
    const vox_item *x = (const vox_item *)a, *y = (const vox_item *)b;
    if (x->key != y->key) return x->key < y->key ? -1 : 1;
    return x->idx < y->idx ? -1 : (x->idx > y->idx);
}

int64_t oracle_voxel(const float *P, int64_t n, double leaf, float *out, int32_t *counts)
{
    int64_t *v = (int64_t *)malloc((size_t)(n > 0 ? n : 1) * 3 * sizeof(int64_t));
    vox_item *it = (vox_item *)malloc((size_t)(n > 0 ? n : 1) * sizeof(vox_item));
    int64_t lo[3] = {0, 0, 0}, hi[3] = {0, 0, 0}, nf = 0;
    for (int64_t i = 0; i < n; ++i) {
        const float *p = P + 3 * i;
        if (!(isfinite(p[0]) && isfinite(p[1]) && isfinite(p[2]))) continue;
        for (int a = 0; a < 3; ++a) {
            const int64_t c = (int64_t)floor((double)p[a] / leaf);
            v[3 * i + a] = c;
            if (nf == 0 || c < lo[a]) lo[a] = c;
            if (nf == 0 || c > hi[a]) hi[a] = c;
        }
        ++nf;
    }
    const int64_t nx = hi[0] - lo[0] + 1, ny = hi[1] - lo[1] + 1;
    int64_t k = 0;
    for (int64_t i = 0; i < n; ++i) {
        const float *p = P + 3 * i;
        if (!(isfinite(p[0]) && isfinite(p[1]) && isfinite(p[2]))) continue;
        it[k].key = (v[3 * i] - lo[0]) + nx * ((v[3 * i + 1] - lo[1]) + ny * (v[3 * i + 2] - lo[2]));
        it[k].idx = i;
        ++k;
    }
    qsort(it, (size_t)nf, sizeof(vox_item), cmp_vox);
    int64_t m = 0;
    for (int64_t s = 0; s < nf;) {
        int64_t e = s;
        double sx = 0.0, sy = 0.0, sz = 0.0;
        while (e < nf && it[e].key == it[s].key) {
            const float *p = P + 3 * it[e].idx;
            sx += (double)p[0];
            sy += (double)p[1];
            sz += (double)p[2];
            ++e;
        }
        const double c = (double)(e - s);
        out[3 * m] = (float)(sx / c);
        out[3 * m + 1] = (float)(sy / c);
        out[3 * m + 2] = (float)(sz / c);
        counts[m] = (int32_t)(e - s);
        ++m;
        s = e;
    }
    free(v);
    free(it);
    return m;
}
