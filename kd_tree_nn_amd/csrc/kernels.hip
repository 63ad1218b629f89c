// HIP kernels for gfx950 (CDNA4, wave64): exact KD-tree nearest-neighbour
// traversal, the fused ICP correspondence + fp64 reduction, the Morton
// ordering of queries (two stable 8-bit radix passes), and the rigid
// transform.  Built with -ffp-contract=off: every fp32 product and sum of
// the distance code is rounded on its own, exactly as the host-side
// definition writes it.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cfloat>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "kdnn_internal.hpp"
#include "rigid_solve.hpp"

namespace kdnn {

// Compile-time tuning knobs (defaults are the shipped configuration).
#ifndef KDNN_WG
#define KDNN_WG 256
#endif
#ifndef KDNN_XCD_REMAP
#define KDNN_XCD_REMAP 1
#endif
constexpr int kWG = KDNN_WG;                      // traversal work-group size
// Queries owned per wave in the one-lane-per-query kernels: q <= 64, chosen
// per launch (wave_plan); with q < 64 the other lanes start idle and take
// over pending subtrees.  (kWG / 64) q queries per work-group and sweep.
#ifndef KDNN_Q_TARGET_NN
#define KDNN_Q_TARGET_NN 33
#endif
#ifndef KDNN_Q_TARGET_ICP
#define KDNN_Q_TARGET_ICP 43
#endif
#ifndef KDNN_TOP_LOC_LEVELS
#define KDNN_TOP_LOC_LEVELS 8
#endif
constexpr uint32_t kQFull = 64;
constexpr int kLeafChunk = 16;                    // leaf points loaded per batch (one lane)
constexpr int kLeafChunkSmall = 8;                // the same for trees whose leaves hold <= 8
constexpr int kSortThreads = 256;
constexpr int kSortItems = 8;
constexpr int kSortTile = kSortThreads * kSortItems;  // keys per radix tile
constexpr int kIcpMaxBlocks = 4096;
constexpr int kNumXcd = 8;
constexpr int kS = KDNN_SUMS_DOUBLES;

// ------------------------------------------------------------------ helpers


// Work-groups are dealt round-robin to the 8 XCDs (each with its own L2).
// Map them so that every XCD works on one contiguous run of logical blocks,
// i.e. on one spatially coherent slice of the Morton-ordered queries.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t b, uint32_t nb)
{
    if (!KDNN_XCD_REMAP) return b;
    const uint32_t x = b % kNumXcd, slot = b / kNumXcd;
    const uint32_t q = nb / kNumXcd, r = nb % kNumXcd;
    return x * q + (x < r ? x : r) + slot;
}

// Which queries share a wave in the one-lane-per-query kernels.  The lanes
// of a wave balance their searches among themselves, which only helps when a
// wave mixes easy and hard queries; hard queries (sparse regions, points far
// from the target) sit close together in space, hence in a Morton order or a
// scan order, and a wave full of them leaves no lane idle to help: that
// wave runs long.  So the kernels deal the positions of the order to lanes
// through a bijection that spreads every wave's q queries evenly over the
// segment of the order its XCD works on.  In each sweep of nb * (kWG / 64) q
// slots the logical blocks of XCD x (xcd_remap) cover one contiguous segment
// [s0, s0 + L), so every XCD still works on one run of the order (one region
// of space for a Morton order: L2 locality).  Inside the segment (W =
// ceil(L / q) waves, the last one d = q W - L queries short), query lane l of
// the segment's wave w takes position s0 + start(l) + w, where start(l) =
// l W - max(0, l - (q - d)) lays the q lanes' rows end to end.
__device__ __forceinline__ int64_t spread_in(int64_t j, int64_t L, uint32_t q)
{
    const int Q = int(q);
    const int64_t W = (L + Q - 1) / Q;
    const int64_t w = j / Q;
    const int l = int(j - w * Q);
    const int d = int(int64_t(Q) * W - L);
    const int64_t start = int64_t(l) * W - (l > Q - d ? l - (Q - d) : 0);
    return start + w;
}

// Position for slot k < m (blk = xcd_remap(blockIdx.x, nb); base = the
// sweep's first slot of this block).  spread == false: position k.
__device__ __forceinline__ int64_t spread_pos(bool spread, uint32_t wq, int64_t k, int64_t blk,
                                              int64_t base, uint32_t nb, int64_t m)
{
    if (!KDNN_XCD_REMAP || !spread) return k;
    const int64_t QB = int64_t(kWG / 64) * wq;
    const int64_t sweep = base - blk * QB;
    const uint32_t x = blockIdx.x % kNumXcd;
    const uint32_t q = nb / kNumXcd, r = nb % kNumXcd;
    const int64_t s0 = sweep + (int64_t(x) * q + (x < r ? x : r)) * QB;
    const int64_t e = s0 + (int64_t(q) + (x < r ? 1 : 0)) * QB;
    return s0 + spread_in(k - s0, (e < m ? e : m) - s0, wq);
}

// ----------------------------------------------------------- NN traversal
//
// Exact nearest neighbour on the implicit heap (root 1, children 2i, 2i+1).
// Depth-first, nearer child first (the child on the query's side of the
// split plane); a subtree is entered only if the fp32 distance from the
// query to its bounding box is <= the best distance so far.  The box of the
// far child lies entirely beyond the split plane, so this prunes everything
// the plane test prunes and more.  That distance is a lower bound of every
// fp32 point distance in the box (each rounding step is monotone), so a
// point that could beat or tie the best is never skipped.
//
// Candidates are ranked by the 64-bit key (fp32 distance bits, original
// index): distances are >= 0, whose bit patterns order like their values, so
// "closer, or as close with a lower index" is one unsigned comparison and
// the result is the lowest-index nearest point whatever the visiting order.
// A distance that overflows to +inf is never an answer (nothing is strictly
// closer than the initial +inf), hence the final fix-up to index -1.
//
// No stack: the node index spells the path from the root, and bit d of
// `far` records whether the path node at depth d+1 is a far child.  After a
// subtree is done, the next subtree is the far sibling of the deepest path
// node that is still a near child.  Node steps are branch-free (selects), so
// the two 16-byte loads of a node are in flight together and lanes of a
// wave that disagree on the way only differ in data, not in control flow.
//
// Wave shape: lanes walk internal nodes until every lane of the wave has
// reached a leaf (or finished), then all of them scan their leaves at once.
// Leaf j owns point slots [floor(j n/2^D), floor((j+1) n/2^D)), so its points
// are loaded together with its record.
constexpr uint32_t kDone = 0xFFFFFFFFu;

struct Best {
    float d;
    int32_t idx;
    uint32_t slot;  // leaf-order slot of the winner (when idx >= 0)
};

struct TreeView {
    const float4 *__restrict__ nodes;
    const float4 *__restrict__ boxes;     // children of i: boxes[3i .. 3i+2] (48 B)
    const float4 *__restrict__ pts;
    const int32_t *__restrict__ slot_of;  // original index -> leaf-order slot
    const uint4 *__restrict__ paths;      // per leaf: 64-byte plane record (kPathWords)
    uint32_t first_leaf;  // 2^D
    int32_t depth;        // D
    int64_t n;
};

__device__ __forceinline__ uint64_t nn_key(float d, uint32_t idx)
{
    return (uint64_t(__float_as_uint(d)) << 32) | idx;
}

__device__ __forceinline__ float key_dist(uint64_t k) { return __uint_as_float(uint32_t(k >> 32)); }

// A search starts from a bound key (d_max bits, index 0xFFFFFFFF): no real
// point has that index, so a point at exactly d_max still ranks below it,
// and a key still carrying the index field 0xFFFFFFFF at the end is a miss.
__device__ __forceinline__ uint64_t bound_key(float dmax2) { return nn_key(dmax2, 0xFFFFFFFFu); }

__device__ __forceinline__ void finish(uint64_t key, uint32_t slot, Best &b)
{
    const float d = key_dist(key);
    const bool hit = uint32_t(key) != 0xFFFFFFFFu && d < INFINITY;
    b.d = hit ? d : INFINITY;
    b.idx = hit ? int32_t(uint32_t(key)) : -1;
    b.slot = slot;
}

// The subtree that follows the finished subtree i (kDone when none is left
// at depth >= floor, `floor_mask` = ~(2^floor - 1)); updates `far`.
__device__ __forceinline__ uint32_t next_subtree(uint32_t i, uint32_t &far, uint32_t floor_mask)
{
    const uint32_t dep = 31u - uint32_t(__clz(int(i)));
    const uint32_t open = ~far & ((1u << dep) - 1u) & floor_mask;
    const uint32_t h = 31u - uint32_t(__clz(int(open | 1u)));
    const uint32_t nxt = (i >> ((dep - h - 1u) & 31u)) ^ 1u;
    const uint32_t nfar = (far & ((1u << h) - 1u)) | (1u << h);
    far = open ? nfar : far;
    return open ? nxt : kDone;
}

// fp32 squared distance from q to the box (lo = A.xyz, hi = (A.w, B.x, B.y)).
// Per axis the gap is max(lo - q, q - hi, 0): the same single fp32
// subtraction as "lo - q if q < lo, q - hi if q > hi, else 0".
__device__ __forceinline__ float box_lb(float qx, float qy, float qz, const float4 &A,
                                        const float4 &B)
{
    const float gx = fmaxf(fmaxf(A.x - qx, qx - A.w), 0.0f);
    const float gy = fmaxf(fmaxf(A.y - qy, qy - B.x), 0.0f);
    const float gz = fmaxf(fmaxf(A.z - qz, qz - B.y), 0.0f);
    return (gx * gx + gy * gy) + gz * gz;
}

// A search's best distance starts finite (the largest float when there is no
// bound, see host_bound_key), so a subtree whose bound overflowed to +inf is
// never entered; that is exact: every fp32 point distance in such a box is
// +inf as well (the rounding is monotone), and a point at +inf is never a
// match.
__device__ __forceinline__ bool enters(float lb, float best) { return lb <= best; }

__device__ __forceinline__ uint32_t near_child(uint32_t i, const float4 &B, float qx, float qy,
                                               float qz)
{
    const uint32_t axis = __float_as_uint(B.w);
    const float qa = axis == 0 ? qx : (axis == 1 ? qy : qz);
    return 2 * i + (qa >= B.z ? 1u : 0u);
}

__device__ __forceinline__ void leaf_range(const TreeView &t, uint32_t i, int32_t &begin,
                                           int32_t &last, int32_t &end)
{
    const uint64_t j = uint64_t(i - t.first_leaf);
    begin = int32_t((j * uint64_t(t.n)) >> t.depth);
    end = int32_t(((j + 1) * uint64_t(t.n)) >> t.depth);
    last = end > begin ? end - 1 : begin;  // a valid slot even for an empty leaf
}

// The leaf (heap index) whose range holds leaf-order slot s < n: leaf j starts
// at floor(j n / 2^D), so j is the largest with floor(j n / 2^D) <= s, i.e.
// ceil((s + 1) 2^D / n) - 1.
__device__ __forceinline__ uint32_t leaf_of_slot(const TreeView &t, uint32_t s)
{
    const uint64_t num = (uint64_t(s + 1u) << t.depth) - 1u;
    return t.first_leaf + uint32_t(num / uint64_t(t.n));
}

// Load C points (slots first, first + S, ...; clamped to `last`), then rank
// them.  Clamped repeats of the last point carry its own key and never
// replace it.
template <int C, int S>
__device__ __forceinline__ void load_points(const TreeView &t, int32_t first, int32_t last,
                                            float4 (&p)[C], int32_t (&sl)[C])
{
#pragma unroll
    for (int c = 0; c < C; ++c) {
        sl[c] = min(first + c * S, last);
        p[c] = t.pts[sl[c]];
    }
}

template <int C>
__device__ __forceinline__ void rank_points(const float4 (&p)[C], const int32_t (&sl)[C], float qx,
                                            float qy, float qz, uint64_t &key, uint32_t &slot)
{
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const float dx = p[c].x - qx;
        const float dy = p[c].y - qy;
        const float dz = p[c].z - qz;
        const float d = (dx * dx + dy * dy) + dz * dz;
        const uint64_t k = nn_key(d, __float_as_uint(p[c].w));
        const bool lt = k < key;
        key = lt ? k : key;
        slot = lt ? uint32_t(sl[c]) : slot;
    }
}

// Single-lane search from the bound key `init` (bound +inf: none).  Stops
// after `budget` node records when the budget is below kNoBudget; returns
// whether the search completed.  key/slot hold the best candidate seen so far
// either way (a valid upper bound to resume from).
constexpr uint32_t kNoBudget = 0xFFFFFFFFu;

// Node record i: from the LDS copy of the top levels when i < lds_first.
__device__ __forceinline__ void fetch_node(const TreeView &t, const float4 *lds, uint32_t lds_first,
                                           uint32_t i, float4 &A, float4 &B)
{
    if (i < lds_first) {
        A = lds[2 * i];
        B = lds[2 * i + 1];
    } else {
        A = t.nodes[2 * i];
        B = t.nodes[2 * i + 1];
    }
}

template <bool STATS>
__device__ __forceinline__ bool nn_search(const TreeView &t, float qx, float qy, float qz,
                                          uint64_t init, uint32_t budget, uint64_t &key,
                                          uint32_t &slot, uint32_t &cn, uint32_t &cp,
                                          const float4 *lds = nullptr, uint32_t lds_first = 0)
{
    key = init;
    slot = 0;
    if (!(isfinite(qx) && isfinite(qy) && isfinite(qz))) return true;
    uint32_t i = 1, far = 0, steps = 0;
    for (;;) {
        // Phase 1: internal nodes, until a leaf or the end of the search.
        while (i < t.first_leaf) {
            if (steps >= budget) return false;
            float4 A, B;
            fetch_node(t, lds, lds_first, i, A, B);
            ++steps;
            if (STATS) ++cn;
            const bool in = enters(box_lb(qx, qy, qz, A, B), key_dist(key));
            const uint32_t child = near_child(i, B, qx, qy, qz);
            uint32_t f2 = far;
            const uint32_t nx = next_subtree(i, f2, ~0u);
            i = in ? child : nx;
            far = in ? far : f2;
        }
        if (i == kDone) return true;
        if (steps >= budget) return false;
        // Phase 2: leaf i -- its record and first points in flight together.
        int32_t begin, last, end;
        leaf_range(t, i, begin, last, end);
        const float4 A = t.nodes[2 * i];
        const float4 B = t.nodes[2 * i + 1];
        float4 p[kLeafChunk];
        int32_t sl[kLeafChunk];
        load_points<kLeafChunk, 1>(t, begin, last, p, sl);
        ++steps;
        if (STATS) ++cn;
        if (enters(box_lb(qx, qy, qz, A, B), key_dist(key))) {
            rank_points<kLeafChunk>(p, sl, qx, qy, qz, key, slot);
            for (int32_t k0 = begin + kLeafChunk; k0 < end; k0 += kLeafChunk) {
                load_points<kLeafChunk, 1>(t, k0, last, p, sl);
                rank_points<kLeafChunk>(p, sl, qx, qy, qz, key, slot);
            }
            if (STATS) cp += uint32_t(end - begin);
        }
        i = next_subtree(i, far, ~0u);
    }
}

// ------------------------------------------------ cooperative (G-lane) search
//
// At small query counts the GPU is mostly idle and a launch lasts as long as
// its slowest query chain, so G consecutive lanes share one query:
//  1. all G lanes walk the greedy root-to-leaf path of the query, keeping the
//     fp32 squared distance from the query to each split plane on the path
//     (lane l % G keeps depth l);
//  2. they scan the query's own leaf together and agree on a first best;
//  3. the shallowest path depth k whose plane distance is <= best marks the
//     deepest ancestor v_k whose cell contains the search ball: any point
//     outside v_k's subtree is on the other side of some split of v_0..v_k-1
//     and therefore at fp32 distance >= that plane distance > best (rounding
//     is monotone), so it can neither beat nor tie the best;
//  4. the subtree of v_k is cut into min(G, 2^(D-k)) disjoint subtrees, one
//     per lane, each searched depth-first as above with the group's best
//     (minimum key over the G lanes) for pruning.
// The answer is the minimum key over everything scanned: the same exact
// lowest-index nearest point.
constexpr int kDevMaxDepth = 28;

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int off)
{
    const uint32_t lo = uint32_t(__shfl_xor(int(uint32_t(v)), off, 64));
    const uint32_t hi = uint32_t(__shfl_xor(int(uint32_t(v >> 32)), off, 64));
    return (uint64_t(hi) << 32) | lo;
}

template <int G>
__device__ __forceinline__ uint64_t group_min_key(uint64_t k)
{
#pragma unroll
    for (int off = 1; off < G; off <<= 1) {
        const uint64_t o = shfl_xor_u64(k, off);
        k = o < k ? o : k;
    }
    return k;
}

template <int G>
__device__ __forceinline__ uint32_t group_sum_u32(uint32_t v)
{
#pragma unroll
    for (int off = 1; off < G; off <<= 1) v += uint32_t(__shfl_xor(int(v), off, 64));
    return v;
}

// `key`/`slot` come in as an upper bound (a bound key when nothing is found yet) and go out as the
// group's answer; with `resume` the query's own leaf is known to be scanned.
template <int G, bool STATS>
__device__ __forceinline__ void nn_search_group(const TreeView &t, float qx, float qy, float qz,
                                                bool resume, uint64_t &key, uint32_t &slot,
                                                uint32_t &cn, uint32_t &cp)
{
    constexpr int LOG_G = G == 2 ? 1 : G == 4 ? 2 : G == 8 ? 3 : G == 16 ? 4 : 5;
    constexpr int SLOTS = (kDevMaxDepth + G - 1) / G;
    constexpr int C = 16 / G > 1 ? 16 / G : 2;  // own-leaf points per lane per round
    constexpr int CL = 8;                        // points per batch in a lane's own leaves
    const int lane = threadIdx.x & 63;
    const int gl = lane & (G - 1);
    const int gbase = lane & ~(G - 1);
    const uint64_t gmask = (G == 64 ? ~uint64_t(0) : ((uint64_t(1) << G) - 1)) << gbase;
    const int D = t.depth;

    // 1. greedy descent, plane distances kept round-robin over the group
    uint32_t i = 1;
    float pd[SLOTS];
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) pd[s] = INFINITY;
#pragma unroll
    for (int l = 0; l < kDevMaxDepth; ++l) {
        if (l < D) {
            const float4 B = t.nodes[2 * i + 1];  // hi.y hi.z split axis
            const uint32_t axis = __float_as_uint(B.w);
            const float qa = axis == 0 ? qx : (axis == 1 ? qy : qz);
            const bool right = qa >= B.z;
            const float dl = right ? qa - B.z : B.z - qa;
            if ((l & (G - 1)) == gl) pd[l / G] = dl * dl;
            i = 2 * i + (right ? 1u : 0u);
        }
    }
    if (STATS && gl == 0) cn += uint32_t(D);

    // 2. the query's own leaf, scanned by the whole group (a resumed search
    //    has scanned it already when it holds any candidate: a first pass
    //    always reaches the greedy leaf first unless a bound prunes it)
    if (!resume || uint32_t(key) == 0xFFFFFFFFu) {
        int32_t begin, last, end;
        leaf_range(t, i, begin, last, end);
        for (int32_t k0 = begin; k0 < end; k0 += G * C) {
            float4 p[C];
            int32_t sl[C];
            load_points<C, G>(t, k0 + gl, last, p, sl);
            rank_points<C>(p, sl, qx, qy, qz, key, slot);
        }
        if (STATS && gl == 0) {
            ++cn;
            cp += uint32_t(end - begin);
        }
    }
    uint64_t gkey = group_min_key<G>(key);

    // 3. shallowest path depth whose split plane is within the best distance
    int kstar = D;
    {
        const float gb = key_dist(gkey);
#pragma unroll
        for (int s = 0; s < SLOTS; ++s) {
            const int l = s * G + gl;
            const uint64_t m = __ballot(l < D && pd[s] <= gb) & gmask;
            if (m != 0 && kstar == D) kstar = s * G + (__ffsll((unsigned long long)m) - 1 - gbase);
        }
    }

    // 4. lanes search disjoint parts of the subtree of v_kstar
    if (kstar < D) {
        const int gp = LOG_G < D - kstar ? LOG_G : D - kstar;
        const uint32_t vk = i >> (D - kstar);
        const uint32_t floor_mask = ~((1u << uint32_t(kstar + gp)) - 1u);
        uint32_t ci = gl < (1 << gp) ? ((vk << gp) | uint32_t(gl)) : kDone;
        uint32_t far = 0;
        for (;;) {
            if (ci != kDone) {
                const float4 A = t.nodes[2 * ci];
                const float4 B = t.nodes[2 * ci + 1];
                if (STATS) ++cn;
                const bool in = enters(box_lb(qx, qy, qz, A, B), key_dist(gkey));
                if (ci < t.first_leaf) {
                    const uint32_t child = near_child(ci, B, qx, qy, qz);
                    uint32_t f2 = far;
                    const uint32_t nx = next_subtree(ci, f2, floor_mask);
                    ci = in ? child : nx;
                    far = in ? far : f2;
                } else {
                    if (in) {
                        int32_t begin, last, end;
                        leaf_range(t, ci, begin, last, end);
                        for (int32_t k0 = begin; k0 < end; k0 += CL) {
                            float4 p[CL];
                            int32_t sl[CL];
                            load_points<CL, 1>(t, k0, last, p, sl);
                            rank_points<CL>(p, sl, qx, qy, qz, key, slot);
                        }
                        if (STATS) cp += uint32_t(end - begin);
                    }
                    ci = next_subtree(ci, far, floor_mask);
                }
            }
            gkey = group_min_key<G>(key);
            if ((__ballot(ci != kDone) & gmask) == 0) break;
        }
    }

    // 5. the group's answer and the winning lane's slot
    const uint64_t wm = __ballot(key == gkey) & gmask;
    const int win = __ffsll((unsigned long long)wm) - 1;
    slot = uint32_t(__shfl(int(slot), win, 64));
    key = gkey;
    if (STATS) {
        cn = group_sum_u32<G>(cn);
        cp = group_sum_u32<G>(cp);
    }
}

// ------------------------------------------------ pair-load search (one lane)
//
// The single-lane search of the default schedule.  Entering an internal node
// loads the boxes of both its children together (one 48-byte run of the box
// array, three 16-byte loads); their
// box bounds set the visiting order (smaller bound first) and tell at once
// whether the other child can be dropped -- for good, since the best
// distance only shrinks.  The other child's bound is kept per path level in
// LDS (one float per level and lane) and a bit of `pend` marks it as still
// pending, so coming back to it costs an LDS read instead of a memory round
// trip, and a node is never fetched twice.  Exactness is as above: a child is
// skipped only when its box bound exceeds the best distance at that moment.
//
// Path levels: bit d of `pend` and lbs[d * kWG] belong to depth d + 1.

// The node to enter after the subtree of i is finished: the pending second
// child at the deepest path level whose bound is still <= best; kDone if none.
__device__ __forceinline__ uint32_t pair_next(uint32_t i, uint32_t &pend, const float *lbs,
                                              float best)
{
    const uint32_t dep = 31u - uint32_t(__clz(int(i)));
    uint32_t cand = pend & ((1u << dep) - 1u);
    while (cand != 0u) {
        const uint32_t h = 31u - uint32_t(__clz(int(cand)));
        if (enters(lbs[h * kWG], best)) {
            pend &= (1u << h) - 1u;  // level h + 1 now holds its second child
            return (i >> (dep - h - 1u)) ^ 1u;
        }
        cand &= ~(1u << h);
    }
    return kDone;
}

// --------------------------------------- in-wave load balancing of the search
//
// A wave's queries need very different amounts of work, and a wave lives
// as long as its busiest lane.  Here every lane owns one query but works on a
// task: its own query, or a subtree of another lane's query taken over when
// it has nothing left to do.  After each round of leaf scans the idle lanes
// are paired (by rank, via wave ballots) with lanes that still hold pending
// second children, and each such donor hands over its shallowest pending
// subtree (root node, box bound, query, owner) through lane shuffles.  The
// best key of each query lives in LDS (okey); workers merge into it with a
// 64-bit atomic minimum and prune with it, so every worker of a query
// shares the best found so far.  The answer is the minimum key over a
// superset of the leaves the single-lane search must scan, hence the same
// exact, unique result.  Everything is wave-synchronous: lanes never wait on
// each other, and the loop ends once no lane holds a task.
constexpr uint32_t kNoOwner = 0xFFFFFFFFu;
#ifndef KDNN_DONATE_DEEPEST
#define KDNN_DONATE_DEEPEST 0
#endif
// Give pending subtrees away only once the task's query has a candidate (0:
// never gate), in launches whose waves start about half idle:
// KDNN_DONATE_GATE_Q <= queries per wave < KDNN_P1_Q_SPLIT.  There the idle
// lanes would otherwise take far subtrees during the first descents and
// search them with nothing to prune.  Measured against no gate: Scene fused
// kernel (33 per wave) 36.2 -> 35.6 us, its nn_query search 30.8 -> 29.9 us;
// fuller waves lost (Stress 1M leaf 8, 64 per wave: 213 -> 219 us; the LiDAR
// batch, 43 per wave: 7.93 -> 8.03 ms) and so did a 1,024-point launch of 8
// per wave, so those stay ungated.
#ifndef KDNN_DONATE_GATE_Q
#define KDNN_DONATE_GATE_Q 24
#endif
#ifndef KDNN_P1_HANDOVER
#define KDNN_P1_HANDOVER 1
#endif
// Leaf-round quorum (in 64ths of the busy lanes) for waves that own 64
// queries: an internal-node phase ends once that share of the busy lanes waits
// at a leaf, instead of when all of them do; lanes still descending sit the
// leaf round out and go on after it.  Measured: uniform Stress 1M (leaf 8)
// 327 -> 295 us at 48, the 131k LiDAR frame 3% faster; waves that start with
// idle lanes (single-round launches, fewer than 64 queries) lost 1-5%, so they
// keep the full quorum.
#ifndef KDNN_LEAF_QUORUM_FULL
#define KDNN_LEAF_QUORUM_FULL 48
#endif
#ifndef KDNN_XFER_LDS
#define KDNN_XFER_LDS 1
#endif
#ifndef KDNN_QLDS
#define KDNN_QLDS 1  // query coordinates in LDS (wave_search QL) where the kernel allows
#endif
// Idle lanes that trigger a hand-over inside the internal-node phase: 8 when
// a wave starts with many idle lanes (fewer than KDNN_P1_Q_SPLIT queries per
// wave), 24 when it starts (nearly) full.  Measured: Scene ICP (33 per wave)
// with searches from the root best at 14-20; since the searches start at a
// leaf (warm start, point location), 8: warm fused kernel 24.4 -> 23.5 us
// (mean of three A/B pairs; 16, 12, 4 and 24+ measured too), nn_query 26.1 ->
// 25.4 us.  The 131k LiDAR frame's fused kernel (43 per wave) 39.9 -> 38.2 us
// at 24, Skewed 500k (64 per wave) -2.5%, uniform Stress 1M -1.5%.
#ifndef KDNN_P1_MIN_IDLE_FULL
#define KDNN_P1_MIN_IDLE_FULL 24
#endif
#ifndef KDNN_P1_Q_SPLIT
#define KDNN_P1_Q_SPLIT 40
#endif
#ifndef KDNN_P1_MIN_IDLE
#define KDNN_P1_MIN_IDLE 8
#endif

// Position of the r-th (0-based) set bit of m (m has more than r set bits).
__device__ __forceinline__ uint32_t nth_set_bit(uint64_t m, uint32_t r)
{
    uint32_t pos = 0;
#pragma unroll
    for (int w = 32; w >= 1; w >>= 1) {
        const uint32_t c = uint32_t(__popcll(m & ((uint64_t(1) << w) - 1u)));
        if (r >= c) {
            r -= c;
            m >>= w;
            pos += uint32_t(w);
        }
    }
    return pos;
}

// Per-lane state of the balanced search.
struct WaveTask {
    uint32_t owner;  // slot of the query this lane works for (kNoOwner: idle)
    float qx, qy, qz;
    uint64_t key;    // best key seen by this lane for that query
    uint32_t i;      // node being processed (kDone: task finished)
    uint32_t pend;   // pending second children, per path level
    uint32_t cn, cp;
    uint32_t nt;     // instrumented search: visits recorded so far (trace_visit)
};

// A finished task publishes its best (and counts) to the owner's slot.
template <bool STATS>
__device__ __forceinline__ void task_finish(WaveTask &w, unsigned long long *okey, uint32_t *ocn,
                                            uint32_t *ocp)
{
    if (w.i == kDone && w.owner != kNoOwner) {
        atomicMin(&okey[w.owner], (unsigned long long)w.key);
        if (STATS) {
            atomicAdd(&ocn[w.owner], w.cn);
            atomicAdd(&ocp[w.owner], w.cp);
            w.cn = 0u;
            w.cp = 0u;
        }
        w.owner = kNoOwner;
    }
}

// The instrumented search's visit stream, one row per query: 0 for the root's
// box, an internal node i for the run of its two children's boxes, a leaf
// node for that leaf's points, kPlaneVisit | leaf for that leaf's plane
// record and kSiblingVisit | v for the box of node v alone (both read by a
// warm start), kLocateVisit | i for node i's split plane (read by the point
// location of a search from the root).  Visits beyond the row's tcap entries
// are counted, not stored.
constexpr uint32_t kSiblingVisit = 0x80000000u;
constexpr uint32_t kPlaneVisit = 0x40000000u;
constexpr uint32_t kLocateVisit = 0x20000000u;
__device__ __forceinline__ void trace_visit(WaveTask &w, uint32_t *trow, uint32_t tcap,
                                            uint32_t e)
{
    if (trow && w.nt < tcap) trow[w.nt] = e;
    ++w.nt;
}

// Hand-over round: idle lanes take the shallowest pending subtree of busy
// lanes, paired by rank.  Every lane of the wave must call it together.
// xfer: this wave's 64-entry LDS table (donor rank -> donor lane).
// need_cand: only tasks whose best key holds a candidate give work away.
template <bool QL = false>
__device__ __forceinline__ void task_handover(WaveTask &w, const float *lbs,
                                              const unsigned long long *okey, uint32_t *xfer,
                                              uint32_t min_idle = 1u, bool need_cand = false)
{
    const uint32_t lane = threadIdx.x & 63u;
    const uint64_t below = (uint64_t(1) << lane) - 1u;
    const bool idle = w.owner == kNoOwner;
    const uint64_t idle_m = __ballot(idle);
    if (idle_m == 0 || uint32_t(__popcll(idle_m)) < min_idle) return;
    const uint32_t dep = idle ? 0u : 31u - uint32_t(__clz(int(w.i)));
    const bool hold = idle || (need_cand && uint32_t(w.key) == 0xFFFFFFFFu);
    const uint32_t avail = hold ? 0u : (w.pend & ((1u << dep) - 1u));
    const uint64_t don_m = __ballot(avail != 0u);
    if (don_m == 0) return;
    const uint32_t nidle = uint32_t(__popcll(idle_m)), ndon = uint32_t(__popcll(don_m));
    const uint32_t np = nidle < ndon ? nidle : ndon;
    const bool gives = avail != 0u && uint32_t(__popcll(don_m & below)) < np;
    uint32_t gv = 0u;
    float glb = 0.0f;
    if (gives) {
#if KDNN_DONATE_DEEPEST
        const uint32_t h = 31u - uint32_t(__clz(int(avail)));  // deepest pending level
#else
        const uint32_t h = uint32_t(__ffs(int(avail))) - 1u;  // shallowest pending level
#endif
        glb = lbs[h * kWG];
        gv = (w.i >> (dep - h - 1u)) ^ 1u;
        w.pend &= ~(1u << h);
    }
    const uint32_t trank = uint32_t(__popcll(idle_m & below));
    const bool takes = idle && trank < np;
#if KDNN_XFER_LDS
    // the donor of rank r publishes its lane in slot r; the taker of rank r reads it
    if (gives) xfer[__popcll(don_m & below)] = lane;
    __builtin_amdgcn_wave_barrier();
    const int src = takes ? int(xfer[trank]) : int(lane);
#else
    const int src = takes ? int(nth_set_bit(don_m, trank)) : int(lane);
#endif
    const uint32_t tv = uint32_t(__shfl(int(gv), src, 64));
    const float tlb = __shfl(glb, src, 64);
    const uint32_t town = uint32_t(__shfl(int(w.owner), src, 64));
    if constexpr (!QL) {  // QL: the query's coordinates are read from LDS by owner
        const float tqx = __shfl(w.qx, src, 64);
        const float tqy = __shfl(w.qy, src, 64);
        const float tqz = __shfl(w.qz, src, 64);
        if (takes) {
            w.qx = tqx;
            w.qy = tqy;
            w.qz = tqz;
        }
    }
    if (takes) {
        w.owner = town;
        w.pend = 0u;
        w.key = okey[town];
        w.i = enters(tlb, key_dist(w.key)) ? tv : kDone;
    }
}

// Point location: the leaf whose cell holds the query, found by the split
// planes of its ancestors (node i's split value and axis, the last 8 bytes of
// its 32-byte record), one dependent 8-byte load per level -- the levels
// below the LDS copy (next) shared by the wave's lanes and cached.  A search
// without a start leaf of
// its own (the first ICP iteration, nn_query) starts there as a warm start
// would (below): the same exact answer as a descent from the root, whose
// child-pair runs (three 16-byte loads per level, each lane's own lines below
// the top) and box-bounded backtracking it replaces.  Measured (search
// kernels, MI355X): nn_query Scene 30.2 -> 26.5 us, Stress 1M leaf 8 213 ->
// 148 us, Skewed 500k leaf 16 168 -> 157 us; the first ICP iteration's fused
// kernel, Scene 33.3 -> 30.4 us, the 131k LiDAR frames ~47 -> ~39 us.
// The planes of the top KDNN_TOP_LOC_LEVELS levels are read from a copy each
// work-group keeps in LDS (top; null: none), staged once per launch
// (stage_top_planes): every lane's first dependent loads become LDS reads
// (Scene nn_query search 26.3 -> 25.5 us, Stress 1M leaf 8 156 -> 152 us,
// Skewed 500k leaf 16 156 -> 154 us; 10 levels: no better).
// STATS: each plane read from memory counts as one node record (traced
// kLocateVisit | i); the LDS reads are not memory records.
constexpr uint32_t kTopLocEnd = 1u << KDNN_TOP_LOC_LEVELS;  // nodes [1, kTopLocEnd)

// A work-group's copy of the top levels' (split, axis) pairs, entry i for
// node i (entry 0 unused); all threads call it together.
__device__ __forceinline__ void stage_top_planes(const TreeView &t, float2 *top)
{
    const float2 *const sa = reinterpret_cast<const float2 *>(t.nodes) + 3;
    const uint32_t lim = t.first_leaf < kTopLocEnd ? t.first_leaf : kTopLocEnd;
    for (uint32_t j = threadIdx.x; j < lim; j += kWG)
        if (j >= 1u) top[j] = sa[4 * size_t(j)];
    __syncthreads();
}

template <bool STATS>
__device__ __forceinline__ uint32_t locate_leaf(const TreeView &t, float qx, float qy, float qz,
                                                WaveTask &w, uint32_t *trow, uint32_t tcap,
                                                const float2 *top = nullptr)
{
    const float2 *const sa = reinterpret_cast<const float2 *>(t.nodes) + 3;
    uint32_t i = 1u;
    if (top) {
        const uint32_t lim = t.first_leaf < kTopLocEnd ? t.first_leaf : kTopLocEnd;
        while (i < lim) {
            const float2 S = top[i];
            const uint32_t ax = __float_as_uint(S.y);
            const float qa = ax == 0u ? qx : (ax == 1u ? qy : qz);
            i = 2u * i + (qa > S.x ? 1u : 0u);
        }
    }
    while (i < t.first_leaf) {
        const float2 S = sa[4 * size_t(i)];
        if constexpr (STATS) {
            ++w.cn;
            trace_visit(w, trow, tcap, kLocateVisit | i);
        }
        const uint32_t ax = __float_as_uint(S.y);
        const float qa = ax == 0u ? qx : (ax == 1u ? qy : qz);
        i = 2u * i + (qa > S.x ? 1u : 0u);  // left points <= split
    }
    return i;
}

// Warm start of a task at `leaf` (a heap index in [2^D, 2^(D+1)); the ICP
// loop passes the leaf that held the query's match in the previous
// iteration, usually at or next to the new one).  The subtrees beside the
// leaf's path -- the sibling of its ancestor at every depth 0 .. D-1 -- cover
// the rest of the tree, so the task begins as if it had descended to the
// leaf: it scans the leaf, each sibling is pending under a lower bound of its
// distance (lbs, one level per ancestor depth) while that bound lets it in,
// and the walk goes on exactly as after a descent, visiting pending subtrees
// deepest first.  The result is the same as from the root.
//
// The bounds come from the ancestors' split planes.  The sibling below the
// depth-d ancestor lies wholly on the far side of that ancestor's plane (left
// points <= split <= right points), and its box's near face along the split
// axis lies at or beyond the plane: the squared gap between the query and
// that face, when the query is on the leaf's side of it, bounds every point
// of the sibling from below; computed as fl(gap)^2 it is also no larger than
// the rounded squared distance of any such point (each rounding step is
// monotone), so pruning with it drops no point that could tie or win.  (An
// empty sibling's face is at infinity: never entered.)  The faces of the
// deepest kPathLevels ancestors' siblings sit in the leaf's 64-byte plane
// record, one cache line loaded in the same round trip as the leaf's points;
// the siblings' boxes would take a line each, and a scattered gather costs
// about a line fetch per lane whatever its width (Scene, warm searches of the
// ICP loop: 25.1 -> 24.2 us with the split values themselves; the 131k LiDAR
// frames 24.9 -> 22.3 us; the same planes read from the 32-byte node records,
// a line each, measured no faster than the boxes).  The face prunes more than
// the split: Scene (host simulation) 0.71 siblings entered per query with the
// splits, 0.63 with the faces, 0.60 with the whole boxes.  Shallower levels
// (trees deeper than kPathLevels) load their sibling boxes, kWarmBatch at a
// time: those sit near the root, shared by the wave's lanes.  A one-axis
// bound is looser than the box, so a sibling may be entered that its box
// would have kept out; its children's boxes are tested as usual.
// STATS: the plane record counts as two node records (64 bytes; traced as one
// kPlaneVisit entry for the leaf), each sibling box as one.
#ifndef KDNN_WARM_BATCH
#define KDNN_WARM_BATCH 4
#endif
constexpr int kWarmBatch = KDNN_WARM_BATCH;
template <bool STATS, int CH>
__device__ __forceinline__ void warm_start(const TreeView &t, uint32_t leaf, float qx, float qy,
                                           float qz, float *lbs, WaveTask &w, uint32_t *trow,
                                           uint32_t tcap, unsigned long long *okey_own)
{
    const uint32_t D = uint32_t(t.depth);
    int32_t begin, last, end;
    leaf_range(t, leaf, begin, last, end);
    float4 p[CH];
    const float4 *pc = t.pts + begin;
#pragma unroll
    for (int c = 0; c < CH; ++c) p[c] = pc[c];
    const uint4 *const pr = t.paths + 4 * size_t(leaf - t.first_leaf);
    uint4 R[kPathWords / 4];
#pragma unroll
    for (int v = 0; v < kPathWords / 4; ++v) R[v] = pr[v];
    uint64_t key = w.key;
    for (uint32_t k0 = uint32_t(begin);;) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const float dx = p[c].x - qx;
            const float dy = p[c].y - qy;
            const float dz = p[c].z - qz;
            const float dd = (dx * dx + dy * dy) + dz * dz;
            const uint64_t k = nn_key(dd, __float_as_uint(p[c].w));
            key = k < key ? k : key;
        }
        k0 += CH;
        if (k0 >= uint32_t(end)) break;
        pc = t.pts + k0;
#pragma unroll
        for (int c = 0; c < CH; ++c) p[c] = pc[c];
    }
    if constexpr (STATS) {
        w.cp += uint32_t(end - begin);
        trace_visit(w, trow, tcap, leaf);
        w.cn += 2;
        trace_visit(w, trow, tcap, kPlaneVisit | leaf);
    }
    const float best = key_dist(key);
    uint32_t pend = 0u;
    const uint32_t axes = R[0].x;
#pragma unroll
    for (int k = 0; k < kPathLevels; ++k) {
        // the ancestor at depth d = D-1-k: record word 1+k
        const int d = int(D) - 1 - k;
        if (d >= 0) {
            const uint4 Rv = R[(k + 1) / 4];
            const uint32_t wv = (k + 1) % 4 == 0 ? Rv.x : (k + 1) % 4 == 1 ? Rv.y
                                : (k + 1) % 4 == 2 ? Rv.z : Rv.w;
            const float face = __uint_as_float(wv);
            const uint32_t ax = (axes >> (2 * k)) & 3u;
            const float qa = ax == 0u ? qx : (ax == 1u ? qy : qz);
            // the leaf's side: right child of its depth-d ancestor (the
            // sibling's points then lie at or below its face, else at or above)
            const bool right = ((leaf >> k) & 1u) != 0u;
            const float gap = right ? qa - face : face - qa;
            const float lb = gap > 0.0f ? gap * gap : 0.0f;
            lbs[d * kWG] = lb;
            pend |= enters(lb, best) ? (1u << d) : 0u;
        }
    }
    // levels above the record: their sibling boxes
    for (int d0 = int(D) - 1 - kPathLevels; d0 >= 0; d0 -= kWarmBatch) {
        float4 P[kWarmBatch][2];
#pragma unroll
        for (int u = 0; u < kWarmBatch; ++u) {
            const uint32_t d = uint32_t(d0 - u < 0 ? 0 : d0 - u);
            const uint32_t parent = leaf >> (D - d);
            const uint32_t odd = ((leaf >> (D - d - 1u)) & 1u) ^ 1u;
            const float4 *pb = t.boxes + 3 * size_t(parent) + odd;
            P[u][0] = pb[0];
            P[u][1] = pb[1];
        }
#pragma unroll
        for (int u = 0; u < kWarmBatch; ++u) {
            const int d = d0 - u;
            if (d >= 0) {
                const bool odd = (((leaf >> (D - uint32_t(d) - 1u)) & 1u) ^ 1u) != 0u;
                const float4 A = odd ? make_float4(P[u][0].z, P[u][0].w, P[u][1].x, P[u][1].y)
                                     : P[u][0];
                const float4 B = odd ? make_float4(P[u][1].z, P[u][1].w, 0.0f, 0.0f)
                                     : make_float4(P[u][1].x, P[u][1].y, 0.0f, 0.0f);
                const float lb = box_lb(qx, qy, qz, A, B);
                lbs[d * kWG] = lb;
                pend |= enters(lb, best) ? (1u << d) : 0u;
                if constexpr (STATS) {
                    ++w.cn;
                    trace_visit(w, trow, tcap,
                                kSiblingVisit | ((leaf >> (D - uint32_t(d) - 1u)) ^ 1u));
                }
            }
        }
    }
    const uint64_t seen = atomicMin(okey_own, (unsigned long long)key);
    w.key = seen < key ? seen : key;
    w.pend = pend;
    w.i = pair_next(leaf, w.pend, lbs, key_dist(w.key));
}

// The pending-bound array of a balanced-search work-group (one float per path
// level and lane): a static array of kDevMaxDepth levels, or (DYN) dynamic LDS
// of lbs_bytes(D) sized to the tree, which leaves room for more resident
// groups where registers allow them (the 8-point leaf batches, the batched
// kernel).  The 16-point kernels keep the static array: their occupancy is
// set by registers, and they measured faster in that form.
template <bool DYN>
__device__ __forceinline__ float *lbs_array()
{
    if constexpr (DYN) {
        extern __shared__ float lbs_dyn[];
        return lbs_dyn;
    } else {
        __shared__ float lbs_static[kDevMaxDepth * kWG];
        return lbs_static;
    }
}

// All lanes of the wave must call this together.  okey / ocn / ocp: the
// work-group's LDS arrays [kWG], slot threadIdx.x = this lane's own query.
// On return okey[threadIdx.x] holds the answer key of this lane's query (the
// bound key when there is none), ocn / ocp its node / point counts (STATS).
// BALANCE == false: no hand-over, every lane searches its own query alone
// (the plain single-lane pair search; its counts are the method's own work,
// independent of which queries share a wave).
// CH: leaf points loaded per batch (kLeafChunk, or kLeafChunkSmall for a tree
// whose leaves hold at most that many: fewer registers, more resident waves).
// QL: the queries' coordinates live in qpool (LDS, one float4 per owner slot)
// and each step reads its task's from there, instead of every task carrying
// them in registers: a hand-over moves the owner only, and the loop carries
// three registers fewer (which the compiler otherwise merges by copies).
// trow / tcap / tcnt (STATS only, each lane its own query's): the row its
// visits are recorded in (trace_visit), its capacity, and where the number of
// visits goes (null: none recorded).
// hint (this lane's own query; 0: none): the leaf to start from (warm_start);
// without one the search starts at the leaf whose cell holds the query
// (locate_leaf).
template <bool STATS, bool BALANCE = true, int CH = kLeafChunk, bool QL = false>
__device__ __forceinline__ void wave_search(const TreeView &t, bool own, float oqx, float oqy,
                                            float oqz, uint64_t init, float *lbs,
                                            unsigned long long *okey, uint32_t *ocn,
                                            uint32_t *ocp, uint32_t *xfer, uint32_t quorum = 64u,
                                            float4 *qpool = nullptr, uint32_t wq = 64u,
                                            uint32_t *trow = nullptr, uint32_t tcap = 0u,
                                            uint32_t *tcnt = nullptr, uint32_t hint = 0u,
                                            const float2 *top = nullptr)
{
    const uint32_t p1_idle = wq < KDNN_P1_Q_SPLIT ? KDNN_P1_MIN_IDLE : KDNN_P1_MIN_IDLE_FULL;
    const bool need_cand = KDNN_DONATE_GATE_Q > 0 && wq >= uint32_t(KDNN_DONATE_GATE_Q) &&
                           wq < uint32_t(KDNN_P1_Q_SPLIT);
    okey[threadIdx.x] = init;
    if constexpr (QL) qpool[threadIdx.x] = make_float4(oqx, oqy, oqz, 0.0f);
    if (STATS) {
        ocn[threadIdx.x] = 0u;
        ocp[threadIdx.x] = 0u;
    }
    WaveTask w;
    w.owner = own ? threadIdx.x : kNoOwner;
    w.qx = oqx;
    w.qy = oqy;
    w.qz = oqz;
    w.key = init;
    w.i = kDone;
    w.pend = 0u;
    w.cn = 0u;
    w.cp = 0u;
    w.nt = 0u;
    if (own && isfinite(oqx) && isfinite(oqy) && isfinite(oqz)) {
        // the start leaf: the hint, else the query's own leaf
        const uint32_t start =
            hint != 0u ? hint : locate_leaf<STATS>(t, oqx, oqy, oqz, w, trow, tcap, top);
        warm_start<STATS, CH>(t, start, oqx, oqy, oqz, lbs, w, trow, tcap, &okey[threadIdx.x]);
    }
    for (;;) {
        // Phase 1: internal nodes, as in the single-lane pair search; lanes
        // that run out of work take some over on every pass.
        while (__ballot(w.i < t.first_leaf) != 0) {
            if (quorum < 64u) {
                // start the leaf round once enough of the busy lanes wait at a leaf
                const uint32_t at_leaf =
                    uint32_t(__popcll(__ballot(w.i != kDone && w.i >= t.first_leaf)));
                const uint32_t busy = uint32_t(__popcll(__ballot(w.i != kDone)));
                if (at_leaf * 64u >= busy * quorum) break;
            }
            if (w.i < t.first_leaf) {
                // the two children's boxes: one 48-byte run, three loads
                const uint32_t i = w.i;
                // one address, the three loads at immediate offsets 0, 16, 32
                const float4 *const pb = t.boxes + 3 * size_t(i);
                const float4 P0 = pb[0];
                const float4 P1 = pb[1];
                const float4 P2 = pb[2];
                const float4 A0 = P0;
                const float4 B0 = make_float4(P1.x, P1.y, 0.0f, 0.0f);
                const float4 A1 = make_float4(P1.z, P1.w, P2.x, P2.y);
                const float4 B1 = make_float4(P2.z, P2.w, 0.0f, 0.0f);
                if constexpr (STATS) {
                    w.cn += 2;
                    trace_visit(w, trow, tcap, i);
                }
                float qx = w.qx, qy = w.qy, qz = w.qz;
                if constexpr (QL) {
                    const float4 q = qpool[w.owner];
                    qx = q.x;
                    qy = q.y;
                    qz = q.z;
                }
                const float l0 = box_lb(qx, qy, qz, A0, B0);
                const float l1 = box_lb(qx, qy, qz, A1, B1);
                const bool swap = l1 < l0;
                const float lf = swap ? l1 : l0, ls = swap ? l0 : l1;
                const float best = key_dist(w.key);
                const uint32_t d = 31u - uint32_t(__clz(int(i)));
                if (enters(lf, best)) {
                    lbs[d * kWG] = ls;
                    w.pend = enters(ls, best) ? (w.pend | (1u << d)) : (w.pend & ~(1u << d));
                    w.i = 2 * i + (swap ? 1u : 0u);
                } else {
                    w.i = pair_next(i, w.pend, lbs, best);
                }
            }
            task_finish<STATS>(w, okey, ocn, ocp);
            if (BALANCE && KDNN_P1_HANDOVER)
                task_handover<QL>(w, lbs, okey, xfer, p1_idle, need_cand);
        }
        // Phase 2: leaves, then share the improved best of the query.
        if (w.i != kDone && w.i >= t.first_leaf) {
            int32_t begin, last, end;
            leaf_range(t, w.i, begin, last, end);
            uint32_t k0 = uint32_t(begin);
            uint64_t key = w.key;
            float qx = w.qx, qy = w.qy, qz = w.qz;
            if constexpr (QL) {
                const float4 q = qpool[w.owner];
                qx = q.x;
                qy = q.y;
                qz = q.z;
            }
            do {
                const float4 *pc = t.pts + k0;
                float4 p[CH];
#pragma unroll
                for (int c = 0; c < CH; ++c) p[c] = pc[c];
#pragma unroll
                for (int c = 0; c < CH; ++c) {
                    const float dx = p[c].x - qx;
                    const float dy = p[c].y - qy;
                    const float dz = p[c].z - qz;
                    const float dd = (dx * dx + dy * dy) + dz * dz;
                    const uint64_t k = nn_key(dd, __float_as_uint(p[c].w));
                    key = k < key ? k : key;
                }
                k0 += CH;
            } while (k0 < uint32_t(end));
            if constexpr (STATS) {
                w.cp += uint32_t(end - begin);
                trace_visit(w, trow, tcap, w.i);
            }
            const uint64_t seen = atomicMin(&okey[w.owner], (unsigned long long)key);
            w.key = seen < key ? seen : key;
            w.i = pair_next(w.i, w.pend, lbs, key_dist(w.key));
        }
        task_finish<STATS>(w, okey, ocn, ocp);
        if (__ballot(w.owner != kNoOwner) == 0) break;
        if (BALANCE) task_handover<QL>(w, lbs, okey, xfer, 1u, need_cand);
    }
    // without hand-overs (STATS) the lane did all of its own query's visits
    if constexpr (STATS)
        if (tcnt) *tcnt = w.nt;
}

struct NnArgs {
    TreeView tree;
    uint64_t init;    // bound key (bound +inf: none)
    uint32_t budget;  // pass-1 node budget (two-pass mode)
    const float *q;
    int64_t m;
    const int32_t *perm;
    int32_t *idx;
    float *d2;
    uint32_t *cnt_nodes;
    uint32_t *cnt_pts;
    bool spread;  // one-lane-per-query kernel: spread_pos
    uint32_t wq;  // one-lane-per-query kernel: queries per wave (1..64)
    uint32_t *trace;   // instrumented one-lane kernel: [m][tcap] visit rows, or null
    uint32_t *tcount;  // [m] visits of each query (may exceed tcap)
    uint32_t tcap;
    const uint32_t *hint;  // instrumented one-lane kernel: [m] warm-start leaves (0: none), or null
};

// Cooperative search of one query by G >= 2 lanes.
template <int G, bool STATS>
__device__ __forceinline__ void search_query(const TreeView &t, float qx, float qy, float qz,
                                             uint64_t init, Best &b, uint32_t &cn, uint32_t &cp)
{
    uint64_t key = init;
    uint32_t slot = 0;
    if (isfinite(qx) && isfinite(qy) && isfinite(qz))
        nn_search_group<G, STATS>(t, qx, qy, qz, false, key, slot, cn, cp);
    finish(key, slot, b);
}

// One query per lane (G = 1: the balanced wave search) or G lanes per query.
// A block handles kWG / G queries per sweep; the loop bound is uniform over the
// block so a wave's (or group's) lanes always stay together.
// QL: the query coordinates in LDS (wave_search QL); more LDS per group, so
// used for one-round launches only, where the groups fit anyway.
template <int G, bool STATS, int CH = kLeafChunk, bool QL = false>
__global__ __launch_bounds__(kWG) void nn_kernel(NnArgs a)
{
    constexpr int QPB = kWG / G;
    const uint32_t nb = gridDim.x;
    const uint32_t blk = xcd_remap(blockIdx.x, nb);
    if constexpr (G == 1) {
        float *const lbs = lbs_array<CH == kLeafChunkSmall>();
        __shared__ unsigned long long okey[kWG];
        __shared__ uint32_t ocn[STATS ? kWG : 1], ocp[STATS ? kWG : 1];
        __shared__ uint32_t xfer[kWG];
        __shared__ float4 qpool[QL ? kWG : 1];
        // the top planes for point location, in LDS (the instrumented kernel
        // too: its counts and records are the memory loads of the search)
        constexpr bool kTop = KDNN_TOP_LOC_LEVELS > 0;
        __shared__ float2 top[kTop ? kTopLocEnd : 1];
        if constexpr (kTop) stage_top_planes(a.tree, top);
        const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
        const uint32_t wq = a.wq;
        const int64_t QB = int64_t(kWG / 64) * wq;
        for (int64_t base = int64_t(blk) * QB; base < a.m; base += int64_t(nb) * QB) {
            const int64_t k = base + int64_t(wv) * wq + lane;
            const bool own = uint32_t(lane) < wq && k < a.m;
            const int64_t pos = own ? spread_pos(a.spread, wq, k, blk, base, nb, a.m) : k;
            const int64_t i = own ? (a.perm ? int64_t(a.perm[pos]) : pos) : 0;
            const float qx = own ? a.q[3 * i] : 0.0f;
            const float qy = own ? a.q[3 * i + 1] : 0.0f;
            const float qz = own ? a.q[3 * i + 2] : 0.0f;
            // the instrumented kernel counts (and may record) the single-lane
            // search of each query
            const bool tr = STATS && own && a.trace;
            uint32_t hint = STATS && own && a.hint ? a.hint[i] : 0u;
            hint = hint >= a.tree.first_leaf && hint < 2u * a.tree.first_leaf ? hint : 0u;
            wave_search<STATS, !STATS, CH, QL>(a.tree, own, qx, qy, qz, a.init,
                                               lbs + threadIdx.x, okey, ocn, ocp,
                                               xfer + (threadIdx.x & ~63u),
                                               wq == kQFull ? KDNN_LEAF_QUORUM_FULL : 64u, qpool,
                                               wq, tr ? a.trace + size_t(i) * a.tcap : nullptr,
                                               a.tcap, tr ? a.tcount + i : nullptr, hint,
                                               kTop ? top : nullptr);
            if (own) {
                Best b;
                finish(okey[threadIdx.x], 0u, b);
                a.idx[i] = b.idx;
                a.d2[i] = b.d;
                if (STATS) {
                    if (a.cnt_nodes) a.cnt_nodes[i] = ocn[threadIdx.x];
                    if (a.cnt_pts) a.cnt_pts[i] = ocp[threadIdx.x];
                }
            }
        }
    } else {
        const int gl = threadIdx.x & (G - 1);
        for (int64_t base = int64_t(blk) * QPB; base < a.m; base += int64_t(nb) * QPB) {
            const int64_t k = base + threadIdx.x / G;
            if (k < a.m) {
                const int64_t i = a.perm ? int64_t(a.perm[k]) : k;
                const float qx = a.q[3 * i], qy = a.q[3 * i + 1], qz = a.q[3 * i + 2];
                Best b;
                uint32_t cn = 0, cp = 0;
                search_query<G, STATS>(a.tree, qx, qy, qz, a.init, b, cn, cp);
                if (gl == 0) {
                    a.idx[i] = b.idx;
                    a.d2[i] = b.d;
                    if (STATS) {
                        if (a.cnt_nodes) a.cnt_nodes[i] = cn;
                        if (a.cnt_pts) a.cnt_pts[i] = cp;
                    }
                }
            }
        }
    }
}

// ---------------------------------------- persistent search, top levels in LDS
//
// One work-group of kPWG lanes per CU.  It first copies the node records of
// the top L levels (heap indices 1 .. 2^L - 1, 32 bytes each, L <= 12 so at
// most 128 KB) into LDS, then walks a contiguous slice of the (Morton
// ordered) queries, one lane per query; node fetches above depth L hit LDS
// instead of L2, which removes most of the descent's memory round trips.
constexpr int kPWG = 512;
constexpr int kLdsMaxLevels = 12;

__device__ __forceinline__ void stage_top_levels(const TreeView &t, float4 *lds, uint32_t lds_first)
{
    for (uint32_t j = 2 + threadIdx.x; j < 2 * lds_first; j += blockDim.x) lds[j] = t.nodes[j];
    __syncthreads();
}

template <bool STATS>
__global__ __launch_bounds__(kPWG) void nn_persist_kernel(NnArgs a, uint32_t lds_first)
{
    extern __shared__ float4 lds_nodes[];
    stage_top_levels(a.tree, lds_nodes, lds_first);
    const int64_t chunk = (a.m + gridDim.x - 1) / gridDim.x;
    const int64_t k0 = int64_t(blockIdx.x) * chunk;
    const int64_t k1 = k0 + chunk < a.m ? k0 + chunk : a.m;
    for (int64_t k = k0 + threadIdx.x; k < k1; k += kPWG) {
        const int64_t i = a.perm ? int64_t(a.perm[k]) : k;
        uint64_t key;
        uint32_t slot, cn = 0, cp = 0;
        nn_search<STATS>(a.tree, a.q[3 * i], a.q[3 * i + 1], a.q[3 * i + 2], a.init, kNoBudget,
                         key, slot, cn, cp, lds_nodes, lds_first);
        Best b;
        finish(key, slot, b);
        a.idx[i] = b.idx;
        a.d2[i] = b.d;
        if (STATS) {
            if (a.cnt_nodes) a.cnt_nodes[i] = cn;
            if (a.cnt_pts) a.cnt_pts[i] = cp;
        }
    }
}

// ------------------------------------------------------------ two-pass search
//
// Opt-in schedule (a node budget in the flags).  A launch lasts as long as
// its slowest waves, the ones holding queries that need a wide search.
// Pass 1 gives every query one lane and a budget of node records; most
// queries finish.  The slots left unfinished are compacted, per work-group
// and in lane order, into a list.  Pass 2 hands list entry e to group
// e mod (number of groups) of kPass2Lanes lanes, which completes the query
// with the cooperative search starting from pass 1's best.  Every step is a
// fixed function of the input, so the ICP sums are reproducible.
// nn_query keeps an unfinished query's state in its own outputs:
// idx = -(best index + 3) (so <= -2) and dist2 = best distance so far.
constexpr int kPass2Lanes = 16;
constexpr int kPass1MaxBlocks = 4096;
constexpr int kPass2Blocks = 256;

// Rank of this lane among the lanes of the work-group whose flag is set,
// in lane order; *total = number of flagged lanes.  Whole group must call.
__device__ __forceinline__ uint32_t block_rank(bool flag, uint32_t *wcount, uint32_t &total)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const uint64_t bal = __ballot(flag);
    const uint32_t in_wave = uint32_t(__popcll(bal & ((uint64_t(1) << lane) - 1u)));
    if (lane == 0) wcount[w] = uint32_t(__popcll(bal));
    __syncthreads();
    uint32_t before = 0;
    total = 0;
    for (int ww = 0; ww < kWG / 64; ++ww) {
        before += ww < w ? wcount[ww] : 0u;
        total += wcount[ww];
    }
    __syncthreads();
    return before + in_wave;
}

// pre[0..nb] = exclusive prefix sums of counts[0..nb) (pre[nb] = total).
__device__ __forceinline__ void load_prefix(const uint32_t *counts, int32_t nb, uint32_t *pre)
{
    __shared__ uint32_t wsum[kWG / 64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    uint32_t carry = 0;
    for (int32_t b0 = 0; b0 < nb; b0 += kWG) {
        const int32_t b = b0 + threadIdx.x;
        const uint32_t v = b < nb ? counts[b] : 0u;
        uint32_t x = v;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const uint32_t y = __shfl_up(x, off, 64);
            if (lane >= off) x += y;
        }
        if (lane == 63) wsum[w] = x;
        __syncthreads();
        uint32_t before = 0, tot = 0;
        for (int ww = 0; ww < kWG / 64; ++ww) {
            before += ww < w ? wsum[ww] : 0u;
            tot += wsum[ww];
        }
        if (b < nb) pre[b] = carry + before + x - v;
        carry += tot;
        __syncthreads();
    }
    if (threadIdx.x == 0) pre[nb] = carry;
    __syncthreads();
}

// The work-group b holding list entry e: largest b with pre[b] <= e.
__device__ __forceinline__ int32_t entry_block(const uint32_t *pre, int32_t nb, uint32_t e)
{
    int32_t lo = 0, hi = nb - 1;
    while (lo < hi) {
        const int32_t mid = (lo + hi + 1) >> 1;
        if (pre[mid] <= e)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

struct TwoPass {
    int32_t *list;     // [nb1 * cap] slots left by pass 1, per work-group segment
    uint32_t *counts;  // [nb1]
    int32_t nb1;       // pass-1 work-groups
    int32_t cap;       // slots per work-group segment
};

template <bool STATS>
__global__ __launch_bounds__(kWG) void nn_pass1_kernel(NnArgs a, TwoPass tp)
{
    __shared__ uint32_t wcount[kWG / 64];
    int32_t *seg = tp.list + int64_t(blockIdx.x) * tp.cap;
    uint32_t run = 0;
    const int64_t stride = int64_t(gridDim.x) * kWG;
    for (int64_t base = int64_t(blockIdx.x) * kWG; base < a.m; base += stride) {
        const int64_t k = base + threadIdx.x;
        bool hard = false;
        if (k < a.m) {
            const int64_t i = a.perm ? int64_t(a.perm[k]) : k;
            uint64_t key;
            uint32_t slot, cn = 0, cp = 0;
            const bool done = nn_search<STATS>(a.tree, a.q[3 * i], a.q[3 * i + 1], a.q[3 * i + 2],
                                               a.init, a.budget, key, slot, cn, cp);
            Best b;
            finish(key, slot, b);
            a.idx[i] = done ? b.idx : -(int32_t(uint32_t(key)) + 3);
            a.d2[i] = done ? b.d : key_dist(key);
            if (STATS) {
                if (a.cnt_nodes) a.cnt_nodes[i] = cn;
                if (a.cnt_pts) a.cnt_pts[i] = cp;
            }
            hard = !done;
        }
        uint32_t tot;
        const uint32_t r = block_rank(hard, wcount, tot);
        if (hard) seg[run + r] = int32_t(k);
        run += tot;
    }
    if (threadIdx.x == 0) tp.counts[blockIdx.x] = run;
}

template <bool STATS>
__global__ __launch_bounds__(kWG) void nn_pass2_kernel(NnArgs a, TwoPass tp)
{
    constexpr int G = kPass2Lanes;
    __shared__ uint32_t pre[kPass1MaxBlocks + 1];
    load_prefix(tp.counts, tp.nb1, pre);
    const uint32_t H = pre[tp.nb1];
    const uint32_t ng = gridDim.x * (kWG / G);
    const int gl = threadIdx.x & (G - 1);
    for (uint32_t e = blockIdx.x * (kWG / G) + threadIdx.x / G; e < H; e += ng) {
        const int32_t b = entry_block(pre, tp.nb1, e);
        const int64_t k = tp.list[int64_t(b) * tp.cap + (e - pre[b])];
        const int64_t i = a.perm ? int64_t(a.perm[k]) : k;
        const int32_t enc = a.idx[i];
        uint64_t key = nn_key(a.d2[i], uint32_t(-enc - 3));
        uint32_t slot = 0, cn = 0, cp = 0;
        nn_search_group<G, STATS>(a.tree, a.q[3 * i], a.q[3 * i + 1], a.q[3 * i + 2], true, key,
                                  slot, cn, cp);
        if (gl == 0) {
            Best bb;
            finish(key, slot, bb);
            a.idx[i] = bb.idx;
            a.d2[i] = bb.d;
            if (STATS) {
                if (a.cnt_nodes) a.cnt_nodes[i] += cn;
                if (a.cnt_pts) a.cnt_pts[i] += cp;
            }
        }
    }
}

// ------------------------------------------------------ fused ICP kernel
//
// Per source point: q = fl32(R s + t) evaluated in fp64 with a fixed
// association; nearest target point m; accumulate in fp64, shifted by c,
//   (s-c), (m-c), (s-c)(m-c)^T, d2, 1.
// Per lane -> wave (reduce-scatter, one component per lane pair) -> work-group (waves
// summed in order) -> per-group partials; reduce_partials_kernel then sums
// the partials in a fixed order.  The result does not depend on scheduling.
struct Rt12 {  // 12 doubles by value (kernel argument)
    double v[12];
};

struct IcpArgs {
    TreeView tree;
    const float *src;
    int64_t n;
    const int32_t *perm;
    double R[9];
    double t[3];
    double c[3];
    double *partials;   // [kS][nb] of the kernel that reduces (single pass / pass 1)
    double *partials2;  // [kS][nb2] of pass 2
    int32_t nb1;        // pass-1 block count (two-pass mode)
    double *sums;       // [kS]
    uint32_t budget;    // pass-1 node budget
    uint64_t *pkey;     // [n] pass-1 best key of unfinished slots
    uint32_t *pslot;    // [n] pass-1 best point slot of unfinished slots
    int32_t *idx;
    float *d2;
    uint64_t init;      // bound key (bound +inf: none)
    int32_t *mslot;     // [n] or null: original index of each source point's match, -1 if none
    float *md2;         // [n] or null: its squared distance
    bool spread;        // one-lane-per-query kernel: spread_pos
    uint32_t wq;        // one-lane-per-query kernel: queries per wave (1..64)
    const double *rt_dev;  // one-lane-per-query kernel, device loop: (R, t) here, not in R / t
    const uint32_t *stop;  // the same: nonzero = the loop has stopped, do nothing
    // one-lane-per-query kernel: per source point, the heap index of the leaf
    // that held its match (0: none) -- written after the search when non-null,
    // and read before it as a warm start (wave_search hint) when hint_in
    uint32_t *hint;
    bool hint_in;
};

__device__ __forceinline__ float rigid_row(double r0, double r1, double r2, double tr, double x,
                                           double y, double z)
{
    return float(((r0 * x + r1 * y) + r2 * z) + tr);
}

// ---- wave sums of the kS fp64 components: a reduce-scatter over the lanes
//
// Summing each of the kS components over the wave by its own log2(64)-step
// butterfly moves every component through every step (~500 VALU instructions
// per wave).  A reduce-scatter halves the number of values a lane carries at
// each step: at a step, a lane pairs with a partner lane in the other half of
// its group, keeps one of two components (its half decides which), receives
// the partner's copy of that same component and adds it.  Steps: the upper
// and lower 32 lanes (permlane32 swap), the odd and even rows of 16 lanes
// (permlane16 swap), then within a row the mirror pairs l <-> 15 - l, the
// half-row mirror pairs l <-> 7 - l, and lanes l <-> l ^ 2, l <-> l ^ 1 (DPP).
// kS = 17 values -> 9 -> 5 -> 3 -> 2 -> 1: ~90 instructions.  Each output is
// a fixed sum tree over the 64 lanes, the same in every run.

// (a, b) -> (half of the lanes: a + partner's a, the rest: b + partner's b)
// through a permlane swap; `tag` says which (0: a, 1: b) this lane now holds.
template <bool ROWS16>
__device__ __forceinline__ double swap_step(double a, double b, uint32_t &tag)
{
    const uint64_t ba = uint64_t(__double_as_longlong(a)), bb = uint64_t(__double_as_longlong(b));
    uint32_t alo = uint32_t(ba), ahi = uint32_t(ba >> 32), blo = uint32_t(bb), bhi = uint32_t(bb >> 32);
    uint32_t ta = 0u, tb = 1u;
    if constexpr (ROWS16) {
        const auto l = __builtin_amdgcn_permlane16_swap(alo, blo, false, false);
        const auto h = __builtin_amdgcn_permlane16_swap(ahi, bhi, false, false);
        const auto t = __builtin_amdgcn_permlane16_swap(ta, tb, false, false);
        alo = l[0]; blo = l[1]; ahi = h[0]; bhi = h[1]; ta = t[0];
    } else {
        const auto l = __builtin_amdgcn_permlane32_swap(alo, blo, false, false);
        const auto h = __builtin_amdgcn_permlane32_swap(ahi, bhi, false, false);
        const auto t = __builtin_amdgcn_permlane32_swap(ta, tb, false, false);
        alo = l[0]; blo = l[1]; ahi = h[0]; bhi = h[1]; ta = t[0];
    }
    tag = ta;  // both registers now hold parts of the same component
    return __longlong_as_double((long long)((uint64_t(ahi) << 32) | alo)) +
           __longlong_as_double((long long)((uint64_t(bhi) << 32) | blo));
}

template <int CTRL>
__device__ __forceinline__ double dpp_mov(double v)
{
    const uint64_t b = uint64_t(__double_as_longlong(v));
    const uint32_t lo = uint32_t(__builtin_amdgcn_mov_dpp(int(uint32_t(b)), CTRL, 0xF, 0xF, false));
    const uint32_t hi = uint32_t(__builtin_amdgcn_mov_dpp(int(uint32_t(b >> 32)), CTRL, 0xF, 0xF, false));
    return __longlong_as_double((long long)((uint64_t(hi) << 32) | lo));
}

// Within-row step with a symmetric DPP pairing that crosses lane bit `hi`:
// the lower lane keeps a (+ partner's a), the upper one b (+ partner's b).
template <int CTRL>
__device__ __forceinline__ double row_step(double a, double b, bool hi)
{
    const double send = hi ? a : b;
    const double keep = hi ? b : a;
    return keep + dpp_mov<CTRL>(send);
}

constexpr int kDppRowMirror = 0x140, kDppRowHalfMirror = 0x141;
constexpr int kDppXor2 = 0x4E, kDppXor1 = 0xB1;  // quad_perm [2,3,0,1], [1,0,3,2]

// On return v = the sum over the 64 lanes of component c (the return value;
// c >= kS: padding, no component).  Lanes l and l ^ 1 return the same c and
// v.  Every lane of the wave must call it together.
__device__ __forceinline__ int wave_scatter_sums(const double (&acc)[kS], double &v)
{
    static_assert(kS == 17, "the step sequence below is laid out for 17 components");
    const uint32_t lane = threadIdx.x & 63u;
    uint32_t t32 = 0u, t16 = 0u;
    double v1[9], v2[5], v3[3], v4[2];
#pragma unroll
    for (int j = 0; j < 9; ++j) v1[j] = swap_step<false>(acc[2 * j], 2 * j + 1 < kS ? acc[2 * j + 1] : 0.0, t32);
#pragma unroll
    for (int k = 0; k < 5; ++k) v2[k] = swap_step<true>(v1[2 * k], 2 * k + 1 < 9 ? v1[2 * k + 1] : 0.0, t16);
    const bool b3 = lane & 8u, b2 = lane & 4u, b1 = lane & 2u;
#pragma unroll
    for (int k = 0; k < 3; ++k) v3[k] = row_step<kDppRowMirror>(v2[2 * k], 2 * k + 1 < 5 ? v2[2 * k + 1] : 0.0, b3);
#pragma unroll
    for (int k = 0; k < 2; ++k) v4[k] = row_step<kDppRowHalfMirror>(v3[2 * k], 2 * k + 1 < 3 ? v3[2 * k + 1] : 0.0, b2);
    const double v5 = row_step<kDppXor2>(v4[0], v4[1], b1);
    v = v5 + dpp_mov<kDppXor1>(v5);
    // v1[j] holds component 2j + t32, v2[k] = v1[2k + t16], v3[k] = v2[2k + b3], ...
    return 16 * int(b1) + 8 * int(b2) + 4 * int(b3) + 2 * int(t16) + int(t32);
}

// Sum acc[] over a work-group of WG lanes (all active); thread c < kS gets
// component c in out[c * out_stride] (fixed order: lanes by wave_scatter_sums,
// then waves in order).  acc[] is left holding partial sums.
template <int WG>
__device__ __forceinline__ void block_sum_n(double (&acc)[kS], double *red /* LDS [waves][kS] */,
                                            double *out, int64_t out_stride)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    double v;
    const int cw = wave_scatter_sums(acc, v);
    if (cw < kS && !(lane & 1)) red[w * kS + cw] = v;
    __syncthreads();
    if (threadIdx.x < kS) {
        double s = 0.0;
        for (int ww = 0; ww < WG / 64; ++ww) s += red[ww * kS + threadIdx.x];
        out[threadIdx.x * out_stride] = s;
    }
}

__device__ __forceinline__ void block_sum(double (&acc)[kS], double *red, double *out,
                                          int64_t out_stride)
{
    block_sum_n<kWG>(acc, red, out, out_stride);
}

// The query of source point i: q = fl32(R s + t), fp64 with a fixed association.
__device__ __forceinline__ void icp_query(const IcpArgs &a, int64_t i, double &X, double &Y,
                                          double &Z, float &qx, float &qy, float &qz)
{
    X = a.src[3 * i];
    Y = a.src[3 * i + 1];
    Z = a.src[3 * i + 2];
    qx = rigid_row(a.R[0], a.R[1], a.R[2], a.t[0], X, Y, Z);
    qy = rigid_row(a.R[3], a.R[4], a.R[5], a.t[1], X, Y, Z);
    qz = rigid_row(a.R[6], a.R[7], a.R[8], a.t[2], X, Y, Z);
}

// The same with (R, t) read from device memory (the device-side ICP loop).
__device__ __forceinline__ void icp_query_dev(const double *__restrict__ rt,
                                              const float *__restrict__ src, int64_t i, double &X,
                                              double &Y, double &Z, float &qx, float &qy,
                                              float &qz)
{
    X = src[3 * i];
    Y = src[3 * i + 1];
    Z = src[3 * i + 2];
    qx = rigid_row(rt[0], rt[1], rt[2], rt[9], X, Y, Z);
    qy = rigid_row(rt[3], rt[4], rt[5], rt[10], X, Y, Z);
    qz = rigid_row(rt[6], rt[7], rt[8], rt[11], X, Y, Z);
}

// Record a finished pair: optional per-point outputs, then the fp64 sums
// (s - c), (m - c), (s - c)(m - c)^T, d2, 1.
__device__ __forceinline__ void icp_accumulate(const IcpArgs &a, int64_t i, double X, double Y,
                                               double Z, const Best &b, double (&acc)[kS])
{
    if (a.idx) a.idx[i] = b.idx;
    if (a.d2) a.d2[i] = b.d;
    if (a.mslot) {
        a.mslot[i] = b.idx;
        a.md2[i] = b.d;
    }
    if (b.idx < 0) return;
    const float4 mp = a.tree.pts[a.tree.slot_of[b.idx]];
    const double s0 = X - a.c[0], s1 = Y - a.c[1], s2 = Z - a.c[2];
    const double m0 = double(mp.x) - a.c[0], m1 = double(mp.y) - a.c[1],
                 m2 = double(mp.z) - a.c[2];
    acc[0] += s0; acc[1] += s1; acc[2] += s2;
    acc[3] += m0; acc[4] += m1; acc[5] += m2;
    acc[6] += s0 * m0; acc[7] += s0 * m1; acc[8] += s0 * m2;
    acc[9] += s1 * m0; acc[10] += s1 * m1; acc[11] += s1 * m2;
    acc[12] += s2 * m0; acc[13] += s2 * m1; acc[14] += s2 * m2;
    acc[15] += double(b.d);
    acc[16] += 1.0;
}

// Sums of per-work-group partials, in a separate launch: one work-group adds
// the columns of p1 (n1 of them) and then of p2 (n2) in a fixed order and
// writes the KDNN_SUMS_DOUBLES totals to out.  The kernel boundary makes the
// partials visible; a last-work-group ticket inside the producing kernel
// would need a device-scope release in every work-group, which on MI355X
// writes back the L2 of its XCD (the L2s are not coherent with each other).
// With stat (residual rejection): stat_out = (stat[0] / stat[1], stat[2]).
// done (optional): after the sums (and stat_out) are written and made visible
// at system scope, seq is stored there, so a host polling that word of pinned
// memory knows the sums are complete without waiting for the stream.
// WG lanes: one per partial column in a single pass (1024 up to 1024 columns;
// 256 for a few columns, cheaper to start); more columns loop.
template <int WG>
__global__ __launch_bounds__(WG) void reduce_partials_kernel(const double *p1, int32_t n1,
                                                             const double *p2, int32_t n2,
                                                             double *out, const double *stat,
                                                             double *stat_out, uint64_t *done,
                                                             uint64_t seq)
{
    __shared__ double red[(WG / 64) * kS];
    double acc[kS];
#pragma unroll
    for (int c = 0; c < kS; ++c) acc[c] = 0.0;
    for (int32_t g = threadIdx.x; g < n1 + n2; g += WG) {
#pragma unroll
        for (int c = 0; c < kS; ++c)
            acc[c] += g < n1 ? p1[int64_t(c) * n1 + g] : p2[int64_t(c) * n2 + (g - n1)];
    }
    block_sum_n<WG>(acc, red, out, 1);
    if (stat && stat_out && threadIdx.x == 0) {
        stat_out[0] = stat[0] / stat[1];
        stat_out[1] = stat[2];
    }
    if (done) {
        if (threadIdx.x < kS) __threadfence_system();
        __syncthreads();
        if (threadIdx.x == 0)
            __hip_atomic_store(done, seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
    }
}

#ifndef KDNN_RED_WG
#define KDNN_RED_WG 512
#endif
static void launch_reduce_partials(const double *p1, int32_t n1, const double *p2, int32_t n2,
                                   double *out, const double *stat, double *stat_out,
                                   uint64_t *done, uint64_t seq, hipStream_t s)
{
    if (n1 + n2 <= kWG || KDNN_RED_WG == kWG)
        reduce_partials_kernel<kWG><<<1, kWG, 0, s>>>(p1, n1, p2, n2, out, stat, stat_out, done,
                                                      seq);
    else
        reduce_partials_kernel<KDNN_RED_WG><<<1, KDNN_RED_WG, 0, s>>>(p1, n1, p2, n2, out, stat,
                                                                      stat_out, done, seq);
}

// ------------------------------------------- ICP iterations on the device
//
// One iteration = the fused kernel (transform from st->rt, search, partials)
// + icp_loop_step_kernel (one work-group): the partials summed in the same
// fixed order as reduce_partials_kernel, then on one lane the rigid solve,
// the convergence rule (|MSE_k - MSE_{k-1}| < eps on two consecutive
// iterations, as the host loop applies it) and the next transform.  A failed
// solve keeps the last good transform and sets stop; so does convergence.
// Once stop is set the remaining launches of the queue return at once.
// The per-iteration record (E_k, the transform used) stays in device memory;
// the host copies it once the registration has run (a store to host memory
// would hold up each step kernel's completion by a PCIe round trip).
__global__ __launch_bounds__(64) void icp_loop_init_kernel(IcpLoopState *st, IcpLoopOut *out,
                                                           Rt12 rt0)
{
    if (threadIdx.x != 0) return;
    for (int k = 0; k < 12; ++k) {
        st->rt[k] = rt0.v[k];
        out->rt[k] = rt0.v[k];
    }
    st->prev_mse = 0.0;
    st->small = 0;
    st->stop = 0u;
    out->iters = 0;
    out->status = 0;
    out->fail_iter = -1;
    out->fail_phase = 0;
    out->stopped = 0;
    st->mse = 0.0;
}

// One lane: record E_k and the transform used, solve, and advance the loop
// state (mode as IcpLoop::mode).  tot: the iteration's (or the kept pairs')
// 17 sums; rt_used: the transform this iteration searched with.
__device__ __forceinline__ void loop_finish(const double *tot, IcpLoopState *st, IcpLoopOut *out,
                                            int32_t k, double eps, const double *c, int32_t mode,
                                            const double (&rt_used)[12])
{
    const double n = tot[16], E = tot[15];
    if (mode != 2 && k >= 0 && k < kLoopMaxIter) {  // the host never launches beyond the record
        out->E[k] = E;
        for (int j = 0; j < 12; ++j) out->rt_hist[k][j] = rt_used[j];
    }
    double R[9], t[3];
    const int32_t rs = rigid_from_sums(&tot[0], &tot[3], &tot[6], n, c, R, t);
    if (rs != kRigidOk) {
        out->status = rs;
        out->fail_iter = k;
        out->fail_phase = mode == 2 ? 1 : 0;
        out->stopped = 1;
        st->stop = 1u;
        return;
    }
    if (mode == 1) {  // first solve of a rejection iteration: the residuals use it
        for (int j = 0; j < 9; ++j) st->rt1[j] = R[j];
        for (int j = 0; j < 3; ++j) st->rt1[9 + j] = t[j];
        st->mse = E / n;
        return;
    }
    for (int j = 0; j < 9; ++j) {
        st->rt[j] = R[j];
        out->rt[j] = R[j];
    }
    for (int j = 0; j < 3; ++j) {
        st->rt[9 + j] = t[j];
        out->rt[9 + j] = t[j];
    }
    out->iters = k + 1;
    const double mse = mode == 2 ? st->mse : E / n;  // the first pass's, as the host loop
    if (eps > 0.0 && k > 0) {
        st->small = fabs(mse - st->prev_mse) < eps ? st->small + 1 : 0;
        if (st->small >= 2) {
            st->stop = 1u;
            out->stopped = 1;
        }
    }
    st->prev_mse = mse;
}

template <int WG>
__global__ __launch_bounds__(WG) void icp_loop_step_kernel(const double *p, int32_t np,
                                                           IcpLoopState *st, IcpLoopOut *out,
                                                           int32_t k, double eps, Rt12 c,
                                                           int32_t mode)
{
    __shared__ double red[(WG / 64) * kS];
    __shared__ double tot[kS];
    // the state's words are read up front, in the shadow of the partials'
    // loads (a stopped loop sums stale partials and then discards them)
    const uint32_t stopped = st->stop;
    double rt_used[12];
    if (threadIdx.x == 0)
        for (int j = 0; j < 12; ++j) rt_used[j] = st->rt[j];
    double acc[kS];
#pragma unroll
    for (int j = 0; j < kS; ++j) acc[j] = 0.0;
    for (int32_t g = threadIdx.x; g < np; g += WG) {
#pragma unroll
        for (int j = 0; j < kS; ++j) acc[j] += p[int64_t(j) * np + g];
    }
    block_sum_n<WG>(acc, red, tot, 1);
    __syncthreads();
    if (threadIdx.x != 0 || stopped) return;
    loop_finish(tot, st, out, k, eps, c.v, mode, rt_used);
}

hipError_t launch_icp_loop_init(IcpLoopState *state, IcpLoopOut *out, const double *R0,
                                const double *t0, hipStream_t s)
{
    Rt12 rt0;
    for (int k = 0; k < 9; ++k) rt0.v[k] = R0[k];
    for (int k = 0; k < 3; ++k) rt0.v[9 + k] = t0[k];
    icp_loop_init_kernel<<<1, 64, 0, s>>>(state, out, rt0);
    return hipGetLastError();
}

static void launch_icp_loop_step(const double *p, int32_t np, const IcpLoop &L,
                                 const double *center, hipStream_t s)
{
    Rt12 c{};
    for (int k = 0; k < 3; ++k) c.v[k] = center[k];
    if (np <= kWG || KDNN_RED_WG == kWG)
        icp_loop_step_kernel<kWG><<<1, kWG, 0, s>>>(p, np, L.state, L.out, L.iter, L.eps, c,
                                                    L.mode);
    else
        icp_loop_step_kernel<KDNN_RED_WG><<<1, KDNN_RED_WG, 0, s>>>(p, np, L.state, L.out,
                                                                     L.iter, L.eps, c, L.mode);
}

// Single pass, one kernel: transform, search (balanced wave search for G = 1,
// G lanes per point otherwise) and the fp64 reduction.
// Occupancy: the one-lane-per-query kernels hold the queries' coordinates in
// LDS (wave_search QL), 36 KB per group with the 16-point kernel's static
// bound array, so 4 groups per CU (one-round launches use at most 3); the
// registers are held to what that occupancy allows.  The 8-point kernels
// (bound array sized to the tree) keep 5 waves per SIMD: the reduce-scatter's
// 17 live sums would otherwise take them past the register budget of 5.
#ifndef KDNN_FUSED_WPE
#define KDNN_FUSED_WPE 5
#endif
// WARM (one lane per query): the instance that starts searches from a.hint
// (hint_in); the other one searches from the root and has the warm start's
// registers to spare (only its own hints are written).
template <int G, int CH = kLeafChunk, bool WARM = false>
__global__ __launch_bounds__(kWG) __attribute__((amdgpu_waves_per_eu(
    G == 1 && CH == kLeafChunk && KDNN_QLDS ? 4 : KDNN_FUSED_WPE))) void
icp_fused_kernel(IcpArgs a)
{
    __shared__ double red[(kWG / 64) * kS];
    const uint32_t nb = gridDim.x;
    const uint32_t blk = xcd_remap(blockIdx.x, nb);
    if constexpr (G == 1) {
        // One lane owns each source point; the wave balances the searches.
        // Each sweep's pairs are summed over the wave at once and added to the
        // wave's row of red (by the lanes the reduce-scatter leaves a component
        // in), so no sums stay live in registers across the next search.
        float *const lbs = lbs_array<CH == kLeafChunkSmall>();
        __shared__ unsigned long long okey[kWG];
        __shared__ uint32_t xfer[kWG];
        __shared__ float4 qpool[KDNN_QLDS ? kWG : 1];
        constexpr bool kTop = !WARM && KDNN_TOP_LOC_LEVELS > 0;  // searches all locate
        __shared__ float2 top[kTop ? kTopLocEnd : 1];
        const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
        if (a.stop && *a.stop) return;  // device loop already stopped (uniform)
        if constexpr (kTop) stage_top_planes(a.tree, top);
        if (lane == 63) {
#pragma unroll
            for (int c = 0; c < kS; ++c) red[wv * kS + c] = 0.0;
        }
        const uint32_t wq = a.wq;
        const int64_t QB = int64_t(kWG / 64) * wq;
        for (int64_t base = int64_t(blk) * QB; base < a.n; base += int64_t(nb) * QB) {
            const int64_t k = base + int64_t(wv) * wq + lane;
            const bool own = uint32_t(lane) < wq && k < a.n;
            const int64_t pos = own ? spread_pos(a.spread, wq, k, blk, base, nb, a.n) : k;
            const int64_t i = own ? (a.perm ? int64_t(a.perm[pos]) : pos) : 0;
            float qx = 0.0f, qy = 0.0f, qz = 0.0f;
            if (own) {
                double X, Y, Z;
                if (a.rt_dev)
                    icp_query_dev(a.rt_dev, a.src, i, X, Y, Z, qx, qy, qz);
                else
                    icp_query(a, i, X, Y, Z, qx, qy, qz);
            }
            // the leaf of the point's previous match, checked to be a leaf
            uint32_t hint = WARM && own && a.hint_in ? a.hint[i] : 0u;
            hint = hint >= a.tree.first_leaf && hint < 2u * a.tree.first_leaf ? hint : 0u;
            wave_search<false, true, CH, KDNN_QLDS>(a.tree, own, qx, qy, qz, a.init,
                                                    lbs + threadIdx.x, okey, nullptr, nullptr,
                                                    xfer + (threadIdx.x & ~63u),
                                                    wq == kQFull ? KDNN_LEAF_QUORUM_FULL : 64u,
                                                    qpool, wq, nullptr, 0u, nullptr, hint,
                                                    kTop ? top : nullptr);
            double acc[kS];
#pragma unroll
            for (int c = 0; c < kS; ++c) acc[c] = 0.0;
            if (own) {
                Best b;
                finish(okey[threadIdx.x], 0u, b);
                // the source point again (cheaper than keeping it in registers)
                const double X = a.src[3 * i], Y = a.src[3 * i + 1], Z = a.src[3 * i + 2];
                icp_accumulate(a, i, X, Y, Z, b, acc);
                if (a.hint)
                    a.hint[i] = b.idx >= 0 ? leaf_of_slot(a.tree, uint32_t(a.tree.slot_of[b.idx]))
                                           : 0u;
            }
            double v;
            const int cw = wave_scatter_sums(acc, v);
            if (cw < kS && !(lane & 1)) red[wv * kS + cw] += v;
        }
        __syncthreads();
        if (threadIdx.x < kS) {
            double s = 0.0;
            for (int ww = 0; ww < kWG / 64; ++ww) s += red[ww * kS + threadIdx.x];
            a.partials[int64_t(threadIdx.x) * nb + blockIdx.x] = s;
        }
    } else {
        double acc[kS];
#pragma unroll
        for (int c = 0; c < kS; ++c) acc[c] = 0.0;
        constexpr int QPB = kWG / G;
        const int gl = threadIdx.x & (G - 1);
        for (int64_t base = int64_t(blk) * QPB; base < a.n; base += int64_t(nb) * QPB) {
            const int64_t k = base + threadIdx.x / G;
            if (k >= a.n) continue;
            const int64_t i = a.perm ? int64_t(a.perm[k]) : k;
            double X, Y, Z;
            float qx, qy, qz;
            icp_query(a, i, X, Y, Z, qx, qy, qz);
            Best b;
            uint32_t cn = 0, cp = 0;
            search_query<G, false>(a.tree, qx, qy, qz, a.init, b, cn, cp);
            if (gl == 0) icp_accumulate(a, i, X, Y, Z, b, acc);
        }
        block_sum(acc, red, a.partials + blockIdx.x, nb);
    }
}

// Two-pass mode, pass 1: one lane per point with a node budget; unfinished
// slots keep their best so far and are compacted into the pass-2 list.
__global__ __launch_bounds__(kWG) void icp_pass1_kernel(IcpArgs a, TwoPass tp)
{
    __shared__ double red[(kWG / 64) * kS];
    __shared__ uint32_t wcount[kWG / 64];
    double acc[kS];
#pragma unroll
    for (int c = 0; c < kS; ++c) acc[c] = 0.0;
    int32_t *seg = tp.list + int64_t(blockIdx.x) * tp.cap;
    uint32_t run = 0;
    const int64_t stride = int64_t(gridDim.x) * kWG;
    for (int64_t base = int64_t(blockIdx.x) * kWG; base < a.n; base += stride) {
        const int64_t k = base + threadIdx.x;
        bool hard = false;
        if (k < a.n) {
            const int64_t i = a.perm ? int64_t(a.perm[k]) : k;
            double X, Y, Z;
            float qx, qy, qz;
            icp_query(a, i, X, Y, Z, qx, qy, qz);
            uint64_t key;
            uint32_t slot, cn = 0, cp = 0;
            const bool done =
                nn_search<false>(a.tree, qx, qy, qz, a.init, a.budget, key, slot, cn, cp);
            if (done) {
                Best b;
                finish(key, slot, b);
                icp_accumulate(a, i, X, Y, Z, b, acc);
            } else {
                a.pkey[k] = key;
                a.pslot[k] = slot;
            }
            hard = !done;
        }
        uint32_t tot;
        const uint32_t r = block_rank(hard, wcount, tot);
        if (hard) seg[run + r] = int32_t(k);
        run += tot;
    }
    if (threadIdx.x == 0) tp.counts[blockIdx.x] = run;
    block_sum(acc, red, a.partials + blockIdx.x, gridDim.x);
}

// Two-pass mode, pass 2: groups of kPass2Lanes complete the listed points
// and write their partials after pass 1's.
__global__ __launch_bounds__(kWG) void icp_pass2_kernel(IcpArgs a, TwoPass tp)
{
    constexpr int G = kPass2Lanes;
    __shared__ double red[(kWG / 64) * kS];
    __shared__ uint32_t pre[kPass1MaxBlocks + 1];
    load_prefix(tp.counts, tp.nb1, pre);
    const uint32_t H = pre[tp.nb1];
    const uint32_t ng = gridDim.x * (kWG / G);
    const int gl = threadIdx.x & (G - 1);
    double acc[kS];
#pragma unroll
    for (int c = 0; c < kS; ++c) acc[c] = 0.0;
    for (uint32_t e = blockIdx.x * (kWG / G) + threadIdx.x / G; e < H; e += ng) {
        const int32_t b = entry_block(pre, tp.nb1, e);
        const int64_t k = tp.list[int64_t(b) * tp.cap + (e - pre[b])];
        const int64_t i = a.perm ? int64_t(a.perm[k]) : k;
        double X, Y, Z;
        float qx, qy, qz;
        icp_query(a, i, X, Y, Z, qx, qy, qz);
        uint64_t key = a.pkey[k];
        uint32_t slot = a.pslot[k], cn = 0, cp = 0;
        nn_search_group<G, false>(a.tree, qx, qy, qz, true, key, slot, cn, cp);
        if (gl == 0) {
            Best bb;
            finish(key, slot, bb);
            icp_accumulate(a, i, X, Y, Z, bb, acc);
        }
    }
    block_sum(acc, red, a.partials2 + blockIdx.x, gridDim.x);
}

// Persistent single-lane correspondence kernel with the top levels in LDS.
__global__ __launch_bounds__(kPWG) void icp_persist_kernel(IcpArgs a, uint32_t lds_first)
{
    extern __shared__ float4 lds_nodes[];
    __shared__ double red[(kPWG / 64) * kS];
    stage_top_levels(a.tree, lds_nodes, lds_first);
    double acc[kS];
#pragma unroll
    for (int c = 0; c < kS; ++c) acc[c] = 0.0;
    const int64_t chunk = (a.n + gridDim.x - 1) / gridDim.x;
    const int64_t k0 = int64_t(blockIdx.x) * chunk;
    const int64_t k1 = k0 + chunk < a.n ? k0 + chunk : a.n;
    for (int64_t k = k0 + threadIdx.x; k < k1; k += kPWG) {
        const int64_t i = a.perm ? int64_t(a.perm[k]) : k;
        double X, Y, Z;
        float qx, qy, qz;
        icp_query(a, i, X, Y, Z, qx, qy, qz);
        uint64_t key;
        uint32_t slot, cn = 0, cp = 0;
        nn_search<false>(a.tree, qx, qy, qz, a.init, kNoBudget, key, slot, cn, cp, lds_nodes,
                         lds_first);
        Best b;
        finish(key, slot, b);
        icp_accumulate(a, i, X, Y, Z, b, acc);
    }
    block_sum_n<kPWG>(acc, red, a.partials + blockIdx.x, gridDim.x);
}

// ------------------------------------------------- batched ICP (frame pairs)
//
// Several registrations advance in lock-step: one launch runs the fused
// correspondence step of up to kBatchMax (source, tree) pairs.  Work-groups
// are dealt round-robin to the 8 XCDs, so work-group b runs on XCD b % 8;
// pair p of a launch with B pairs gets the XCDs x with x % B == p.  Every XCD
// then walks a single tree, which stays in its own L2 (a 131k-point frame
// tree is ~2.6 MB of the 4 MB), instead of all of them thrashing it.  Each
// pair's work-group partials are then summed in a fixed order into its 17
// sums (batch_reduce_kernel, one work-group per pair).
constexpr int kBatchMax = 8;

struct BatchPair {
    TreeView tree;
    const float *src;
    int64_t n;
    double R[9];
    double t[3];
    double c[3];
    int32_t nb;       // work-groups of this pair: ceil(n / kWG)
    int32_t part;     // first partial column of this pair
    double *sums;     // [kS] out
    uint64_t *done;   // null, or a word set to the launch's sequence number after the sums
    IcpLoopState *st; // device loop: the pair's state ((R, t) from here), else null
    IcpLoopOut *out;  // device loop: the pair's record
    uint32_t *hint;   // null, or per source point the leaf of its match (written after the
    bool hint_in;     // search; read before it as a warm start when hint_in)
};

struct BatchArgs {
    BatchPair p[kBatchMax];
    int32_t B;
    int32_t total;    // partial columns (stride of one component)
    uint64_t init;    // bound key
    double *partials; // [kS][total]
    uint64_t seq;     // value stored into each pair's done word
    int32_t iter;     // device loop: iteration index
    double eps;       // device loop: convergence threshold
};

#ifndef KDNN_BATCH_QUORUM
#define KDNN_BATCH_QUORUM KDNN_LEAF_QUORUM_FULL
#endif
template <int CH, bool WARM = false>  // WARM: as icp_fused_kernel's
__global__ __launch_bounds__(kWG) void icp_batch_kernel(BatchArgs a)
{
    __shared__ double red[(kWG / 64) * kS];
    float *const lbs = lbs_array<true>();
    const int x = int(blockIdx.x % uint32_t(kNumXcd));
    const int pi = x % a.B;
    const BatchPair &P = a.p[pi];
    const int kx = (kNumXcd - pi + a.B - 1) / a.B;  // XCDs serving this pair
    const int32_t j = int32_t(blockIdx.x / uint32_t(kNumXcd)) * kx + x / a.B;
    if (j >= P.nb) return;  // uniform over the work-group
    if (P.st && P.st->stop) return;  // the pair's device loop has stopped (uniform)
    double acc[kS];
#pragma unroll
    for (int c = 0; c < kS; ++c) acc[c] = 0.0;
    __shared__ unsigned long long okey[kWG];
    __shared__ uint32_t xfer[kWG];
    const int64_t i = int64_t(j) * kWG + threadIdx.x;
    const bool own = i < P.n;
    double X = 0.0, Y = 0.0, Z = 0.0;
    float qx = 0.0f, qy = 0.0f, qz = 0.0f;
    if (own) {
        if (P.st) {
            icp_query_dev(P.st->rt, P.src, i, X, Y, Z, qx, qy, qz);
        } else {
            X = P.src[3 * i];
            Y = P.src[3 * i + 1];
            Z = P.src[3 * i + 2];
            qx = rigid_row(P.R[0], P.R[1], P.R[2], P.t[0], X, Y, Z);
            qy = rigid_row(P.R[3], P.R[4], P.R[5], P.t[1], X, Y, Z);
            qz = rigid_row(P.R[6], P.R[7], P.R[8], P.t[2], X, Y, Z);
        }
    }
    uint32_t hint = WARM && own && P.hint_in ? P.hint[i] : 0u;
    hint = hint >= P.tree.first_leaf && hint < 2u * P.tree.first_leaf ? hint : 0u;
    wave_search<false, true, CH>(P.tree, own, qx, qy, qz, a.init, lbs + threadIdx.x, okey,
                                 nullptr, nullptr, xfer + (threadIdx.x & ~63u),
                                 KDNN_BATCH_QUORUM, nullptr, 64u, nullptr, 0u, nullptr, hint);
    if (own) {
        Best b;
        finish(okey[threadIdx.x], 0u, b);
        if (P.hint)
            P.hint[i] = b.idx >= 0 ? leaf_of_slot(P.tree, uint32_t(P.tree.slot_of[b.idx])) : 0u;
        if (b.idx >= 0) {
            const float4 mp = P.tree.pts[P.tree.slot_of[b.idx]];
            const double s0 = X - P.c[0], s1 = Y - P.c[1], s2 = Z - P.c[2];
            const double m0 = double(mp.x) - P.c[0], m1 = double(mp.y) - P.c[1],
                         m2 = double(mp.z) - P.c[2];
            acc[0] = s0; acc[1] = s1; acc[2] = s2;
            acc[3] = m0; acc[4] = m1; acc[5] = m2;
            acc[6] = s0 * m0; acc[7] = s0 * m1; acc[8] = s0 * m2;
            acc[9] = s1 * m0; acc[10] = s1 * m1; acc[11] = s1 * m2;
            acc[12] = s2 * m0; acc[13] = s2 * m1; acc[14] = s2 * m2;
            acc[15] = double(b.d);
            acc[16] = 1.0;
        }
    }
    block_sum(acc, red, a.partials + P.part + j, a.total);
}

// Work-group p: the sums of pair p from its work-groups' partial columns.
// Device loop (P.st set): the pair's step instead -- sums into LDS, then the
// rigid solve and the loop state on one lane, as icp_loop_step_kernel.
__global__ __launch_bounds__(kWG) void batch_reduce_kernel(BatchArgs a)
{
    __shared__ double red[(kWG / 64) * kS];
    __shared__ double tot[kS];
    const BatchPair &P = a.p[blockIdx.x];
    const uint32_t stopped = P.st ? P.st->stop : 0u;
    double rt_used[12];
    if (P.st && threadIdx.x == 0)
        for (int j = 0; j < 12; ++j) rt_used[j] = P.st->rt[j];
    double acc[kS];
#pragma unroll
    for (int c = 0; c < kS; ++c) acc[c] = 0.0;
    for (int32_t g = threadIdx.x; g < P.nb; g += kWG) {
#pragma unroll
        for (int c = 0; c < kS; ++c) acc[c] += a.partials[int64_t(c) * a.total + P.part + g];
    }
    if (P.st) {
        block_sum(acc, red, tot, 1);
        __syncthreads();
        if (threadIdx.x == 0 && !stopped)
            loop_finish(tot, P.st, P.out, a.iter, a.eps, P.c, 0, rt_used);
        return;
    }
    block_sum(acc, red, P.sums, 1);
    if (P.done) {  // sums visible at system scope first (polled from the host)
        if (threadIdx.x < kS) __threadfence_system();
        __syncthreads();
        if (threadIdx.x == 0)
            __hip_atomic_store(P.done, a.seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
    }
}

// ------------------------------------------- residual rejection (3 sigma)
//
// After the first solve (R1, t1) of an iteration, with the matches the fused
// kernel stored per source point:
//   icp_residual_kernel: r_i^2 = ||R1 s_i + t1 - m_i||^2 in fp64 (the moved
//     point is not rounded), summed over the pairs with their count; the last
//     work-group turns them into sigma^2 = sum / count and the threshold
//     (k k) sigma^2, kept in device memory for the next kernel;
//   icp_reject_kernel: the 17 sums of the pairs with r_i^2 <= threshold.
// Both reduce in a fixed order.  A stored slot outside the tree is treated as
// "no match", so any content of the match buffer is safe to read.
struct RejArgs {
    TreeView tree;
    const float *src;
    int64_t n;
    double R[9];
    double t[3];
    double c[3];
    double kk;             // k * k
    const int32_t *mslot;  // [n] original index of the match, -1 if none
    const float *md2;      // [n]
    double *partials;      // [kS][gridDim.x]
    double *stat;          // device: sum r^2, pairs, threshold
    uint8_t *kept;         // [n] or null: 1 where the pair is kept
    const double *rt_dev;  // device loop: (R, t) here (its first solve), not in R / t
};

// The matched target point of source point i, if any (a stored index outside
// the tree counts as none, so any buffer content is safe to read).
__device__ __forceinline__ bool rej_pair(const RejArgs &a, int64_t i, float4 &m)
{
    const int32_t j = a.mslot[i];
    if (!(j >= 0 && int64_t(j) < a.tree.n)) return false;
    m = a.tree.pts[a.tree.slot_of[j]];
    return true;
}

__device__ __forceinline__ double rej_residual_sq(const double (&T)[12], double X, double Y,
                                                  double Z, const float4 &m)
{
    const double e0 = (((T[0] * X + T[1] * Y) + T[2] * Z) + T[9]) - double(m.x);
    const double e1 = (((T[3] * X + T[4] * Y) + T[5] * Z) + T[10]) - double(m.y);
    const double e2 = (((T[6] * X + T[7] * Y) + T[8] * Z) + T[11]) - double(m.z);
    return (e0 * e0 + e1 * e1) + e2 * e2;
}

// (R, t) of a rejection kernel: the arguments, or the device loop's state.
__device__ __forceinline__ void rej_transform(const RejArgs &a, double (&T)[12])
{
#pragma unroll
    for (int k = 0; k < 12; ++k) T[k] = a.rt_dev ? a.rt_dev[k] : (k < 9 ? a.R[k] : a.t[k - 9]);
}

__global__ __launch_bounds__(kWG) void icp_residual_kernel(RejArgs a)
{
    __shared__ double red[(kWG / 64) * kS];
    double acc[kS];
#pragma unroll
    for (int c = 0; c < kS; ++c) acc[c] = 0.0;
    double T[12];
    rej_transform(a, T);
    for (int64_t i = int64_t(blockIdx.x) * kWG + threadIdx.x; i < a.n;
         i += int64_t(gridDim.x) * kWG) {
        float4 m;
        if (!rej_pair(a, i, m)) continue;
        acc[0] += rej_residual_sq(T, a.src[3 * i], a.src[3 * i + 1], a.src[3 * i + 2], m);
        acc[1] += 1.0;
    }
    block_sum(acc, red, a.partials + blockIdx.x, gridDim.x);
}

// sigma^2 and the threshold from the residual kernel's partials (one group).
__global__ __launch_bounds__(kWG) void residual_stat_kernel(const double *p, int32_t nb, double kk,
                                                            double *stat)
{
    __shared__ double red[(kWG / 64) * kS];
    __shared__ double tot[kS];
    double acc[kS];
#pragma unroll
    for (int c = 0; c < kS; ++c) acc[c] = 0.0;
    for (int32_t g = threadIdx.x; g < nb; g += kWG) {
        acc[0] += p[g];
        acc[1] += p[int64_t(nb) + g];
    }
    block_sum(acc, red, tot, 1);
    __syncthreads();
    if (threadIdx.x == 0) {
        const double sum = tot[0];
        const double cnt = tot[1];
        stat[0] = sum;
        stat[1] = cnt;
        stat[2] = kk * (sum / cnt);
    }
}

__global__ __launch_bounds__(kWG) void icp_reject_kernel(RejArgs a)
{
    __shared__ double red[(kWG / 64) * kS];
    double acc[kS];
#pragma unroll
    for (int c = 0; c < kS; ++c) acc[c] = 0.0;
    const double thr = a.stat[2];
    double T[12];
    rej_transform(a, T);
    for (int64_t i = int64_t(blockIdx.x) * kWG + threadIdx.x; i < a.n;
         i += int64_t(gridDim.x) * kWG) {
        float4 mp;
        bool keep = false;
        if (rej_pair(a, i, mp)) {
            const double X = a.src[3 * i], Y = a.src[3 * i + 1], Z = a.src[3 * i + 2];
            keep = rej_residual_sq(T, X, Y, Z, mp) <= thr;
            if (keep) {
                const double s0 = X - a.c[0], s1 = Y - a.c[1], s2 = Z - a.c[2];
                const double m0 = double(mp.x) - a.c[0], m1 = double(mp.y) - a.c[1],
                             m2 = double(mp.z) - a.c[2];
                acc[0] += s0; acc[1] += s1; acc[2] += s2;
                acc[3] += m0; acc[4] += m1; acc[5] += m2;
                acc[6] += s0 * m0; acc[7] += s0 * m1; acc[8] += s0 * m2;
                acc[9] += s1 * m0; acc[10] += s1 * m1; acc[11] += s1 * m2;
                acc[12] += s2 * m0; acc[13] += s2 * m1; acc[14] += s2 * m2;
                acc[15] += double(a.md2[i]);
                acc[16] += 1.0;
            }
        }
        if (a.kept) a.kept[i] = keep ? 1 : 0;
    }
    block_sum(acc, red, a.partials + blockIdx.x, gridDim.x);
}

// --------------------------------------------------------------- transform

__global__ __launch_bounds__(256) void transform_kernel(const float *in, float *out, int64_t n,
                                                        double r0, double r1, double r2,
                                                        double r3, double r4, double r5,
                                                        double r6, double r7, double r8,
                                                        double t0, double t1, double t2)
{
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n;
         i += int64_t(gridDim.x) * 256) {
        const double x = in[3 * i], y = in[3 * i + 1], z = in[3 * i + 2];
        const float a = rigid_row(r0, r1, r2, t0, x, y, z);
        const float b = rigid_row(r3, r4, r5, t1, x, y, z);
        const float c = rigid_row(r6, r7, r8, t2, x, y, z);
        out[3 * i] = a;
        out[3 * i + 1] = b;
        out[3 * i + 2] = c;
    }
}

// ------------------------------------------------------- Morton ordering
//
// Queries are ordered by the top key_bits bits of their 30-bit Morton code
// in the target's bounding box (10 bits per axis, clamped), so that each
// XCD's segment of the order is one region of space (its L2 holds that part
// of the tree).  Stable LSD radix sort, one 8-bit pass per 8 key bits; the
// permutation is a deterministic function of the input.  nn_query takes 8
// bits (one pass: Stress 1M leaf 8 / 16 call 186 / 193 -> 175 / 187 us; the
// search is 9-11% slower on the coarser order, the sort half as long), the
// ICP entry points 16 (two passes, paid once for 30 searches).

struct OrderArgs {
    const float *pts;
    int64_t m;
    float R[12];  // row-major R then t; used when moved != 0
    int32_t moved;
    int32_t key_shift;  // 30 - key bits
    float lo[3];
    float inv[3];
};

__device__ __forceinline__ uint32_t spread10(uint32_t v)
{
    v &= 0x3ffu;
    v = (v | (v << 16)) & 0x030000FFu;
    v = (v | (v << 8)) & 0x0300F00Fu;
    v = (v | (v << 4)) & 0x030C30C3u;
    v = (v | (v << 2)) & 0x09249249u;
    return v;
}

__device__ __forceinline__ uint32_t quant10(float x, float lo, float inv)
{
    const float f = (x - lo) * inv * 1024.0f;
    if (!(f > 0.0f)) return 0u;  // also NaN
    if (f >= 1023.0f) return 1023u;
    return uint32_t(f);
}

__device__ __forceinline__ uint32_t order_key(const OrderArgs &a, int64_t i)
{
    float x = a.pts[3 * i], y = a.pts[3 * i + 1], z = a.pts[3 * i + 2];
    if (a.moved) {
        const float u = a.R[0] * x + a.R[1] * y + a.R[2] * z + a.R[9];
        const float v = a.R[3] * x + a.R[4] * y + a.R[5] * z + a.R[10];
        const float w = a.R[6] * x + a.R[7] * y + a.R[8] * z + a.R[11];
        x = u;
        y = v;
        z = w;
    }
    const uint32_t code = (spread10(quant10(x, a.lo[0], a.inv[0])) << 2) |
                          (spread10(quant10(y, a.lo[1], a.inv[1])) << 1) |
                          spread10(quant10(z, a.lo[2], a.inv[2]));
    return code >> a.key_shift;
}

template <bool FROM_POINTS>
__global__ __launch_bounds__(kSortThreads) void radix_hist_kernel(OrderArgs oa, const uint32_t *keys,
                                                                  int shift, uint32_t *hist,
                                                                  int32_t ntiles)
{
    __shared__ uint32_t h[256];
    h[threadIdx.x] = 0u;
    __syncthreads();
    const int64_t base = int64_t(blockIdx.x) * kSortTile;
    uint32_t key[kSortItems];
#pragma unroll
    for (int r = 0; r < kSortItems; ++r) {
        const int64_t e = base + r * kSortThreads + threadIdx.x;
        key[r] = e < oa.m ? (FROM_POINTS ? order_key(oa, e) : keys[e]) : 0u;
    }
#pragma unroll
    for (int r = 0; r < kSortItems; ++r)
        if (base + r * kSortThreads + threadIdx.x < oa.m) atomicAdd(&h[(key[r] >> shift) & 255u], 1u);
    __syncthreads();
    hist[int64_t(threadIdx.x) * ntiles + blockIdx.x] = h[threadIdx.x];
}

// Per-digit exclusive scan over tiles: work-group d scans row d of hist
// (the tile counts of digit d, contiguous) in place and writes the row total
// to totals[d].  The scatter kernel adds the digit bases.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t *wsum /* LDS [4] */,
                                                         uint32_t &total)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    uint32_t before = 0;
    total = 0;
#pragma unroll
    for (int ww = 0; ww < kSortThreads / 64; ++ww) {
        before += ww < w ? wsum[ww] : 0u;
        total += wsum[ww];
    }
    __syncthreads();
    return before + x - v;
}

__global__ __launch_bounds__(kSortThreads) void radix_scan_kernel(uint32_t *hist, int32_t ntiles,
                                                                  uint32_t *totals,
                                                                  uint32_t *zero_me)
{
    __shared__ uint32_t wsum[kSortThreads / 64];
    uint32_t *row = hist + int64_t(blockIdx.x) * ntiles;
    uint32_t carry = 0;
    for (int32_t k0 = 0; k0 < ntiles; k0 += kSortThreads) {
        const int32_t k = k0 + threadIdx.x;
        const uint32_t v = k < ntiles ? row[k] : 0u;
        uint32_t total;
        const uint32_t ex = block_exclusive_scan(v, wsum, total);
        if (k < ntiles) row[k] = carry + ex;
        carry += total;
    }
    if (threadIdx.x == 0) {
        totals[blockIdx.x] = carry;
        if (zero_me && blockIdx.x == 0) *zero_me = 0u;
    }
}

// Stable scatter of one tile.  Element e = tile*2048 + r*256 + tid is the
// r-th round of thread tid, so (r, tid) is the input order inside the tile.
// Within a wave, lanes holding the same digit are found with 8 ballots; the
// rank of an element = running count of its digit in this tile (earlier
// rounds) + counts of earlier waves in this round + lanes below it.
template <bool FROM_POINTS, bool WRITE_KEYS>
__global__ __launch_bounds__(kSortThreads) void radix_scatter_kernel(
    OrderArgs oa, const uint32_t *keys_in, const int32_t *vals_in, int shift,
    const uint32_t *hist, const uint32_t *totals, int32_t ntiles, uint32_t *keys_out,
    int32_t *vals_out)
{
    __shared__ uint32_t base[256];
    __shared__ uint32_t wcnt[kSortThreads / 64][256];
    __shared__ uint32_t wsum[kSortThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const uint64_t below = (uint64_t(1) << lane) - 1u;
    uint32_t all;
    const uint32_t digit_base = block_exclusive_scan(totals[tid], wsum, all);
    base[tid] = digit_base + hist[int64_t(tid) * ntiles + blockIdx.x];
    const int64_t tbase = int64_t(blockIdx.x) * kSortTile;
    uint32_t keys_r[kSortItems];
    int32_t vals_r[kSortItems];
#pragma unroll
    for (int r = 0; r < kSortItems; ++r) {
        const int64_t e = tbase + r * kSortThreads + tid;
        keys_r[r] = 0u;
        vals_r[r] = 0;
        if (e < oa.m) {
            keys_r[r] = FROM_POINTS ? order_key(oa, e) : keys_in[e];
            vals_r[r] = FROM_POINTS ? int32_t(e) : vals_in[e];
        }
    }
#pragma unroll
    for (int r = 0; r < kSortItems; ++r) {
        const int64_t e = tbase + r * kSortThreads + tid;
        const bool valid = e < oa.m;
        const uint32_t key = keys_r[r];
        const int32_t val = vals_r[r];
        const uint32_t dig = (key >> shift) & 255u;
#pragma unroll
        for (int ww = 0; ww < kSortThreads / 64; ++ww) wcnt[ww][tid] = 0u;
        __syncthreads();
        uint64_t peers = __ballot(valid);
#pragma unroll
        for (int bit = 0; bit < 8; ++bit) {
            const bool set = (dig >> bit) & 1u;
            const uint64_t bal = __ballot(set);
            peers &= set ? bal : ~bal;
        }
        const uint32_t rank = uint32_t(__popcll(peers & below));
        if (valid && rank == 0) wcnt[w][dig] = uint32_t(__popcll(peers));
        __syncthreads();
        if (valid) {
            uint32_t off = base[dig] + rank;
            for (int ww = 0; ww < w; ++ww) off += wcnt[ww][dig];
            if (WRITE_KEYS) keys_out[off] = key;
            vals_out[off] = val;
        }
        __syncthreads();
        uint32_t add = 0u;
#pragma unroll
        for (int ww = 0; ww < kSortThreads / 64; ++ww) add += wcnt[ww][tid];
        base[tid] += add;
    }
}

// ------------------------------------------------------------ workspaces

static size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

static int32_t sort_tiles(int64_t m) { return int32_t((m + kSortTile - 1) / kSortTile); }

size_t sort_workspace_bytes(int64_t m)
{
    if (m <= 0) return 0;
    const size_t mm = size_t(m);
    return align256(mm * 4) * 3 + align256(size_t(256) * sort_tiles(m) * 4) + align256(256 * 4);
}

SortWorkspace carve_sort_workspace(void *ws, int64_t m)
{
    SortWorkspace w{};
    char *p = static_cast<char *>(ws);
    const size_t a = align256(size_t(m) * 4);
    w.keys_a = nullptr;
    w.keys_b = reinterpret_cast<uint32_t *>(p);
    w.vals_b = reinterpret_cast<int32_t *>(p + a);
    w.vals_a = reinterpret_cast<int32_t *>(p + 2 * a);
    w.hist = reinterpret_cast<uint32_t *>(p + 3 * a);
    w.ntiles = sort_tiles(m);
    w.totals = reinterpret_cast<uint32_t *>(p + 3 * a + align256(size_t(256) * w.ntiles * 4));
    return w;
}

// Pass-1 grid and per-work-group list segment of the two-pass search.
static void twopass_shape(int64_t m, int32_t &nb1, int32_t &cap)
{
    int64_t b = (m + kWG - 1) / kWG;
    nb1 = int32_t(b < 1 ? 1 : (b > kPass1MaxBlocks ? kPass1MaxBlocks : b));
    const int64_t sweeps = (m + int64_t(nb1) * kWG - 1) / (int64_t(nb1) * kWG);
    cap = int32_t((sweeps < 1 ? 1 : sweeps) * kWG);
}

size_t twopass_bytes(int64_t m)
{
    if (m <= 0) return 0;
    int32_t nb1, cap;
    twopass_shape(m, nb1, cap);
    return align256(size_t(nb1) * cap * 4) + align256(size_t(kPass1MaxBlocks) * 4);
}

static TwoPass carve_twopass(void *p, int64_t m)
{
    TwoPass tp{};
    twopass_shape(m, tp.nb1, tp.cap);
    char *c = static_cast<char *>(p);
    tp.list = reinterpret_cast<int32_t *>(c);
    tp.counts = reinterpret_cast<uint32_t *>(c + align256(size_t(tp.nb1) * tp.cap * 4));
    return tp;
}

size_t query_ws_bytes(int64_t m)
{
    return m > 0 ? sort_workspace_bytes(m) + twopass_bytes(m) : 0;
}

QueryWorkspace carve_query_workspace(void *ws, int64_t m)
{
    QueryWorkspace w{};
    w.sort = carve_sort_workspace(ws, m);
    w.twopass = static_cast<char *>(ws) + sort_workspace_bytes(m);
    return w;
}

// Work-groups of a fused launch: `per` points per group and sweep (G lanes per
// point: kWG / G), at most kIcpMaxBlocks (the partials' columns).
static int32_t icp_blocks(int64_t n, int64_t per)
{
    const int64_t b = (n + per - 1) / per;
    return int32_t(b < 1 ? 1 : (b > kIcpMaxBlocks ? kIcpMaxBlocks : b));
}

size_t icp_ws_bytes(int64_t n)
{
    if (n <= 0) return 0;
    const size_t nn = size_t(n);
    return sort_workspace_bytes(n) + align256(size_t(kS) * kIcpMaxBlocks * 8) +
           align256(size_t(kS) * kPass2Blocks * 8) + align256(size_t(kS) * 8) +
           align256(nn * 4) + align256(nn * 8) + twopass_bytes(n) + 2 * align256(nn * 4) + 256 +
           align256(sizeof(IcpLoopState)) + align256(nn * 4);
}

IcpWorkspace carve_icp_workspace(void *ws, int64_t n)
{
    IcpWorkspace w{};
    char *p = static_cast<char *>(ws);
    w.sort = carve_sort_workspace(ws, n);
    p += sort_workspace_bytes(n);
    w.partials = reinterpret_cast<double *>(p);
    p += align256(size_t(kS) * kIcpMaxBlocks * 8);
    w.partials2 = reinterpret_cast<double *>(p);
    p += align256(size_t(kS) * kPass2Blocks * 8);
    w.sums = reinterpret_cast<double *>(p);
    p += align256(size_t(kS) * 8);
    w.pslot = reinterpret_cast<uint32_t *>(p);
    p += align256(size_t(n) * 4);
    w.pkey = reinterpret_cast<uint64_t *>(p);
    p += align256(size_t(n) * 8);
    w.twopass = p;
    p += twopass_bytes(n);
    w.mslot = reinterpret_cast<int32_t *>(p);
    p += align256(size_t(n) * 4);
    w.md2 = reinterpret_cast<float *>(p);
    p += align256(size_t(n) * 4);
    w.stat = reinterpret_cast<double *>(p);
    p += 256;
    w.loop = reinterpret_cast<IcpLoopState *>(p);
    p += align256(sizeof(IcpLoopState));
    w.hint = reinterpret_cast<uint32_t *>(p);
    w.max_blocks = kIcpMaxBlocks;
    return w;
}

// --------------------------------------------------------------- launchers

static TreeView tree_view(const DeviceTree &t)
{
    TreeView v;
    v.nodes = static_cast<const float4 *>(t.nodes);
    v.boxes = static_cast<const float4 *>(t.boxes);
    v.slot_of = static_cast<const int32_t *>(t.slot_of);
    v.paths = static_cast<const uint4 *>(t.paths);
    v.pts = static_cast<const float4 *>(t.points);
    v.first_leaf = t.first_leaf;
    v.depth = t.depth;
    v.n = t.n;
    return v;
}

static OrderArgs make_order_args(const DeviceTree &t, const float *pts, int64_t m, const float *R12,
                                 int key_bits)
{
    OrderArgs oa{};
    oa.pts = pts;
    oa.m = m;
    oa.moved = R12 ? 1 : 0;
    oa.key_shift = 30 - key_bits;
    for (int k = 0; k < 12; ++k) oa.R[k] = R12 ? R12[k] : 0.0f;
    for (int k = 0; k < 3; ++k) {
        oa.lo[k] = t.box_lo[k];
        oa.inv[k] = t.box_inv[k];
    }
    return oa;
}

static hipError_t morton_order_impl(const DeviceTree &t, const float *pts, int64_t m,
                                    const float *R12, int key_bits, const SortWorkspace &ws,
                                    uint32_t *zero_me, const int32_t **perm, hipStream_t s)
{
    const OrderArgs oa = make_order_args(t, pts, m, R12, key_bits);
    const int32_t nt = ws.ntiles;
    radix_hist_kernel<true><<<nt, kSortThreads, 0, s>>>(oa, nullptr, 0, ws.hist, nt);
    radix_scan_kernel<<<256, kSortThreads, 0, s>>>(ws.hist, nt, ws.totals, zero_me);
    if (key_bits <= 8) {  // one pass: the permutation straight out of it
        radix_scatter_kernel<true, false><<<nt, kSortThreads, 0, s>>>(
            oa, nullptr, nullptr, 0, ws.hist, ws.totals, nt, nullptr, ws.vals_a);
        *perm = ws.vals_a;
        return hipGetLastError();
    }
    radix_scatter_kernel<true, true><<<nt, kSortThreads, 0, s>>>(
        oa, nullptr, nullptr, 0, ws.hist, ws.totals, nt, ws.keys_b, ws.vals_b);
    radix_hist_kernel<false><<<nt, kSortThreads, 0, s>>>(oa, ws.keys_b, 8, ws.hist, nt);
    radix_scan_kernel<<<256, kSortThreads, 0, s>>>(ws.hist, nt, ws.totals, nullptr);
    radix_scatter_kernel<false, false><<<nt, kSortThreads, 0, s>>>(
        oa, ws.keys_b, ws.vals_b, 8, ws.hist, ws.totals, nt, nullptr, ws.vals_a);
    *perm = ws.vals_a;
    return hipGetLastError();
}

hipError_t launch_morton_order(const DeviceTree &t, const float *pts, int64_t m, const float *R12,
                               int key_bits, const SortWorkspace &ws, const int32_t **perm,
                               hipStream_t s)
{
    return morton_order_impl(t, pts, m, R12, key_bits, ws, nullptr, perm, s);
}

hipError_t launch_icp_order(const DeviceTree &t, const float *pts, int64_t m, const float *R12,
                            const IcpWorkspace &ws, const int32_t **perm, hipStream_t s)
{
    return morton_order_impl(t, pts, m, R12, kKeyBitsIcp, ws.sort, nullptr, perm, s);
}

// Dynamic LDS of the balanced search kernels: the pending bound of every path
// level of a depth-D tree, for each lane (D x 1 KB per work-group), so a
// shallow tree leaves room for more resident work-groups.
static size_t lbs_bytes(int32_t depth)
{
    return size_t(depth < 1 ? 1 : depth) * kWG * sizeof(float);
}

// Work-groups of `kernel` (kWG lanes, lbs_bytes(depth) of dynamic LDS) the
// current device holds at once: CUs x resident groups per CU (0 on failure;
// *cus_out = CUs when given); cached per device, slot and depth.
template <typename K>
static int64_t resident_groups(K kernel, int slot, int32_t depth, int64_t *cus_out = nullptr)
{
    // slots 2, 3, 5: the 8-point kernels, with dynamic LDS (4, 5: nn_kernel QL)
    const size_t dyn = (slot == 2 || slot == 3 || slot == 5) ? lbs_bytes(depth) : 0;
    static std::atomic<int64_t> cache[64][6][kDevMaxDepth + 1];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    const int d = depth < 0 ? 0 : (depth > kDevMaxDepth ? kDevMaxDepth : depth);
    int64_t v = cache[dev][slot][d].load(std::memory_order_relaxed);
    if (v <= 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kWG, dyn) !=
                hipSuccess ||
            cus <= 0 || per_cu <= 0)
            return 0;
        v = (int64_t(cus) << 8) | per_cu;  // per_cu < 256
        cache[dev][slot][d].store(v, std::memory_order_relaxed);
    }
    if (cus_out) *cus_out = v >> 8;
    return (v >> 8) * (v & 0xFF);
}

// Spread the queries of a one-lane-per-query launch (spread_pos)?  Always for
// the given order.  For a Morton order only while the launch fills at most
// kSpreadMaxRounds rounds of resident work-groups: such a launch lasts as
// long as its longest wave, so mixing easy and hard queries in every wave
// pays; a longer launch overlaps its long waves with others, and keeping
// each wave's queries side by side (fewer distinct cache lines per load)
// pays more.
constexpr int64_t kSpreadMaxRounds = 3;
template <typename K>
static bool spread_wanted(K kernel, int slot, int32_t depth, int64_t m, bool ordered)
{
    if (!ordered) return true;
    const int64_t groups = (m + kWG - 1) / kWG, res = resident_groups(kernel, slot, depth);
    return res > 0 && groups <= kSpreadMaxRounds * res;
}

// Queries per wave and work-groups of a one-lane-per-query launch of m
// queries.  64 per wave (and as many groups as that takes) when 64 per wave
// would fill more than one round of resident work-groups, or under a
// distance bound: on a full machine extra idle lanes would only add redundant
// subtree work, and under a bound few far subtrees are pending to be taken
// (measured: 57 vs 52 us per Scene ICP iteration).  Otherwise the launch
// lasts as long as its longest wave, and the idle lanes shorten it by taking
// pending subtrees at no cost in occupancy: the launch gets c work-groups on
// every CU (the fewest that leave at most `target` queries to a wave) and
// q = ceil(m / waves) queries per wave.  Whole groups per CU give every SIMD
// the same number of waves; with a remainder of groups, the CUs holding one
// more run longer and set the launch time (Scene 100k: 782 groups of 32
// queries per wave, 46.2 us; 768 groups of 33, 41.8 us; 1,024 of 25, 44.7 us;
// 512 of 49, 42.9 us).  Small launches keep at least KDNN_Q_MIN queries per
// wave and fewer groups.
#ifndef KDNN_Q_MIN
#define KDNN_Q_MIN 8
#endif
struct WavePlan {
    uint32_t q;
    int64_t blocks;
};
static WavePlan full_wave_plan(int64_t m)
{
    constexpr int64_t per = int64_t(kWG / 64) * kQFull;
    const int64_t b = (m + per - 1) / per;
    return WavePlan{kQFull, b < 1 ? 1 : b};
}
template <typename K>
static WavePlan wave_plan(K kernel, int slot, int32_t depth, int64_t m, float bound2,
                          int64_t target)
{
    constexpr int64_t wpg = kWG / 64;  // waves per group
    WavePlan p = full_wave_plan(m);
    if (!(bound2 == INFINITY)) return p;
    int64_t cus = 0;
    const int64_t res = resident_groups(kernel, slot, depth, &cus);
    if (res <= 0 || p.blocks > res) return p;
    const int64_t per_cu = res / cus, tq = target;
    int64_t c = (m + wpg * cus * tq - 1) / (wpg * cus * tq);
    c = c < 1 ? 1 : (c > per_cu ? per_cu : c);
    int64_t blocks = c * cus;
    int64_t q = (m + wpg * blocks - 1) / (wpg * blocks);
    if (q < KDNN_Q_MIN) {
        blocks = (m + wpg * KDNN_Q_MIN - 1) / (wpg * KDNN_Q_MIN);
        if (blocks < 1) blocks = 1;
        q = (m + wpg * blocks - 1) / (wpg * blocks);
    }
    p.q = uint32_t(q);
    p.blocks = blocks;
    return p;
}

template <typename T>
struct same_type {
    using type = T;
};

// Launch through hipExtLaunchKernel: a non-null e0 / e1 is stamped by the
// dispatch itself at its start / end (no marker packets between kernels);
// with both null it is a plain launch.
template <typename... P>
static hipError_t launch_k(void (*k)(P...), dim3 grid, uint32_t block, size_t lds, hipStream_t s,
                           hipEvent_t e0, hipEvent_t e1, typename same_type<P>::type... args)
{
    void *pa[] = {static_cast<void *>(&args)...};
    return hipExtLaunchKernel(reinterpret_cast<const void *>(k), grid, dim3(block), pa, lds, s, e0,
                              e1, 0);
}

template <int G, int CH = kLeafChunk>
static hipError_t launch_nn_g(NnArgs a, bool stats, float bound2, hipStream_t s, hipEvent_t e0,
                              hipEvent_t e1)
{
    int64_t blocks = (a.m + kWG / G - 1) / (kWG / G);  // G lanes per query
    if (G == 1) {
        const int slot = CH == kLeafChunk ? 0 : 2;
        a.spread = spread_wanted(nn_kernel<1, false, CH>, slot, a.tree.depth, a.m,
                                 a.perm != nullptr);
        // the instrumented kernel searches each query alone, 64 per wave
        const WavePlan wp = stats ? full_wave_plan(a.m)
                                  : wave_plan(nn_kernel<1, false, CH>, slot, a.tree.depth, a.m,
                                              bound2, KDNN_Q_TARGET_NN);
        a.wq = wp.q;
        blocks = wp.blocks;
    }
    if (blocks > (int64_t(1) << 20)) blocks = int64_t(1) << 20;
    const size_t lds = G == 1 && CH == kLeafChunkSmall ? lbs_bytes(a.tree.depth) : 0;
    const dim3 grid{uint32_t(blocks)};
    if (stats) return launch_k(nn_kernel<G, true, CH>, grid, kWG, lds, s, e0, e1, a);
    if (G == 1 && KDNN_QLDS && a.wq < kQFull &&
        blocks <= resident_groups(nn_kernel<1, false, CH, true>, CH == kLeafChunk ? 4 : 5,
                                  a.tree.depth))
        // a one-round launch, still resident at once with the larger LDS
        return launch_k(nn_kernel<1, false, CH, true>, grid, kWG, lds, s, e0, e1, a);
    return launch_k(nn_kernel<G, false, CH>, grid, kWG, lds, s, e0, e1, a);
}

// Persistent LDS launch shape for this device: one work-group per CU and
// the deepest L <= min(12, D) whose node records fit the LDS limit.
struct PersistShape {
    uint32_t blocks;
    uint32_t lds_first;  // 2^L
    size_t lds_bytes;
};

static bool persist_shape(const TreeView &t, int64_t m, PersistShape &ps)
{
    static int cached_dev = -1;
    static int cus = 0;
    static size_t lds_max = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return false;
    if (dev != cached_dev) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return false;
        cus = prop.multiProcessorCount;
        lds_max = prop.sharedMemPerBlock;
        cached_dev = dev;
    }
    if (m < int64_t(cus) * 64) return false;  // too few queries to amortise the copy
    int L = t.depth < kLdsMaxLevels ? t.depth : kLdsMaxLevels;
    while (L > 0 && (size_t(32) << L) + 2048 > lds_max) --L;
    if (L < 4) return false;
    ps.lds_first = 1u << L;
    ps.lds_bytes = size_t(32) << L;
    ps.blocks = uint32_t(cus);
    return true;
}

template <typename K>
static void allow_lds(K kernel, size_t bytes)
{
    (void)hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, int(bytes));
}

static hipError_t launch_nn_two_pass(const NnArgs &a, bool stats, void *twopass, hipStream_t s,
                                     hipEvent_t e0, hipEvent_t e1)
{
    const TwoPass tp = carve_twopass(twopass, a.m);
    hipError_t e;
    if (stats) {
        e = launch_k(nn_pass1_kernel<true>, dim3(uint32_t(tp.nb1)), kWG, 0, s, e0, nullptr, a, tp);
        if (e == hipSuccess)
            e = launch_k(nn_pass2_kernel<true>, dim3(kPass2Blocks), kWG, 0, s, nullptr, e1, a, tp);
    } else {
        e = launch_k(nn_pass1_kernel<false>, dim3(uint32_t(tp.nb1)), kWG, 0, s, e0, nullptr, a,
                     tp);
        if (e == hipSuccess)
            e = launch_k(nn_pass2_kernel<false>, dim3(kPass2Blocks), kWG, 0, s, nullptr, e1, a, tp);
    }
    return e;
}

// The start key of a search under the squared-distance bound bound2: no bound
// (+inf) starts from the largest float instead, which accepts every finite
// distance as +inf would (a point at +inf is no match either way) and lets
// enters() drop its own +inf test.
static uint64_t host_bound_key(float bound2)
{
    const float b = bound2 < FLT_MAX ? bound2 : FLT_MAX;
    uint32_t bits;
    std::memcpy(&bits, &b, 4);
    return (uint64_t(bits) << 32) | 0xFFFFFFFFull;
}

hipError_t launch_nn(const DeviceTree &t, const float *q, int64_t m, const int32_t *perm,
                     int32_t *idx, float *d2, uint32_t *cnt_nodes, uint32_t *cnt_pts, bool stats,
                     const Schedule &sc, float bound2, void *twopass, hipStream_t s,
                     const hipEvent_t *timing)
{
    const hipEvent_t e0 = timing ? timing[0] : nullptr, e1 = timing ? timing[1] : nullptr;
    hipError_t e;
    NnArgs a{};
    a.tree = tree_view(t);
    a.init = host_bound_key(bound2);
    a.q = q;
    a.m = m;
    a.perm = perm;
    a.idx = idx;
    a.d2 = d2;
    a.cnt_nodes = cnt_nodes;
    a.cnt_pts = cnt_pts;
    a.budget = sc.budget;
    PersistShape ps;
    if (sc.lanes == 0 && sc.top_lds && persist_shape(a.tree, m, ps)) {
        if (stats) {
            allow_lds(nn_persist_kernel<true>, ps.lds_bytes);
            e = launch_k(nn_persist_kernel<true>, dim3(ps.blocks), kPWG, ps.lds_bytes, s, e0, e1,
                         a, ps.lds_first);
        } else {
            allow_lds(nn_persist_kernel<false>, ps.lds_bytes);
            e = launch_k(nn_persist_kernel<false>, dim3(ps.blocks), kPWG, ps.lds_bytes, s, e0, e1,
                         a, ps.lds_first);
        }
    } else if (sc.lanes == 0 && sc.budget != 0 && twopass) {
        e = launch_nn_two_pass(a, stats, twopass, s, e0, e1);
    } else {
        switch (sc.lanes) {
        case 2: e = launch_nn_g<2>(a, stats, bound2, s, e0, e1); break;
        case 4: e = launch_nn_g<4>(a, stats, bound2, s, e0, e1); break;
        case 8: e = launch_nn_g<8>(a, stats, bound2, s, e0, e1); break;
        case 16: e = launch_nn_g<16>(a, stats, bound2, s, e0, e1); break;
        default:
            if (t.max_leaf <= kLeafChunkSmall)
                e = launch_nn_g<1, kLeafChunkSmall>(a, stats, bound2, s, e0, e1);
            else
                e = launch_nn_g<1>(a, stats, bound2, s, e0, e1);
            break;
        }
    }
    return e != hipSuccess ? e : hipGetLastError();
}

hipError_t launch_transform(const float *in, float *out, int64_t n, const double *R,
                            const double *t, hipStream_t s)
{
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    transform_kernel<<<dim3(uint32_t(blocks)), 256, 0, s>>>(in, out, n, R[0], R[1], R[2], R[3],
                                                             R[4], R[5], R[6], R[7], R[8], t[0],
                                                             t[1], t[2]);
    return hipGetLastError();
}

hipError_t launch_icp_fused(const DeviceTree &t, const float *src, int64_t n, const int32_t *perm,
                            const double *R, const double *tv, const IcpWorkspace &ws,
                            double *sums_out, int32_t *idx, float *d2, const Schedule &sc,
                            float bound2, bool keep_matches, hipStream_t s,
                            const hipEvent_t *timing, uint64_t *done, uint64_t seq,
                            const IcpLoop *loop, int hint_mode)
{
    if (loop && (sc.lanes > 1 || sc.top_lds || sc.budget != 0))
        return hipErrorInvalidValue;  // the device loop runs the one-lane-per-query kernel only
    IcpArgs a{};
    if (loop) {
        a.rt_dev = loop->state->rt;
        a.stop = &loop->state->stop;
    }
    a.tree = tree_view(t);
    a.init = host_bound_key(bound2);
    a.mslot = keep_matches ? ws.mslot : nullptr;
    a.md2 = keep_matches ? ws.md2 : nullptr;
    a.src = src;
    a.n = n;
    a.perm = perm;
    for (int k = 0; k < 9; ++k) a.R[k] = R[k];
    for (int k = 0; k < 3; ++k) {
        a.t[k] = tv[k];
        a.c[k] = t.center[k];
    }
    a.partials = ws.partials;
    a.partials2 = ws.partials2;
    a.sums = sums_out;
    a.pkey = ws.pkey;
    a.pslot = ws.pslot;
    a.idx = idx;
    a.d2 = d2;
    a.budget = sc.budget;
    const bool small = t.max_leaf <= kLeafChunkSmall;
    void (*k1)(IcpArgs) = small ? icp_fused_kernel<1, kLeafChunkSmall> : icp_fused_kernel<1>;
    a.spread = spread_wanted(k1, small ? 3 : 1, t.depth, n, perm != nullptr);
    const WavePlan wp = wave_plan(k1, small ? 3 : 1, t.depth, n, bound2, KDNN_Q_TARGET_ICP);
    a.wq = wp.q;
    // the timing events bracket the search kernel(s), not the reduction
    const hipEvent_t e0 = timing ? timing[0] : nullptr, e1 = timing ? timing[1] : nullptr;
    hipError_t e;
    PersistShape ps;
    if (sc.lanes == 0 && sc.top_lds && persist_shape(a.tree, n, ps)) {
        allow_lds(icp_persist_kernel, ps.lds_bytes);
        e = launch_k(icp_persist_kernel, dim3(ps.blocks), kPWG, ps.lds_bytes, s, e0, e1, a,
                     ps.lds_first);
        if (e != hipSuccess) return e;
        launch_reduce_partials(a.partials, int32_t(ps.blocks), nullptr, 0, sums_out, nullptr,
                               nullptr, done, seq, s);
    } else if (sc.lanes == 0 && sc.budget != 0) {
        const TwoPass tp = carve_twopass(ws.twopass, n);
        e = launch_k(icp_pass1_kernel, dim3(uint32_t(tp.nb1)), kWG, 0, s, e0, nullptr, a, tp);
        if (e == hipSuccess)
            e = launch_k(icp_pass2_kernel, dim3(kPass2Blocks), kWG, 0, s, nullptr, e1, a, tp);
        if (e != hipSuccess) return e;
        launch_reduce_partials(a.partials, tp.nb1, a.partials2, kPass2Blocks, sums_out, nullptr,
                               nullptr, done, seq, s);
    } else {
        const dim3 grid(uint32_t(sc.lanes > 1 ? icp_blocks(n, kWG / sc.lanes)
                                              : (wp.blocks < kIcpMaxBlocks ? wp.blocks
                                                                           : kIcpMaxBlocks)));
        void (*k)(IcpArgs);
        switch (sc.lanes) {
        case 2: k = icp_fused_kernel<2>; break;
        case 4: k = icp_fused_kernel<4>; break;
        case 8: k = icp_fused_kernel<8>; break;
        case 16: k = icp_fused_kernel<16>; break;
        default: k = k1; break;
        }
        if (sc.lanes <= 1 && hint_mode > 0) {  // the one-lane kernel keeps the match leaves
            a.hint = ws.hint;
            a.hint_in = hint_mode > 1;
            if (a.hint_in)
                k = small ? icp_fused_kernel<1, kLeafChunkSmall, true>
                          : icp_fused_kernel<1, kLeafChunk, true>;
        }
        e = launch_k(k, grid, kWG, sc.lanes <= 1 && small ? lbs_bytes(t.depth) : 0, s, e0, e1,
                     a);
        if (e != hipSuccess) return e;
        if (loop)
            launch_icp_loop_step(a.partials, int32_t(grid.x), *loop, t.center, s);
        else
            launch_reduce_partials(a.partials, int32_t(grid.x), nullptr, 0, sums_out, nullptr,
                                   nullptr, done, seq, s);
    }
    return hipGetLastError();
}

// ------------------------------------------------- replay ceiling of a search
//
// A measurement aid (kdnn_replay_bench), not part of any search.  The
// ceiling a search launch is compared against is the time the memory system
// takes to deliver the very records that launch's queries visit, in the same
// work-groups, waves and XCDs, with every dependency removed:
//   1. the instrumented single-lane search records each query's visits
//      (trace_visit: the root box, each child-pair box run, each leaf);
//   2. replay_pack_kernel walks the production launch's shape (blocks, queries
//      per wave, spread positions, order) and lays out each wave's queries'
//      rows step-major in one segment per (sweep, work-group, wave): every
//      query's first visit, then every query's second, ... -- so lanes side
//      by side replay the same step of neighbouring queries, which load the
//      same or nearby records as they do in the search (one query's own
//      visits dealt to adjacent lanes would miss that coherence), while the
//      segment stays dense (no lane idles on a short row); it adds up the
//      visits, bytes and truncated rows;
//   3. replay_kernel, in the same shape, has each wave load its segment's
//      records with its 64 lanes dealt the visits round-robin, two in
//      flight per lane: the root (2 x 16 B), a box run (3 x 16 B) or a leaf
//      (its chunks of CH x 16 B from one base, as the search loads them).
struct ReplayArgs {
    TreeView tree;
    int64_t m;
    const int32_t *perm;
    bool spread;
    uint32_t wq;
    uint32_t tcap;
    const uint32_t *rows;    // [m][tcap]
    const uint32_t *rcount;  // [m]
    uint32_t *packed;        // [segments][64 * tcap]
    uint32_t *seg_total;     // [segments]
    unsigned long long *tally;  // [4]: visits, bytes, node records, leaf points
    unsigned long long *truncated;
    uint32_t *sink;
};

// Bytes the replay loads for visit e (and, for the tally, node records and
// leaf points it stands for).
template <int CH>
__device__ __forceinline__ void replay_cost(const TreeView &t, uint32_t e, uint32_t &bytes,
                                            uint32_t &recs, uint32_t &pts)
{
    if (e == 0u || (e & kSiblingVisit)) {
        bytes = 32u;
        recs = 1u;
        pts = 0u;
    } else if (e & kPlaneVisit) {
        bytes = 16u * uint32_t(kPathWords / 4);
        recs = 2u;
        pts = 0u;
    } else if (e & kLocateVisit) {
        bytes = 8u;
        recs = 1u;
        pts = 0u;
    } else if (e < t.first_leaf) {
        bytes = 48u;
        recs = 2u;
        pts = 0u;
    } else {
        int32_t begin, last, end;
        leaf_range(t, e, begin, last, end);
        const uint32_t chunks = end > begin ? uint32_t((end - begin + CH - 1) / CH) : 1u;
        bytes = chunks * uint32_t(CH) * 16u;
        recs = 0u;
        pts = uint32_t(end - begin);
    }
}

template <int CH>
__global__ __launch_bounds__(kWG) void replay_pack_kernel(ReplayArgs a)
{
    const uint32_t nb = gridDim.x;
    const uint32_t blk = xcd_remap(blockIdx.x, nb);
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const uint32_t wq = a.wq;
    const int64_t QB = int64_t(kWG / 64) * wq;
    int64_t sweep = 0;
    for (int64_t base = int64_t(blk) * QB; base < a.m; base += int64_t(nb) * QB, ++sweep) {
        const int64_t seg = (sweep * nb + blockIdx.x) * (kWG / 64) + wv;
        const int64_t k = base + int64_t(wv) * wq + lane;
        const bool own = uint32_t(lane) < wq && k < a.m;
        const int64_t pos = own ? spread_pos(a.spread, wq, k, blk, base, nb, a.m) : k;
        const int64_t i = own ? (a.perm ? int64_t(a.perm[pos]) : pos) : 0;
        const uint32_t full = own ? a.rcount[i] : 0u;
        const uint32_t len = full < a.tcap ? full : a.tcap;
        uint32_t *const dst = a.packed + size_t(seg) * 64u * a.tcap;
        const uint32_t *const src = a.rows + size_t(i) * a.tcap;
        const uint64_t below = (uint64_t(1) << lane) - 1u;
        // step j of the rows that have one, in lane order, after all of step j - 1
        uint32_t total = 0u;
        unsigned long long b = 0, r = 0, p = 0;
        for (uint32_t j = 0;; ++j) {
            const uint64_t act = __ballot(j < len);
            if (act == 0) break;
            if (j < len) {
                const uint32_t e = src[j];
                dst[total + uint32_t(__popcll(act & below))] = e;
                uint32_t eb, er, ep;
                replay_cost<CH>(a.tree, e, eb, er, ep);
                b += eb;
                r += er;
                p += ep;
            }
            total += uint32_t(__popcll(act));
        }
        if (len) {
            atomicAdd(&a.tally[0], (unsigned long long)len);
            atomicAdd(&a.tally[1], b);
            atomicAdd(&a.tally[2], r);
            atomicAdd(&a.tally[3], p);
        }
        if (full > a.tcap) atomicAdd(a.truncated, 1ull);
        if (lane == 0) a.seg_total[seg] = total;
    }
}

// XOR of the words of the record(s) visit e stands for (loads kept alive).
template <int CH>
__device__ __forceinline__ uint32_t replay_load(const TreeView &t, uint32_t e)
{
    uint32_t x = 0u;
    if (e == 0u) {
        const float4 A = t.nodes[2], B = t.nodes[3];
        x = __float_as_uint(A.x) ^ __float_as_uint(A.y) ^ __float_as_uint(A.z) ^
            __float_as_uint(A.w) ^ __float_as_uint(B.x) ^ __float_as_uint(B.y);
    } else if (e & kSiblingVisit) {
        // the half of its parent's box run that holds node v's box, as warm_start loads it
        const uint32_t v = e & ~kSiblingVisit;
        const float4 *const pb = t.boxes + 3 * size_t(v >> 1) + (v & 1u);
        const float4 P0 = pb[0], P1 = pb[1];
        x = __float_as_uint(P0.x) ^ __float_as_uint(P0.w) ^ __float_as_uint(P1.y) ^
            __float_as_uint(P1.z);
    } else if (e & kLocateVisit) {
        // node i's split value and axis, as locate_leaf loads them
        const float2 S = reinterpret_cast<const float2 *>(t.nodes)[4 * size_t(e & ~kLocateVisit) + 3];
        x = __float_as_uint(S.x) ^ __float_as_uint(S.y);
    } else if (e & kPlaneVisit) {
        // the leaf's plane record, as warm_start loads it
        const uint4 *const pr = t.paths + 4 * size_t((e & ~kPlaneVisit) - t.first_leaf);
#pragma unroll
        for (int v = 0; v < kPathWords / 4; ++v) {
            const uint4 r = pr[v];
            x ^= r.x ^ r.y ^ r.z ^ r.w;
        }
    } else if (e < t.first_leaf) {
        const float4 *const pb = t.boxes + 3 * size_t(e);
        const float4 P0 = pb[0], P1 = pb[1], P2 = pb[2];
        x = __float_as_uint(P0.x) ^ __float_as_uint(P0.w) ^ __float_as_uint(P1.y) ^
            __float_as_uint(P1.z) ^ __float_as_uint(P2.x) ^ __float_as_uint(P2.w);
    } else {
        int32_t begin, last, end;
        leaf_range(t, e, begin, last, end);
        uint32_t k0 = uint32_t(begin);
        do {
            const float4 *pc = t.pts + k0;
            float4 p[CH];
#pragma unroll
            for (int c = 0; c < CH; ++c) p[c] = pc[c];
#pragma unroll
            for (int c = 0; c < CH; ++c)
                x ^= __float_as_uint(p[c].x) ^ __float_as_uint(p[c].y) ^
                     __float_as_uint(p[c].z) ^ __float_as_uint(p[c].w);
            k0 += CH;
        } while (k0 < uint32_t(end));
    }
    return x;
}

template <int CH>
__global__ __launch_bounds__(kWG) void replay_kernel(ReplayArgs a)
{
    const uint32_t nb = gridDim.x;
    const uint32_t blk = xcd_remap(blockIdx.x, nb);
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t QB = int64_t(kWG / 64) * a.wq;
    uint32_t acc = 0u;
    int64_t sweep = 0;
    for (int64_t base = int64_t(blk) * QB; base < a.m; base += int64_t(nb) * QB, ++sweep) {
        const int64_t seg = (sweep * nb + blockIdx.x) * (kWG / 64) + wv;
        const uint32_t T = a.seg_total[seg];
        const uint32_t *const E = a.packed + size_t(seg) * 64u * a.tcap;
        for (uint32_t j = uint32_t(lane); j < T; j += 128u) {
            const uint32_t e0 = E[j];
            const uint32_t e1 = j + 64u < T ? E[j + 64u] : kDone;
            acc ^= replay_load<CH>(a.tree, e0);
            if (e1 != kDone) acc ^= replay_load<CH>(a.tree, e1);
        }
    }
    if (acc == 0x5eed5eedu) a.sink[0] = acc;  // keeps the loads; practically never taken
}

constexpr uint32_t kReplayCap = 512;  // visits recorded per query

struct ReplayPlan {
    int64_t blocks, segments;
    uint32_t wq;
    bool spread, small;
};

// The launch shape of the production kernel the replay stands in for: the
// fused ICP kernel (icp) or nn_query's one-lane-per-query kernel.
static ReplayPlan replay_plan(const DeviceTree &t, int64_t m, bool icp, bool ordered)
{
    ReplayPlan p{};
    p.small = t.max_leaf <= kLeafChunkSmall;
    WavePlan wp;
    if (icp) {
        void (*k1)(IcpArgs) = p.small ? icp_fused_kernel<1, kLeafChunkSmall> : icp_fused_kernel<1>;
        p.spread = spread_wanted(k1, p.small ? 3 : 1, t.depth, m, ordered);
        wp = wave_plan(k1, p.small ? 3 : 1, t.depth, m, INFINITY, KDNN_Q_TARGET_ICP);
        if (wp.blocks > kIcpMaxBlocks) wp.blocks = kIcpMaxBlocks;
    } else if (p.small) {
        p.spread = spread_wanted(nn_kernel<1, false, kLeafChunkSmall>, 2, t.depth, m, ordered);
        wp = wave_plan(nn_kernel<1, false, kLeafChunkSmall>, 2, t.depth, m, INFINITY,
                       KDNN_Q_TARGET_NN);
    } else {
        p.spread = spread_wanted(nn_kernel<1, false>, 0, t.depth, m, ordered);
        wp = wave_plan(nn_kernel<1, false>, 0, t.depth, m, INFINITY, KDNN_Q_TARGET_NN);
    }
    if (wp.blocks > (int64_t(1) << 20)) wp.blocks = int64_t(1) << 20;
    p.blocks = wp.blocks;
    p.wq = wp.q;
    const int64_t per_sweep = p.blocks * int64_t(kWG / 64) * wp.q;
    p.segments = (m + per_sweep - 1) / per_sweep * p.blocks * (kWG / 64);
    return p;
}

struct ReplayWorkspace {
    uint32_t *rows, *rcount, *packed, *seg_total, *sink, *hint;
    int32_t *idx;
    float *d2;
    unsigned long long *tally;  // [5]: tally[0..3], truncated
};

static ReplayWorkspace carve_replay(void *ws, int64_t m, const ReplayPlan &p)
{
    char *c = static_cast<char *>(ws);
    ReplayWorkspace w{};
    w.tally = reinterpret_cast<unsigned long long *>(c);
    c += 256;
    w.sink = reinterpret_cast<uint32_t *>(c);
    c += 256;
    w.rcount = reinterpret_cast<uint32_t *>(c);
    c += align256(size_t(m) * 4);
    w.idx = reinterpret_cast<int32_t *>(c);
    c += align256(size_t(m) * 4);
    w.d2 = reinterpret_cast<float *>(c);
    c += align256(size_t(m) * 4);
    w.seg_total = reinterpret_cast<uint32_t *>(c);
    c += align256(size_t(p.segments) * 4);
    w.hint = reinterpret_cast<uint32_t *>(c);
    c += align256(size_t(m) * 4);
    w.rows = reinterpret_cast<uint32_t *>(c);
    c += align256(size_t(m) * kReplayCap * 4);
    w.packed = reinterpret_cast<uint32_t *>(c);
    return w;
}

size_t replay_ws_bytes(const DeviceTree &t, int64_t m, bool icp)
{
    // the segment count does not depend on the order (spread only permutes)
    const ReplayPlan p = replay_plan(t, m, icp, false);
    return 512 + 4 * align256(size_t(m) * 4) + align256(size_t(p.segments) * 4) +
           align256(size_t(m) * kReplayCap * 4) +
           align256(size_t(p.segments) * 64 * kReplayCap * 4);
}

// Warm-start leaves from matches: the leaf holding each original index's
// point (0 where there is no match), as the fused kernel records them.
__global__ __launch_bounds__(256) void hint_of_match_kernel(TreeView t, const int32_t *idx,
                                                            int64_t m, uint32_t *hint)
{
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < m;
         i += int64_t(gridDim.x) * 256) {
        const int32_t k = idx[i];
        hint[i] = k >= 0 ? leaf_of_slot(t, uint32_t(t.slot_of[k])) : 0u;
    }
}

hipError_t launch_replay(const DeviceTree &t, const float *q, int64_t m, const int32_t *perm,
                         bool icp, const float *q_prev, void *ws, int32_t reps, float *ms_out,
                         ReplayTally *tally, hipStream_t s)
{
    const ReplayPlan p = replay_plan(t, m, icp, perm != nullptr);
    const ReplayWorkspace w = carve_replay(ws, m, p);
    hipError_t e = hipMemsetAsync(w.tally, 0, 5 * sizeof(unsigned long long), s);
    if (e != hipSuccess) return e;
    if (q_prev) {
        // the ICP loop's warm start: each search begins at the leaf of the
        // point's match in the previous iteration, i.e. of q_prev's nearest
        // neighbour
        e = launch_nn(t, q_prev, m, nullptr, w.idx, w.d2, nullptr, nullptr, false, Schedule{},
                      INFINITY, nullptr, s, nullptr);
        if (e != hipSuccess) return e;
        int64_t hb = (m + 255) / 256;
        hint_of_match_kernel<<<dim3(uint32_t(hb < 65536 ? hb : 65536)), 256, 0, s>>>(
            tree_view(t), w.idx, m, w.hint);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    // 1. the visit rows, from the instrumented search
    NnArgs na{};
    na.tree = tree_view(t);
    na.init = host_bound_key(INFINITY);
    na.q = q;
    na.m = m;
    na.idx = w.idx;
    na.d2 = w.d2;
    na.trace = w.rows;
    na.tcount = w.rcount;
    na.tcap = kReplayCap;
    na.hint = q_prev ? w.hint : nullptr;
    const WavePlan fw = full_wave_plan(m);
    na.wq = fw.q;
    const size_t lds = p.small ? lbs_bytes(t.depth) : 0;
    e = p.small ? launch_k(nn_kernel<1, true, kLeafChunkSmall>, dim3(uint32_t(fw.blocks)), kWG, lds,
                           s, nullptr, nullptr, na)
                : launch_k(nn_kernel<1, true>, dim3(uint32_t(fw.blocks)), kWG, 0, s, nullptr,
                           nullptr, na);
    if (e != hipSuccess) return e;
    // 2. the segments, in the production launch's shape
    ReplayArgs a{};
    a.tree = na.tree;
    a.m = m;
    a.perm = perm;
    a.spread = p.spread;
    a.wq = p.wq;
    a.tcap = kReplayCap;
    a.rows = w.rows;
    a.rcount = w.rcount;
    a.packed = w.packed;
    a.seg_total = w.seg_total;
    a.tally = w.tally;
    a.truncated = w.tally + 4;
    a.sink = w.sink;
    const dim3 grid{uint32_t(p.blocks)};
    if (p.small)
        replay_pack_kernel<kLeafChunkSmall><<<grid, kWG, 0, s>>>(a);
    else
        replay_pack_kernel<kLeafChunk><<<grid, kWG, 0, s>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    unsigned long long h[5];
    if ((e = hipMemcpyAsync(h, w.tally, sizeof h, hipMemcpyDeviceToHost, s)) != hipSuccess ||
        (e = hipStreamSynchronize(s)) != hipSuccess)
        return e;
    tally->visits = int64_t(h[0]);
    tally->bytes = int64_t(h[1]);
    tally->node_records = int64_t(h[2]);
    tally->leaf_points = int64_t(h[3]);
    tally->truncated = int64_t(h[4]);
    tally->blocks = p.blocks;
    tally->queries_per_wave = int32_t(p.wq);
    tally->spread = p.spread ? 1 : 0;
    // 3. the timed replays
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if ((e = hipEventCreate(&e0)) != hipSuccess) return e;
    if ((e = hipEventCreate(&e1)) != hipSuccess) {
        (void)hipEventDestroy(e0);
        return e;
    }
    for (int32_t r = 0; r < reps && e == hipSuccess; ++r) {
        e = p.small ? launch_k(replay_kernel<kLeafChunkSmall>, grid, kWG, 0, s, e0, e1, a)
                    : launch_k(replay_kernel<kLeafChunk>, grid, kWG, 0, s, e0, e1, a);
        if (e == hipSuccess) e = hipEventSynchronize(e1);
        if (e == hipSuccess) e = hipEventElapsedTime(&ms_out[r], e0, e1);
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    return e;
}

hipError_t launch_icp_reject(const DeviceTree &t, const float *src, int64_t n, const double *R,
                             const double *tv, double kk, const IcpWorkspace &ws, double *sums_out,
                             double *stat_out, uint8_t *kept, hipStream_t s, uint64_t *done,
                             uint64_t seq, const IcpLoop *loop)
{
    RejArgs a{};
    if (loop) a.rt_dev = loop->state->rt1;
    a.tree = tree_view(t);
    a.src = src;
    a.n = n;
    for (int k = 0; k < 9; ++k) a.R[k] = R[k];
    for (int k = 0; k < 3; ++k) {
        a.t[k] = tv[k];
        a.c[k] = t.center[k];
    }
    a.kk = kk;
    a.mslot = ws.mslot;
    a.md2 = ws.md2;
    a.partials = ws.partials;
    a.stat = ws.stat;
    a.kept = kept;
    const int32_t nb = int32_t(std::min<int64_t>(std::max<int64_t>((n + kWG - 1) / kWG, 1),
                                                 kIcpMaxBlocks));
    icp_residual_kernel<<<dim3(uint32_t(nb)), kWG, 0, s>>>(a);
    residual_stat_kernel<<<1, kWG, 0, s>>>(a.partials, nb, kk, a.stat);
    icp_reject_kernel<<<dim3(uint32_t(nb)), kWG, 0, s>>>(a);
    if (loop)
        launch_icp_loop_step(a.partials, nb, *loop, t.center, s);
    else
        launch_reduce_partials(a.partials, nb, nullptr, 0, sums_out, a.stat, stat_out, done, seq,
                               s);
    return hipGetLastError();
}

int batch_max_pairs() { return kBatchMax; }

int32_t batch_groups(int64_t n) { return int32_t((n + kWG - 1) / kWG); }

size_t icp_batch_ws_bytes(int32_t B, const int64_t *n)
{
    int64_t total = 0;
    for (int32_t p = 0; p < B; ++p) total += batch_groups(n[p]);
    size_t hints = 0;
    for (int32_t p = 0; p < B; ++p) hints += align256(size_t(n[p]) * 4);
    return align256(size_t(kS) * size_t(total) * 8) + batch_loop_bytes(B) + hints;
}

uint32_t *batch_hint(void *ws, int32_t total, int32_t B, const int64_t *n, int32_t p)
{
    size_t off = align256(size_t(kS) * size_t(total) * 8) + batch_loop_bytes(B);
    for (int32_t q = 0; q < p; ++q) off += align256(size_t(n[q]) * 4);
    return reinterpret_cast<uint32_t *>(static_cast<char *>(ws) + off);
}

size_t batch_loop_bytes(int32_t B)
{
    return size_t(B) * (align256(sizeof(IcpLoopState)) + align256(sizeof(IcpLoopOut)));
}

IcpLoopState *batch_loop_state(void *ws, int32_t total, int32_t p)
{
    return reinterpret_cast<IcpLoopState *>(static_cast<char *>(ws) +
                                            align256(size_t(kS) * size_t(total) * 8) +
                                            size_t(p) * align256(sizeof(IcpLoopState)));
}

IcpLoopOut *batch_loop_out(void *ws, int32_t total, int32_t B, int32_t p)
{
    return reinterpret_cast<IcpLoopOut *>(static_cast<char *>(ws) +
                                          align256(size_t(kS) * size_t(total) * 8) +
                                          size_t(B) * align256(sizeof(IcpLoopState)) +
                                          size_t(p) * align256(sizeof(IcpLoopOut)));
}

// One lane per pair: each record's header from its state (set by the host).
__global__ __launch_bounds__(64) void batch_loop_init_kernel(int32_t B, IcpLoopState *st0,
                                                             IcpLoopOut *out0, size_t st_stride,
                                                             size_t out_stride)
{
    const int32_t p = int32_t(blockIdx.x * 64 + threadIdx.x);
    if (p >= B) return;
    const IcpLoopState *st = reinterpret_cast<const IcpLoopState *>(
        reinterpret_cast<const char *>(st0) + size_t(p) * st_stride);
    IcpLoopOut *out = reinterpret_cast<IcpLoopOut *>(reinterpret_cast<char *>(out0) +
                                                     size_t(p) * out_stride);
    for (int k = 0; k < 12; ++k) out->rt[k] = st->rt[k];
    out->iters = 0;
    out->status = 0;
    out->fail_iter = -1;
    out->fail_phase = 0;
    out->stopped = 0;
}

hipError_t launch_batch_loop_init(int32_t B, void *ws, int32_t total, hipStream_t s)
{
    batch_loop_init_kernel<<<dim3(uint32_t((B + 63) / 64)), 64, 0, s>>>(
        B, batch_loop_state(ws, total, 0), batch_loop_out(ws, total, B, 0),
        align256(sizeof(IcpLoopState)), align256(sizeof(IcpLoopOut)));
    return hipGetLastError();
}

hipError_t launch_icp_batch(int32_t B, const BatchJob *jobs, float bound2, void *ws, int32_t total,
                            hipStream_t s, uint64_t seq, int32_t iter, double eps)
{
    BatchArgs a{};
    a.seq = seq;
    a.iter = iter;
    a.eps = eps;
    a.B = B;
    a.total = total;
    a.init = host_bound_key(bound2);
    a.partials = static_cast<double *>(ws);
    int64_t slots = 0;
    int32_t depth = 0;     // the deepest tree sets the launch's LDS
    int32_t max_leaf = 0;  // the largest leaf, the leaf batch
    for (int32_t p = 0; p < B; ++p) {
        const BatchJob &J = jobs[p];
        BatchPair &P = a.p[p];
        P.tree = tree_view(*J.tree);
        depth = J.tree->depth > depth ? J.tree->depth : depth;
        max_leaf = J.tree->max_leaf > max_leaf ? J.tree->max_leaf : max_leaf;
        P.src = J.src;
        P.n = J.n;
        for (int k = 0; k < 9; ++k) P.R[k] = J.R[k];
        for (int k = 0; k < 3; ++k) {
            P.t[k] = J.t[k];
            P.c[k] = J.tree->center[k];
        }
        P.nb = batch_groups(J.n);
        P.part = J.part;
        P.sums = J.sums;
        P.done = J.done;
        P.st = J.st;
        P.out = J.out;
        P.hint = J.hint;
        P.hint_in = J.hint_in;
        const int kx = (kNumXcd - p + B - 1) / B;
        const int64_t per_xcd = (P.nb + kx - 1) / kx;
        slots = per_xcd > slots ? per_xcd : slots;
    }
    const bool warm = B > 0 && jobs[0].hint_in;  // every pair of a launch is at one iteration
    void (*kb)(BatchArgs) =
        max_leaf <= kLeafChunkSmall
            ? (warm ? icp_batch_kernel<kLeafChunkSmall, true> : icp_batch_kernel<kLeafChunkSmall>)
            : (warm ? icp_batch_kernel<kLeafChunk, true> : icp_batch_kernel<kLeafChunk>);
    kb<<<dim3(uint32_t(slots * kNumXcd)), kWG, lbs_bytes(depth), s>>>(a);
    batch_reduce_kernel<<<dim3(uint32_t(B)), kWG, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace kdnn
