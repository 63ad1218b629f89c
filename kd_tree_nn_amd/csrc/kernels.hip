// HIP kernels for gfx950 (CDNA4, wave64): exact KD-tree nearest-neighbour
// traversal, the fused ICP correspondence + fp64 reduction, the Morton
// ordering of queries (two stable 8-bit radix passes), and the rigid
// transform.  Built with -ffp-contract=off: every fp32 product and sum of
// the distance code is rounded on its own, exactly as the host-side
// definition writes it.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "kdnn_internal.hpp"

namespace kdnn {

constexpr int kWG = 256;                          // traversal work-group: 4 wave64
constexpr int kSortThreads = 256;
constexpr int kSortItems = 8;
constexpr int kSortTile = kSortThreads * kSortItems;  // keys per radix tile
constexpr int kKeyBits = 16;                      // Morton prefix used for ordering
constexpr int kScanThreads = 1024;
constexpr int kIcpMaxBlocks = 4096;
constexpr int kNumXcd = 8;
constexpr int kS = KDNN_SUMS_DOUBLES;

// ------------------------------------------------------------------ helpers

// Work-groups are dealt round-robin to the 8 XCDs (each with its own L2).
// Map them so that every XCD works on one contiguous run of logical blocks,
// i.e. on one spatially coherent slice of the Morton-ordered queries.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t b, uint32_t nb)
{
    const uint32_t x = b % kNumXcd, slot = b / kNumXcd;
    const uint32_t q = nb / kNumXcd, r = nb % kNumXcd;
    return x * q + (x < r ? x : r) + slot;
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
// point that could beat or tie the best is never skipped; together with the
// (distance, index) comparison the result is the lowest-index nearest point
// whatever the visiting order.
//
// No stack: the node index spells the path from the root, and bit d of
// `far` records whether the path node at depth d+1 is a far child.  After a
// subtree is done, the next subtree is the far sibling of the deepest path
// node that is still a near child.
struct Best {
    float d;
    int32_t idx;
    float mx, my, mz;  // coordinates of the best target point
};

template <bool STATS>
__device__ __forceinline__ void nn_search(const float4 *__restrict__ nodes,
                                          const float4 *__restrict__ pts, uint32_t first_leaf,
                                          float qx, float qy, float qz, Best &b, uint32_t &cn,
                                          uint32_t &cp)
{
    b.d = INFINITY;
    b.idx = -1;
    b.mx = b.my = b.mz = 0.0f;
    if (!(isfinite(qx) && isfinite(qy) && isfinite(qz))) return;
    uint32_t i = 1, far = 0;
    for (;;) {
        const float4 A = nodes[2 * i];      // lo.x lo.y lo.z hi.x
        const float4 B = nodes[2 * i + 1];  // hi.y hi.z w6 w7
        if (STATS) ++cn;
        const float gx = qx < A.x ? A.x - qx : (qx > A.w ? qx - A.w : 0.0f);
        const float gy = qy < A.y ? A.y - qy : (qy > B.x ? qy - B.x : 0.0f);
        const float gz = qz < A.z ? A.z - qz : (qz > B.y ? qz - B.y : 0.0f);
        const float lb = (gx * gx + gy * gy) + gz * gz;
        if (lb <= b.d && lb < INFINITY) {
            if (i < first_leaf) {
                const uint32_t axis = __float_as_uint(B.w);
                const float qa = axis == 0 ? qx : (axis == 1 ? qy : qz);
                i = 2 * i + (qa >= B.z ? 1u : 0u);
                continue;
            }
            const int32_t begin = __float_as_int(B.z);
            const int32_t count = __float_as_int(B.w);
            for (int32_t k = 0; k < count; ++k) {
                const float4 p = pts[begin + k];
                const float dx = p.x - qx;
                const float dy = p.y - qy;
                const float dz = p.z - qz;
                const float d = (dx * dx + dy * dy) + dz * dz;
                const int32_t j = __float_as_int(p.w);
                if (d < b.d || (d == b.d && j < b.idx)) {
                    b.d = d;
                    b.idx = j;
                    b.mx = p.x;
                    b.my = p.y;
                    b.mz = p.z;
                }
            }
            if (STATS) cp += uint32_t(count);
        }
        const uint32_t dep = 31u - uint32_t(__clz(int(i)));
        const uint32_t open = ~far & ((1u << dep) - 1u);
        if (open == 0) break;
        const uint32_t h = 31u - uint32_t(__clz(int(open)));
        i = (i >> (dep - h - 1u)) ^ 1u;
        far = (far & ((1u << h) - 1u)) | (1u << h);
    }
}

struct NnArgs {
    const float4 *nodes;
    const float4 *pts;
    uint32_t first_leaf;
    const float *q;
    int64_t m;
    const int32_t *perm;
    int32_t *idx;
    float *d2;
    uint32_t *cnt_nodes;
    uint32_t *cnt_pts;
};

template <bool STATS>
__global__ __launch_bounds__(kWG) void nn_kernel(NnArgs a)
{
    const uint32_t nb = gridDim.x;
    const uint32_t blk = xcd_remap(blockIdx.x, nb);
    for (int64_t k = int64_t(blk) * kWG + threadIdx.x; k < a.m; k += int64_t(nb) * kWG) {
        const int64_t i = a.perm ? int64_t(a.perm[k]) : k;
        const float qx = a.q[3 * i], qy = a.q[3 * i + 1], qz = a.q[3 * i + 2];
        Best b;
        uint32_t cn = 0, cp = 0;
        nn_search<STATS>(a.nodes, a.pts, a.first_leaf, qx, qy, qz, b, cn, cp);
        a.idx[i] = b.idx;
        a.d2[i] = b.d;
        if (STATS) {
            if (a.cnt_nodes) a.cnt_nodes[i] = cn;
            if (a.cnt_pts) a.cnt_pts[i] = cp;
        }
    }
}

// ------------------------------------------------------ fused ICP kernel
//
// Per source point: q = fl32(R s + t) evaluated in fp64 with a fixed
// association; nearest target point m; accumulate in fp64, shifted by c,
//   (s-c), (m-c), (s-c)(m-c)^T, d2, 1.
// Per lane -> wave (xor butterfly, lane 0 keeps the total) -> work-group
// (waves summed in order) -> per-group partials; the last group to finish
// (atomic ticket) sums the partials in a fixed order.  The result does not
// depend on scheduling.
struct IcpArgs {
    const float4 *nodes;
    const float4 *pts;
    uint32_t first_leaf;
    const float *src;
    int64_t n;
    const int32_t *perm;
    double R[9];
    double t[3];
    double c[3];
    double *partials;  // [kS][nb], component-major
    uint32_t *ticket;
    double *sums;      // [kS]
    int32_t *idx;
    float *d2;
};

__device__ __forceinline__ float rigid_row(double r0, double r1, double r2, double tr, double x,
                                           double y, double z)
{
    return float(((r0 * x + r1 * y) + r2 * z) + tr);
}

// Sum acc[] over the work-group; thread c < kS of wave 0 gets component c
// in *out (fixed order: lanes by xor butterfly, then waves 0..3).
__device__ __forceinline__ void block_sum(double (&acc)[kS], double *red /* LDS [4][kS] */,
                                          double *out, int64_t out_stride)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int c = 0; c < kS; ++c) {
        double v = acc[c];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
        acc[c] = v;
    }
    if (lane == 0) {
#pragma unroll
        for (int c = 0; c < kS; ++c) red[w * kS + c] = acc[c];
    }
    __syncthreads();
    if (threadIdx.x < kS) {
        double s = 0.0;
        for (int ww = 0; ww < kWG / 64; ++ww) s += red[ww * kS + threadIdx.x];
        out[threadIdx.x * out_stride] = s;
    }
}

__global__ __launch_bounds__(kWG) void icp_fused_kernel(IcpArgs a)
{
    __shared__ double red[(kWG / 64) * kS];
    __shared__ uint32_t is_last;
    double acc[kS];
#pragma unroll
    for (int c = 0; c < kS; ++c) acc[c] = 0.0;

    const uint32_t nb = gridDim.x;
    const uint32_t blk = xcd_remap(blockIdx.x, nb);
    for (int64_t k = int64_t(blk) * kWG + threadIdx.x; k < a.n; k += int64_t(nb) * kWG) {
        const int64_t i = a.perm ? int64_t(a.perm[k]) : k;
        const double X = a.src[3 * i], Y = a.src[3 * i + 1], Z = a.src[3 * i + 2];
        const float qx = rigid_row(a.R[0], a.R[1], a.R[2], a.t[0], X, Y, Z);
        const float qy = rigid_row(a.R[3], a.R[4], a.R[5], a.t[1], X, Y, Z);
        const float qz = rigid_row(a.R[6], a.R[7], a.R[8], a.t[2], X, Y, Z);
        Best b;
        uint32_t cn = 0, cp = 0;
        nn_search<false>(a.nodes, a.pts, a.first_leaf, qx, qy, qz, b, cn, cp);
        if (a.idx) a.idx[i] = b.idx;
        if (a.d2) a.d2[i] = b.d;
        if (b.idx >= 0) {
            const double s0 = X - a.c[0], s1 = Y - a.c[1], s2 = Z - a.c[2];
            const double m0 = double(b.mx) - a.c[0], m1 = double(b.my) - a.c[1],
                         m2 = double(b.mz) - a.c[2];
            acc[0] += s0; acc[1] += s1; acc[2] += s2;
            acc[3] += m0; acc[4] += m1; acc[5] += m2;
            acc[6] += s0 * m0; acc[7] += s0 * m1; acc[8] += s0 * m2;
            acc[9] += s1 * m0; acc[10] += s1 * m1; acc[11] += s1 * m2;
            acc[12] += s2 * m0; acc[13] += s2 * m1; acc[14] += s2 * m2;
            acc[15] += double(b.d);
            acc[16] += 1.0;
        }
    }
    block_sum(acc, red, a.partials + blockIdx.x, nb);

    // Publish this group's partials, then take a ticket; the last group reduces.
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) is_last = (atomicAdd(a.ticket, 1u) == nb - 1) ? 1u : 0u;
    __syncthreads();
    if (!is_last) return;
    __threadfence();
#pragma unroll
    for (int c = 0; c < kS; ++c) acc[c] = 0.0;
    for (uint32_t g = threadIdx.x; g < nb; g += kWG) {
#pragma unroll
        for (int c = 0; c < kS; ++c) acc[c] += a.partials[int64_t(c) * nb + g];
    }
    __syncthreads();  // red[] is reused
    block_sum(acc, red, a.sums, 1);
    if (threadIdx.x == 0) atomicExch(a.ticket, 0u);
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

__global__ void zero_u32_kernel(uint32_t *p, int64_t n)
{
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += int64_t(gridDim.x) * blockDim.x)
        p[i] = 0u;
}

// ------------------------------------------------------- Morton ordering
//
// Queries are ordered by the top kKeyBits bits of their 30-bit Morton code
// in the target's bounding box (10 bits per axis, clamped), so that the 64
// lanes of a wave start from neighbouring points and walk mostly the same
// branches.  Stable LSD radix sort, two 8-bit passes; the permutation is a
// deterministic function of the input.

struct OrderArgs {
    const float *pts;
    int64_t m;
    float R[12];  // row-major R then t; used when moved != 0
    int32_t moved;
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
    return code >> (30 - kKeyBits);
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
    for (int r = 0; r < kSortItems; ++r) {
        const int64_t e = base + r * kSortThreads + threadIdx.x;
        if (e < oa.m) {
            const uint32_t key = FROM_POINTS ? order_key(oa, e) : keys[e];
            atomicAdd(&h[(key >> shift) & 255u], 1u);
        }
    }
    __syncthreads();
    hist[int64_t(threadIdx.x) * ntiles + blockIdx.x] = h[threadIdx.x];
}

// Exclusive scan of hist[0..total) (digit-major, so the result is each
// (digit, tile) pair's first output slot).  One work-group.
__global__ __launch_bounds__(kScanThreads) void radix_scan_kernel(uint32_t *hist, int64_t total,
                                                                  uint32_t *zero_me)
{
    __shared__ uint32_t sums[kScanThreads];
    const int64_t per = (total + kScanThreads - 1) / kScanThreads;
    const int64_t a = int64_t(threadIdx.x) * per;
    const int64_t e = a + per < total ? a + per : total;
    uint32_t s = 0;
    for (int64_t k = a; k < e; ++k) s += hist[k];
    sums[threadIdx.x] = s;
    __syncthreads();
    for (int off = 1; off < kScanThreads; off <<= 1) {
        const uint32_t v = threadIdx.x >= off ? sums[threadIdx.x - off] : 0u;
        __syncthreads();
        sums[threadIdx.x] += v;
        __syncthreads();
    }
    uint32_t run = threadIdx.x ? sums[threadIdx.x - 1] : 0u;
    for (int64_t k = a; k < e; ++k) {
        const uint32_t v = hist[k];
        hist[k] = run;
        run += v;
    }
    if (zero_me && threadIdx.x == 0) *zero_me = 0u;
}

// Stable scatter of one tile.  Element e = tile*2048 + r*256 + tid is the
// r-th round of thread tid, so (r, tid) is the input order inside the tile.
// Within a wave, lanes holding the same digit are found with 8 ballots; the
// rank of an element = running count of its digit in this tile (earlier
// rounds) + counts of earlier waves in this round + lanes below it.
template <bool FROM_POINTS, bool WRITE_KEYS>
__global__ __launch_bounds__(kSortThreads) void radix_scatter_kernel(
    OrderArgs oa, const uint32_t *keys_in, const int32_t *vals_in, int shift,
    const uint32_t *hist, int32_t ntiles, uint32_t *keys_out, int32_t *vals_out)
{
    __shared__ uint32_t base[256];
    __shared__ uint32_t wcnt[kSortThreads / 64][256];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const uint64_t below = (uint64_t(1) << lane) - 1u;
    base[tid] = hist[int64_t(tid) * ntiles + blockIdx.x];
    const int64_t tbase = int64_t(blockIdx.x) * kSortTile;
    for (int r = 0; r < kSortItems; ++r) {
        const int64_t e = tbase + r * kSortThreads + tid;
        const bool valid = e < oa.m;
        uint32_t key = 0u;
        int32_t val = 0;
        if (valid) {
            key = FROM_POINTS ? order_key(oa, e) : keys_in[e];
            val = FROM_POINTS ? int32_t(e) : vals_in[e];
        }
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
    return align256(mm * 4) * 3 + align256(size_t(256) * sort_tiles(m) * 4);
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
    return w;
}

static int32_t icp_blocks(int64_t n)
{
    const int64_t b = (n + kWG - 1) / kWG;
    return int32_t(b < 1 ? 1 : (b > kIcpMaxBlocks ? kIcpMaxBlocks : b));
}

size_t icp_ws_bytes(int64_t n)
{
    if (n <= 0) return 0;
    return sort_workspace_bytes(n) + align256(size_t(kS) * kIcpMaxBlocks * 8) +
           align256(size_t(kS) * 8) + 256;
}

IcpWorkspace carve_icp_workspace(void *ws, int64_t n)
{
    IcpWorkspace w{};
    char *p = static_cast<char *>(ws);
    w.sort = carve_sort_workspace(ws, n);
    p += sort_workspace_bytes(n);
    w.partials = reinterpret_cast<double *>(p);
    p += align256(size_t(kS) * kIcpMaxBlocks * 8);
    w.sums = reinterpret_cast<double *>(p);
    p += align256(size_t(kS) * 8);
    w.ticket = reinterpret_cast<uint32_t *>(p);
    w.max_blocks = kIcpMaxBlocks;
    return w;
}

// --------------------------------------------------------------- launchers

static OrderArgs make_order_args(const DeviceTree &t, const float *pts, int64_t m, const float *R12)
{
    OrderArgs oa{};
    oa.pts = pts;
    oa.m = m;
    oa.moved = R12 ? 1 : 0;
    for (int k = 0; k < 12; ++k) oa.R[k] = R12 ? R12[k] : 0.0f;
    for (int k = 0; k < 3; ++k) {
        oa.lo[k] = t.box_lo[k];
        oa.inv[k] = t.box_inv[k];
    }
    return oa;
}

static hipError_t morton_order_impl(const DeviceTree &t, const float *pts, int64_t m,
                                    const float *R12, const SortWorkspace &ws, uint32_t *zero_me,
                                    const int32_t **perm, hipStream_t s)
{
    const OrderArgs oa = make_order_args(t, pts, m, R12);
    const int32_t nt = ws.ntiles;
    const int64_t total = int64_t(256) * nt;
    radix_hist_kernel<true><<<nt, kSortThreads, 0, s>>>(oa, nullptr, 0, ws.hist, nt);
    radix_scan_kernel<<<1, kScanThreads, 0, s>>>(ws.hist, total, zero_me);
    radix_scatter_kernel<true, true><<<nt, kSortThreads, 0, s>>>(oa, nullptr, nullptr, 0, ws.hist,
                                                                 nt, ws.keys_b, ws.vals_b);
    radix_hist_kernel<false><<<nt, kSortThreads, 0, s>>>(oa, ws.keys_b, 8, ws.hist, nt);
    radix_scan_kernel<<<1, kScanThreads, 0, s>>>(ws.hist, total, nullptr);
    radix_scatter_kernel<false, false><<<nt, kSortThreads, 0, s>>>(
        oa, ws.keys_b, ws.vals_b, 8, ws.hist, nt, nullptr, ws.vals_a);
    *perm = ws.vals_a;
    return hipGetLastError();
}

hipError_t launch_morton_order(const DeviceTree &t, const float *pts, int64_t m, const float *R12,
                               const SortWorkspace &ws, const int32_t **perm, hipStream_t s)
{
    return morton_order_impl(t, pts, m, R12, ws, nullptr, perm, s);
}

hipError_t launch_icp_order(const DeviceTree &t, const float *pts, int64_t m, const float *R12,
                            const IcpWorkspace &ws, const int32_t **perm, hipStream_t s)
{
    return morton_order_impl(t, pts, m, R12, ws.sort, ws.ticket, perm, s);
}

hipError_t launch_nn(const DeviceTree &t, const float *q, int64_t m, const int32_t *perm,
                     int32_t *idx, float *d2, uint32_t *cnt_nodes, uint32_t *cnt_pts, bool stats,
                     hipStream_t s)
{
    NnArgs a{};
    a.nodes = static_cast<const float4 *>(t.nodes);
    a.pts = static_cast<const float4 *>(t.points);
    a.first_leaf = t.first_leaf;
    a.q = q;
    a.m = m;
    a.perm = perm;
    a.idx = idx;
    a.d2 = d2;
    a.cnt_nodes = cnt_nodes;
    a.cnt_pts = cnt_pts;
    int64_t blocks = (m + kWG - 1) / kWG;
    if (blocks > (int64_t(1) << 20)) blocks = int64_t(1) << 20;
    if (stats)
        nn_kernel<true><<<dim3(uint32_t(blocks)), kWG, 0, s>>>(a);
    else
        nn_kernel<false><<<dim3(uint32_t(blocks)), kWG, 0, s>>>(a);
    return hipGetLastError();
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
                            double *sums_out, int32_t *idx, float *d2, hipStream_t s)
{
    IcpArgs a{};
    a.nodes = static_cast<const float4 *>(t.nodes);
    a.pts = static_cast<const float4 *>(t.points);
    a.first_leaf = t.first_leaf;
    a.src = src;
    a.n = n;
    a.perm = perm;
    for (int k = 0; k < 9; ++k) a.R[k] = R[k];
    for (int k = 0; k < 3; ++k) {
        a.t[k] = tv[k];
        a.c[k] = t.center[k];
    }
    a.partials = ws.partials;
    a.ticket = ws.ticket;
    a.sums = sums_out;
    a.idx = idx;
    a.d2 = d2;
    icp_fused_kernel<<<dim3(uint32_t(icp_blocks(n))), kWG, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_zero_u32(uint32_t *p, int64_t n, hipStream_t s)
{
    zero_u32_kernel<<<1, 64, 0, s>>>(p, n);
    return hipGetLastError();
}

}  // namespace kdnn
