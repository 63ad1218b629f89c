// Voxel-grid down-sampling on gfx950 (CUDA-KDTree ICP article, §4.3: the
// voxel filter that shrinks a cloud before its tree is built).
//
// Voxel of a point: floor(p_a / leaf) per axis, the quotient in fp64.  Every
// occupied voxel yields the mean of its points: fp64 sums in ascending point
// index, divided by the count, one round-to-nearest cast to fp32.  Voxels are
// listed by ascending linear key over the grid the occupied voxels span
// (x fastest).  Points with a non-finite coordinate belong to no voxel.
//
// Steps (all streaming, HBM-bound; no step depends on thread timing):
//   1. bbox: fp32 min / max of the finite points and their count (exact,
//      order-independent), so the host can size the key grid;
//   2. keys: linear voxel key per point (non-finite: one past the last key);
//   3. stable LSD radix sort of (key, index), 8 bits per pass, only as many
//      passes as the key range needs -- equal keys keep index order;
//   4. segment heads: per 2048-key tile, count key changes, scan the tile
//      counts, then write each voxel's first sorted position;
//   5. the points' coordinates gathered into sorted order (one lane per
//      point), so that
//   6. one lane per voxel sums its segment -- now one contiguous run -- in
//      sorted (= index) order.  Summing straight from the gather would make
//      each lane walk its voxel's points one dependent random load at a time
//      (the largest voxels of a LiDAR cloud at 0.2 m hold ~200 points).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "kdnn_internal.hpp"

namespace kdnn {

namespace {

constexpr int kVoxThreads = 256;
constexpr int kVoxItems = 8;
constexpr int kVoxTile = kVoxThreads * kVoxItems;  // same tile as the radix passes
constexpr int kVoxBlocks = 1024;                   // bbox partials

size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

int32_t vox_tiles(int64_t n) { return int32_t((n + kVoxTile - 1) / kVoxTile); }

__device__ __forceinline__ bool finite3(float x, float y, float z)
{
    return isfinite(x) && isfinite(y) && isfinite(z);
}

__global__ __launch_bounds__(kVoxThreads) void voxel_bbox_kernel(const float *xyz, int64_t n,
                                                                 float *part)
{
    __shared__ float red[7][kVoxThreads];
    float lo[3] = {INFINITY, INFINITY, INFINITY}, hi[3] = {-INFINITY, -INFINITY, -INFINITY};
    float cnt = 0.0f;  // < 2^24 per lane: exact
    for (int64_t i = int64_t(blockIdx.x) * kVoxThreads + threadIdx.x; i < n;
         i += int64_t(gridDim.x) * kVoxThreads) {
        const float x = xyz[3 * i], y = xyz[3 * i + 1], z = xyz[3 * i + 2];
        if (!finite3(x, y, z)) continue;
        lo[0] = fminf(lo[0], x); lo[1] = fminf(lo[1], y); lo[2] = fminf(lo[2], z);
        hi[0] = fmaxf(hi[0], x); hi[1] = fmaxf(hi[1], y); hi[2] = fmaxf(hi[2], z);
        cnt += 1.0f;
    }
    for (int a = 0; a < 3; ++a) {
        red[a][threadIdx.x] = lo[a];
        red[3 + a][threadIdx.x] = hi[a];
    }
    red[6][threadIdx.x] = cnt;
    __syncthreads();
    for (int w = kVoxThreads / 2; w > 0; w >>= 1) {
        if (threadIdx.x < w) {
            for (int a = 0; a < 3; ++a) {
                red[a][threadIdx.x] = fminf(red[a][threadIdx.x], red[a][threadIdx.x + w]);
                red[3 + a][threadIdx.x] = fmaxf(red[3 + a][threadIdx.x], red[3 + a][threadIdx.x + w]);
            }
            red[6][threadIdx.x] += red[6][threadIdx.x + w];  // <= 2^24 per block: exact
        }
        __syncthreads();
    }
    if (threadIdx.x < 7) part[int64_t(threadIdx.x) * kVoxBlocks + blockIdx.x] = red[threadIdx.x][0];
}

// One work-group: combine the partials of `nb` blocks; the finite count is
// summed as an integer.
__global__ __launch_bounds__(kVoxThreads) void voxel_bbox_final_kernel(const float *part, int nb,
                                                                       float *bbox)
{
    __shared__ float red[6][kVoxThreads];
    __shared__ unsigned long long cnt;
    if (threadIdx.x == 0) cnt = 0ull;
    float v[6] = {INFINITY, INFINITY, INFINITY, -INFINITY, -INFINITY, -INFINITY};
    unsigned long long c = 0ull;
    for (int b = threadIdx.x; b < nb; b += kVoxThreads) {
        for (int a = 0; a < 3; ++a) {
            v[a] = fminf(v[a], part[int64_t(a) * kVoxBlocks + b]);
            v[3 + a] = fmaxf(v[3 + a], part[int64_t(3 + a) * kVoxBlocks + b]);
        }
        c += (unsigned long long)part[int64_t(6) * kVoxBlocks + b];
    }
    for (int a = 0; a < 6; ++a) red[a][threadIdx.x] = v[a];
    __syncthreads();
    atomicAdd(&cnt, c);
    for (int w = kVoxThreads / 2; w > 0; w >>= 1) {
        if (threadIdx.x < w) {
            for (int a = 0; a < 3; ++a) {
                red[a][threadIdx.x] = fminf(red[a][threadIdx.x], red[a][threadIdx.x + w]);
                red[3 + a][threadIdx.x] = fmaxf(red[3 + a][threadIdx.x], red[3 + a][threadIdx.x + w]);
            }
        }
        __syncthreads();
    }
    if (threadIdx.x < 6) bbox[threadIdx.x] = red[threadIdx.x][0];
    if (threadIdx.x == 0) {
        const uint32_t c32 = uint32_t(cnt);
        bbox[6] = __uint_as_float(c32);
    }
}

struct VoxKey {
    const float *xyz;
    int64_t n;
    double leaf;
    int64_t vmin[3];
    uint32_t dims[3];
    uint32_t sentinel;
};

__device__ __forceinline__ int64_t vox_coord(float p, double leaf)
{
    return int64_t(floor(double(p) / leaf));
}

__global__ __launch_bounds__(kVoxThreads) void voxel_key_kernel(VoxKey a, uint32_t *keys,
                                                                int32_t *vals)
{
    for (int64_t i = int64_t(blockIdx.x) * kVoxThreads + threadIdx.x; i < a.n;
         i += int64_t(gridDim.x) * kVoxThreads) {
        const float x = a.xyz[3 * i], y = a.xyz[3 * i + 1], z = a.xyz[3 * i + 2];
        uint32_t key = a.sentinel;
        if (finite3(x, y, z)) {
            // in range: every finite point lies in [min, max], whose voxels
            // bound the grid (floor and a division by leaf > 0 are monotone)
            const uint32_t vx = uint32_t(vox_coord(x, a.leaf) - a.vmin[0]);
            const uint32_t vy = uint32_t(vox_coord(y, a.leaf) - a.vmin[1]);
            const uint32_t vz = uint32_t(vox_coord(z, a.leaf) - a.vmin[2]);
            key = vx + a.dims[0] * (vy + a.dims[1] * vz);
        }
        keys[i] = key;
        vals[i] = int32_t(i);
    }
}

__device__ __forceinline__ bool is_head(const uint32_t *keys, int64_t e, int64_t n,
                                        uint32_t sentinel)
{
    if (e >= n) return false;
    const uint32_t k = keys[e];
    return k != sentinel && (e == 0 || keys[e - 1] != k);
}

// Tile t's number of voxel heads.
__global__ __launch_bounds__(kVoxThreads) void voxel_heads_kernel(const uint32_t *keys, int64_t n,
                                                                  uint32_t sentinel,
                                                                  uint32_t *tile_heads)
{
    __shared__ uint32_t wsum[kVoxThreads / 64];
    const int64_t base = int64_t(blockIdx.x) * kVoxTile;
    uint32_t c = 0;
#pragma unroll
    for (int r = 0; r < kVoxItems; ++r)
        c += is_head(keys, base + r * kVoxThreads + threadIdx.x, n, sentinel) ? 1u : 0u;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) c += uint32_t(__shfl_xor(int(c), off, 64));
    if (lane == 0) wsum[w] = c;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t s = 0;
        for (int k = 0; k < kVoxThreads / 64; ++k) s += wsum[k];
        tile_heads[blockIdx.x] = s;
    }
}

// starts[voxel] = sorted position of its first point.  tile_heads holds the
// exclusive scan of the per-tile head counts.
__global__ __launch_bounds__(kVoxThreads) void voxel_starts_kernel(const uint32_t *keys, int64_t n,
                                                                   uint32_t sentinel,
                                                                   const uint32_t *tile_heads,
                                                                   int32_t *starts)
{
    __shared__ uint32_t wsum[kVoxThreads / 64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const uint64_t below = (uint64_t(1) << lane) - 1u;
    const int64_t base = int64_t(blockIdx.x) * kVoxTile;
    uint32_t run = tile_heads[blockIdx.x];
#pragma unroll
    for (int r = 0; r < kVoxItems; ++r) {
        const int64_t e = base + r * kVoxThreads + threadIdx.x;
        const bool h = is_head(keys, e, n, sentinel);
        const uint64_t bal = __ballot(h);
        if (lane == 0) wsum[w] = uint32_t(__popcll(bal));
        __syncthreads();
        uint32_t before = 0, total = 0;
        for (int k = 0; k < kVoxThreads / 64; ++k) {
            before += k < w ? wsum[k] : 0u;
            total += wsum[k];
        }
        if (h) starts[run + before + uint32_t(__popcll(bal & below))] = int32_t(e);
        run += total;
        __syncthreads();
    }
}

// sorted[k] = the coordinates of the point at sorted position k < n_finite
// (the finite points; non-finite ones carry the largest key and sort last).
__global__ __launch_bounds__(kVoxThreads) void voxel_gather_kernel(const float *xyz,
                                                                   const int32_t *vals,
                                                                   int64_t n_finite, float *sorted)
{
    for (int64_t k = int64_t(blockIdx.x) * kVoxThreads + threadIdx.x; k < n_finite;
         k += int64_t(gridDim.x) * kVoxThreads) {
        const int64_t i = vals[k];
        const float x = xyz[3 * i], y = xyz[3 * i + 1], z = xyz[3 * i + 2];
        sorted[3 * k] = x;
        sorted[3 * k + 1] = y;
        sorted[3 * k + 2] = z;
    }
}

// Lane v: the mean of voxel v's points, summed in sorted (index) order.  The
// segment is read kChunk points at a time (independent loads in flight), the
// additions stay in order.
__global__ __launch_bounds__(kVoxThreads) void voxel_centroid_kernel(
    const float *sorted, const int32_t *starts, const uint32_t *nvox, int64_t n_finite,
    float *out, int32_t *counts)
{
    constexpr int kChunk = 8;
    const int64_t m = int64_t(*nvox);
    for (int64_t v = int64_t(blockIdx.x) * kVoxThreads + threadIdx.x; v < m;
         v += int64_t(gridDim.x) * kVoxThreads) {
        const int64_t s = starts[v];
        const int64_t e = v + 1 < m ? int64_t(starts[v + 1]) : n_finite;
        double sx = 0.0, sy = 0.0, sz = 0.0;
        for (int64_t k0 = s; k0 < e; k0 += kChunk) {
            float px[kChunk], py[kChunk], pz[kChunk];
#pragma unroll
            for (int j = 0; j < kChunk; ++j) {
                const int64_t k = k0 + j < e ? k0 + j : e - 1;  // in bounds; unused past e
                px[j] = sorted[3 * k];
                py[j] = sorted[3 * k + 1];
                pz[j] = sorted[3 * k + 2];
            }
#pragma unroll
            for (int j = 0; j < kChunk; ++j) {
                if (k0 + j < e) {
                    sx += double(px[j]);
                    sy += double(py[j]);
                    sz += double(pz[j]);
                }
            }
        }
        const double c = double(e - s);
        out[3 * v] = float(sx / c);
        out[3 * v + 1] = float(sy / c);
        out[3 * v + 2] = float(sz / c);
        if (counts) counts[v] = int32_t(e - s);
    }
}

uint32_t grid_of(int64_t n, int64_t per)
{
    int64_t b = (n + per - 1) / per;
    if (b < 1) b = 1;
    if (b > 65536) b = 65536;
    return uint32_t(b);
}

}  // namespace

size_t voxel_ws_bytes(int64_t n)
{
    if (n <= 0) return 0;
    const size_t nn = size_t(n);
    const int32_t nt = radix_tiles(n);
    return 4 * align256(nn * 4) + align256(size_t(256) * nt * 4) + align256(256 * 4) +
           align256(size_t(vox_tiles(n)) * 4) + align256(nn * 4) +
           align256(size_t(7) * kVoxBlocks * 4) + 256 + 256 + align256(nn * 12);
}

VoxelWorkspace carve_voxel_workspace(void *ws, int64_t n)
{
    VoxelWorkspace w{};
    char *p = static_cast<char *>(ws);
    const size_t a = align256(size_t(n) * 4);
    w.keys_a = reinterpret_cast<uint32_t *>(p);
    w.keys_b = reinterpret_cast<uint32_t *>(p + a);
    w.vals_a = reinterpret_cast<int32_t *>(p + 2 * a);
    w.vals_b = reinterpret_cast<int32_t *>(p + 3 * a);
    p += 4 * a;
    w.hist = reinterpret_cast<uint32_t *>(p);
    p += align256(size_t(256) * radix_tiles(n) * 4);
    w.totals = reinterpret_cast<uint32_t *>(p);
    p += align256(256 * 4);
    w.tile_heads = reinterpret_cast<uint32_t *>(p);
    p += align256(size_t(vox_tiles(n)) * 4);
    w.starts = reinterpret_cast<int32_t *>(p);
    p += a;
    w.bbox_part = reinterpret_cast<float *>(p);
    p += align256(size_t(7) * kVoxBlocks * 4);
    w.bbox = reinterpret_cast<float *>(p);
    p += 256;
    w.nvox = reinterpret_cast<uint32_t *>(p);
    p += 256;
    w.sorted = reinterpret_cast<float *>(p);
    return w;
}

hipError_t launch_voxel_bbox(const float *xyz, int64_t n, const VoxelWorkspace &w, hipStream_t s)
{
    uint32_t nb = grid_of(n, int64_t(kVoxThreads) * 4);
    if (nb > uint32_t(kVoxBlocks)) nb = kVoxBlocks;
    voxel_bbox_kernel<<<nb, kVoxThreads, 0, s>>>(xyz, n, w.bbox_part);
    voxel_bbox_final_kernel<<<1, kVoxThreads, 0, s>>>(w.bbox_part, int(nb), w.bbox);
    return hipGetLastError();
}

hipError_t launch_voxel_filter(const float *xyz, int64_t n, double leaf, const int64_t *vmin,
                               const uint32_t *dims, uint32_t sentinel, int passes,
                               int64_t n_finite, const VoxelWorkspace &w, float *out,
                               int32_t *counts, hipStream_t s)
{
    VoxKey k{};
    k.xyz = xyz;
    k.n = n;
    k.leaf = leaf;
    for (int a = 0; a < 3; ++a) {
        k.vmin[a] = vmin[a];
        k.dims[a] = dims[a];
    }
    k.sentinel = sentinel;
    voxel_key_kernel<<<grid_of(n, kVoxThreads), kVoxThreads, 0, s>>>(k, w.keys_a, w.vals_a);
    uint32_t *kin = w.keys_a, *kout = w.keys_b;
    int32_t *vin = w.vals_a, *vout = w.vals_b;
    hipError_t e = hipGetLastError();
    for (int p = 0; p < passes && e == hipSuccess; ++p) {
        e = launch_radix_pass(kin, vin, 8 * p, kout, vout, n, w.hist, w.totals, s);
        uint32_t *tk = kin; kin = kout; kout = tk;
        int32_t *tv = vin; vin = vout; vout = tv;
    }
    if (e != hipSuccess) return e;
    const int32_t nt = vox_tiles(n);
    voxel_heads_kernel<<<nt, kVoxThreads, 0, s>>>(kin, n, sentinel, w.tile_heads);
    if ((e = launch_scan_row(w.tile_heads, nt, w.nvox, s)) != hipSuccess) return e;
    voxel_starts_kernel<<<nt, kVoxThreads, 0, s>>>(kin, n, sentinel, w.tile_heads, w.starts);
    voxel_gather_kernel<<<grid_of(n_finite, kVoxThreads), kVoxThreads, 0, s>>>(xyz, vin, n_finite,
                                                                             w.sorted);
    voxel_centroid_kernel<<<grid_of(n_finite, kVoxThreads), kVoxThreads, 0, s>>>(
        w.sorted, w.starts, w.nvox, n_finite, out, counts);
    return hipGetLastError();
}

}  // namespace kdnn
