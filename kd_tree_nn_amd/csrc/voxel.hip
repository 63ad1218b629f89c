// Voxel-grid down-sampling on gfx950 (CUDA-KDTree ICP article, §4.3: the
// voxel filter that shrinks a cloud before its tree is built).
//
// Voxel of a point: floor(p_a / leaf) per axis, the quotient in fp64.  Every
// occupied voxel yields the mean of its points: fp64 sums in ascending point
// index, divided by the count, one round-to-nearest cast to fp32.  Voxels are
// listed by ascending linear key over the grid the occupied voxels span
// (x fastest).  Points with a non-finite coordinate belong to no voxel.
//
// Steps, all on the device and all launched at once (the host reads back the
// voxel count and the grid's error code at the end, nothing in between; no
// step depends on thread timing):
//   1. bbox: per block, the fp32 min / max of the finite points and their
//      count (exact and order-independent);
//   2. keys: every block combines those partials into the key grid (fp64,
//      the same arithmetic in every block, so the same grid), then writes the
//      linear voxel key of its points (non-finite: one past the last key);
//   3. stable LSD radix sort of (key, index) with 8-bit digits.  Four passes
//      cover any 32-bit key; all four are launched and those the grid's key
//      range does not need return at once.  The last pass that runs writes
//      each point's coordinates at its sorted position in place of its index
//      (the gather costs no launch of its own).  8-bit digits beat 10 and 11
//      bits here (1M LiDAR points at 0.2 m: 200 / 208 / 229 us per call):
//      the wider histograms cost more per pass than the pass they save;
//   4. segment heads: per 2048-key tile, count key changes, then write each
//      voxel's first sorted position (each tile adds up the counts before it);
//   5. each voxel's segment -- one contiguous run -- is summed in sorted
//      (= index) order: by one lane for small voxels, by a wave for large
//      ones.  Summing straight from the unsorted cloud would make each lane
//      walk its voxel's points one dependent random load at a time (the
//      largest voxels of a LiDAR cloud hold ~200 points at 0.2 m, ~6,000 at
//      1 m).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "kdnn_internal.hpp"

namespace kdnn {

namespace {

constexpr int kVoxThreads = 256;
constexpr int kVoxWaves = kVoxThreads / 64;
constexpr int kVoxItems = 8;
constexpr int kVoxTile = kVoxThreads * kVoxItems;  // keys per sort / heads tile
constexpr int kVoxBlocks = 1024;                   // bbox partials
constexpr int kVoxDigitBits = 8;
constexpr int kVoxBins = 1 << kVoxDigitBits;
constexpr int kVoxBinsPerThread = kVoxBins / kVoxThreads;
constexpr int kVoxMaxPasses = (32 + kVoxDigitBits - 1) / kVoxDigitBits;

size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

int32_t vox_tiles(int64_t n) { return int32_t((n + kVoxTile - 1) / kVoxTile); }

__device__ __forceinline__ bool finite3(float x, float y, float z)
{
    return isfinite(x) && isfinite(y) && isfinite(z);
}

// Min / max / count over the wave, then over the block's waves (all exact:
// min, max and integer sums do not depend on the order).
struct BoxAcc {
    float lo[3], hi[3];
    uint32_t cnt;
};

__device__ __forceinline__ void wave_box(BoxAcc &b)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
#pragma unroll
        for (int a = 0; a < 3; ++a) {
            b.lo[a] = fminf(b.lo[a], __shfl_xor(b.lo[a], off, 64));
            b.hi[a] = fmaxf(b.hi[a], __shfl_xor(b.hi[a], off, 64));
        }
        b.cnt += uint32_t(__shfl_xor(int(b.cnt), off, 64));
    }
}

// Combines the waves' results in thread 0 (the others' copy is left as is).
__device__ __forceinline__ void block_box(BoxAcc &b, BoxAcc *lds /* [kVoxWaves] */)
{
    wave_box(b);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 0) lds[w] = b;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int k = 1; k < kVoxWaves; ++k) {
            for (int a = 0; a < 3; ++a) {
                b.lo[a] = fminf(b.lo[a], lds[k].lo[a]);
                b.hi[a] = fmaxf(b.hi[a], lds[k].hi[a]);
            }
            b.cnt += lds[k].cnt;
        }
    }
}

__device__ __forceinline__ BoxAcc empty_box()
{
    BoxAcc b;
    for (int a = 0; a < 3; ++a) {
        b.lo[a] = INFINITY;
        b.hi[a] = -INFINITY;
    }
    b.cnt = 0u;
    return b;
}

__global__ __launch_bounds__(kVoxThreads) void voxel_bbox_kernel(const float *xyz, int64_t n,
                                                                 uint32_t *part)
{
    __shared__ BoxAcc lds[kVoxWaves];
    BoxAcc b = empty_box();
    for (int64_t i = int64_t(blockIdx.x) * kVoxThreads + threadIdx.x; i < n;
         i += int64_t(gridDim.x) * kVoxThreads) {
        const float x = xyz[3 * i], y = xyz[3 * i + 1], z = xyz[3 * i + 2];
        if (!finite3(x, y, z)) continue;
        b.lo[0] = fminf(b.lo[0], x); b.lo[1] = fminf(b.lo[1], y); b.lo[2] = fminf(b.lo[2], z);
        b.hi[0] = fmaxf(b.hi[0], x); b.hi[1] = fmaxf(b.hi[1], y); b.hi[2] = fmaxf(b.hi[2], z);
        b.cnt += 1u;
    }
    block_box(b, lds);
    if (threadIdx.x == 0) {
        for (int a = 0; a < 3; ++a) {
            part[a * kVoxBlocks + blockIdx.x] = __float_as_uint(b.lo[a]);
            part[(3 + a) * kVoxBlocks + blockIdx.x] = __float_as_uint(b.hi[a]);
        }
        part[6 * kVoxBlocks + blockIdx.x] = b.cnt;
    }
}

// The grid spanned by the occupied voxels: floor and the division by a
// positive leaf are monotone, so its corners are the voxels of min / max.
__device__ VoxGrid make_grid(const BoxAcc &b, double leaf)
{
    VoxGrid g{};
    g.n_finite = b.cnt;
    if (b.cnt == 0u) return g;  // sentinel 0, no passes: every key is the sentinel
    double cells = 1.0;
    for (int a = 0; a < 3; ++a) {
        const double lo = floor(double(b.lo[a]) / leaf), hi = floor(double(b.hi[a]) / leaf);
        if (!(fabs(lo) < 4.0e18 && fabs(hi) < 4.0e18)) {
            g.err = kVoxErrRange;
            return g;
        }
        const double d = hi - lo + 1.0;
        cells *= d;
        if (!(cells < 4294967295.0)) {
            g.err = kVoxErrCells;
            return g;
        }
        g.vmin[a] = int64_t(lo);
        g.dims[a] = uint32_t(d);
    }
    g.sentinel = uint32_t(cells);
    const int bits = 32 - __clz(int(g.sentinel));  // sentinel >= 1
    g.passes = (bits + kVoxDigitBits - 1) / kVoxDigitBits;
    return g;
}

struct VoxKeyArgs {
    const float *xyz;
    int64_t n;
    double leaf;
    const uint32_t *part;
    int32_t nb;  // bbox blocks
    VoxGrid *grid;
    uint32_t *keys;
};

__device__ __forceinline__ int64_t vox_coord(float p, double leaf)
{
    return int64_t(floor(double(p) / leaf));
}

__global__ __launch_bounds__(kVoxThreads) void voxel_key_kernel(VoxKeyArgs a)
{
    __shared__ BoxAcc lds[kVoxWaves];
    __shared__ VoxGrid g;
    BoxAcc b = empty_box();
    for (int k = threadIdx.x; k < a.nb; k += kVoxThreads) {
        for (int ax = 0; ax < 3; ++ax) {
            b.lo[ax] = fminf(b.lo[ax], __uint_as_float(a.part[ax * kVoxBlocks + k]));
            b.hi[ax] = fmaxf(b.hi[ax], __uint_as_float(a.part[(3 + ax) * kVoxBlocks + k]));
        }
        b.cnt += a.part[6 * kVoxBlocks + k];
    }
    block_box(b, lds);
    if (threadIdx.x == 0) {
        g = make_grid(b, a.leaf);
        if (blockIdx.x == 0) *a.grid = g;
    }
    __syncthreads();
    const bool ok = g.err == kVoxOk;
    for (int64_t i = int64_t(blockIdx.x) * kVoxThreads + threadIdx.x; i < a.n;
         i += int64_t(gridDim.x) * kVoxThreads) {
        const float x = a.xyz[3 * i], y = a.xyz[3 * i + 1], z = a.xyz[3 * i + 2];
        uint32_t key = g.sentinel;
        if (ok && finite3(x, y, z)) {
            // in range: every finite point lies in [min, max], whose voxels
            // bound the grid
            const uint32_t vx = uint32_t(vox_coord(x, a.leaf) - g.vmin[0]);
            const uint32_t vy = uint32_t(vox_coord(y, a.leaf) - g.vmin[1]);
            const uint32_t vz = uint32_t(vox_coord(z, a.leaf) - g.vmin[2]);
            key = vx + g.dims[0] * (vy + g.dims[1] * vz);
        }
        a.keys[i] = key;
    }
}

// One radix pass over (key, value) pairs: digit `pass`, the key bits from
// kVoxDigitBits * pass up.
// Pass 0 takes the point index as the value; the last pass the grid needs
// writes the point's coordinates instead of the value.
struct VoxPass {
    const uint32_t *keys_in;
    const int32_t *vals_in;  // unused in pass 0
    uint32_t *keys_out;
    int32_t *vals_out;  // unused in the last pass
    const float *xyz;
    float4 *sorted;
    uint32_t *hist;
    uint32_t *totals;
    const VoxGrid *grid;
    int64_t n;
    int32_t ntiles;
    int32_t pass;
};

__global__ __launch_bounds__(kVoxThreads) void voxel_hist_kernel(VoxPass p)
{
    __shared__ uint32_t h[kVoxBins];
    if (p.pass >= p.grid->passes) return;  // uniform: a digit the keys do not have
#pragma unroll
    for (int j = 0; j < kVoxBinsPerThread; ++j) h[threadIdx.x + j * kVoxThreads] = 0u;
    __syncthreads();
    const int shift = kVoxDigitBits * p.pass;
    const int64_t base = int64_t(blockIdx.x) * kVoxTile;
#pragma unroll
    for (int r = 0; r < kVoxItems; ++r) {
        const int64_t e = base + r * kVoxThreads + threadIdx.x;
        if (e < p.n) atomicAdd(&h[(p.keys_in[e] >> shift) & (kVoxBins - 1)], 1u);
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kVoxBinsPerThread; ++j) {
        const int d = threadIdx.x + j * kVoxThreads;
        p.hist[int64_t(d) * p.ntiles + blockIdx.x] = h[d];
    }
}

// Exclusive scan over the block of one value per thread; total = the sum.
__device__ __forceinline__ uint32_t vox_block_scan(uint32_t v, uint32_t *wsum /* LDS [waves] */,
                                                   uint32_t &total)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = uint32_t(__shfl_up(int(x), off, 64));
        if (lane >= off) x += y;
    }
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    uint32_t before = 0;
    total = 0;
#pragma unroll
    for (int ww = 0; ww < kVoxWaves; ++ww) {
        before += ww < w ? wsum[ww] : 0u;
        total += wsum[ww];
    }
    __syncthreads();
    return before + x - v;
}

// Work-group d scans row d of rows (len words) in place and writes its sum to
// total[d]; skipped, like the pass's histogram, when the keys lack the digit.
__global__ __launch_bounds__(kVoxThreads) void voxel_scan_kernel(uint32_t *rows, int32_t len,
                                                                 uint32_t *total,
                                                                 const VoxGrid *grid,
                                                                 int32_t pass)
{
    __shared__ uint32_t wsum[kVoxWaves];
    if (pass >= grid->passes) return;
    uint32_t *row = rows + int64_t(blockIdx.x) * len;
    uint32_t carry = 0;
    for (int32_t k0 = 0; k0 < len; k0 += kVoxThreads) {
        const int32_t k = k0 + threadIdx.x;
        const uint32_t v = k < len ? row[k] : 0u;
        uint32_t t;
        const uint32_t ex = vox_block_scan(v, wsum, t);
        if (k < len) row[k] = carry + ex;
        carry += t;
    }
    if (threadIdx.x == 0) total[blockIdx.x] = carry;
}

// Stable scatter of one tile.  Element e = tile * 2048 + r * 256 + tid is the
// r-th round of thread tid, so (r, tid) is the input order inside the tile.
// Within a wave the lanes holding the same digit are found with one ballot
// per digit bit; the lowest of them (the leader) publishes the group's size in
// wcnt, tagged with the round so that no clearing is needed between rounds.
// Rank of an element = the digit's running base (earlier tiles, earlier
// rounds) + the group sizes of earlier waves this round + the lanes below it
// in its group.
__global__ __launch_bounds__(kVoxThreads) void voxel_scatter_kernel(VoxPass p)
{
    __shared__ uint32_t base[kVoxBins];
    __shared__ uint32_t wcnt[kVoxWaves][kVoxBins];
    __shared__ uint32_t wsum[kVoxWaves];
    const int passes = p.grid->passes;
    if (p.pass >= passes) return;  // uniform
    const bool last = p.pass == passes - 1;
    const int shift = kVoxDigitBits * p.pass;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const uint64_t below = (uint64_t(1) << lane) - 1u;
    // digit bases: kVoxBinsPerThread consecutive digits per thread
    uint32_t tot[kVoxBinsPerThread], s = 0;
#pragma unroll
    for (int j = 0; j < kVoxBinsPerThread; ++j) {
        tot[j] = p.totals[tid * kVoxBinsPerThread + j];
        s += tot[j];
    }
    uint32_t all;
    uint32_t run = vox_block_scan(s, wsum, all);
#pragma unroll
    for (int j = 0; j < kVoxBinsPerThread; ++j) {
        const int d = tid * kVoxBinsPerThread + j;
        base[d] = run + p.hist[int64_t(d) * p.ntiles + blockIdx.x];
        run += tot[j];
    }
#pragma unroll
    for (int ww = 0; ww < kVoxWaves; ++ww)
#pragma unroll
        for (int j = 0; j < kVoxBinsPerThread; ++j) wcnt[ww][tid + j * kVoxThreads] = 0u;
    const int64_t tbase = int64_t(blockIdx.x) * kVoxTile;
    uint32_t keys_r[kVoxItems];
    int32_t vals_r[kVoxItems];
#pragma unroll
    for (int r = 0; r < kVoxItems; ++r) {
        const int64_t e = tbase + r * kVoxThreads + tid;
        keys_r[r] = 0u;
        vals_r[r] = 0;
        if (e < p.n) {
            keys_r[r] = p.keys_in[e];
            vals_r[r] = p.pass == 0 ? int32_t(e) : p.vals_in[e];
        }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kVoxItems; ++r) {
        const bool valid = tbase + r * kVoxThreads + tid < p.n;
        const uint32_t key = keys_r[r];
        const int32_t val = vals_r[r];
        const uint32_t dig = (key >> shift) & uint32_t(kVoxBins - 1);
        uint64_t peers = __ballot(valid);
#pragma unroll
        for (int bit = 0; bit < kVoxDigitBits; ++bit) {
            const bool set = (dig >> bit) & 1u;
            const uint64_t bal = __ballot(set);
            peers &= set ? bal : ~bal;
        }
        const uint32_t rank = uint32_t(__popcll(peers & below));
        const uint32_t size = uint32_t(__popcll(peers));
        const uint32_t tag = uint32_t(r + 1) << 16;  // sizes are <= 64
        if (valid && rank == 0) wcnt[w][dig] = tag | size;
        __syncthreads();
        if (valid) {
            uint32_t off = base[dig] + rank;
            for (int ww = 0; ww < w; ++ww) {
                const uint32_t c = wcnt[ww][dig];
                off += (c & 0xffff0000u) == tag ? (c & 0xffffu) : 0u;
            }
            p.keys_out[off] = key;
            if (last) {
                const float *q = p.xyz + 3 * int64_t(val);
                p.sorted[off] = make_float4(q[0], q[1], q[2], 0.0f);
            } else {
                p.vals_out[off] = val;
            }
        }
        __syncthreads();  // every lane has read base before it moves on
        if (valid && rank == 0) atomicAdd(&base[dig], size);
    }
}

// The sorted keys: pass k reads buffer a when k is even and writes b, so an
// odd number of passes leaves them in b.
__device__ __forceinline__ const uint32_t *sorted_keys(int32_t passes, const uint32_t *ka,
                                                       const uint32_t *kb)
{
    return (passes & 1) ? kb : ka;
}

__device__ __forceinline__ bool is_head(const uint32_t *keys, int64_t e, int64_t n,
                                        uint32_t sentinel)
{
    if (e >= n) return false;
    const uint32_t k = keys[e];
    return k != sentinel && (e == 0 || keys[e - 1] != k);
}

// Tile t's number of voxel heads.
__global__ __launch_bounds__(kVoxThreads) void voxel_heads_kernel(const uint32_t *ka,
                                                                  const uint32_t *kb, int64_t n,
                                                                  const VoxGrid *grid,
                                                                  uint32_t *tile_heads)
{
    __shared__ uint32_t wsum[kVoxWaves];
    const VoxGrid g = *grid;
    const uint32_t *keys = sorted_keys(g.passes, ka, kb);
    const int64_t base = int64_t(blockIdx.x) * kVoxTile;
    uint32_t c = 0;
#pragma unroll
    for (int r = 0; r < kVoxItems; ++r)
        c += is_head(keys, base + r * kVoxThreads + threadIdx.x, n, g.sentinel) ? 1u : 0u;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) c += uint32_t(__shfl_xor(int(c), off, 64));
    if (lane == 0) wsum[w] = c;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t s = 0;
        for (int k = 0; k < kVoxWaves; ++k) s += wsum[k];
        tile_heads[blockIdx.x] = s;
    }
}

// starts[voxel] = sorted position of its first point.  Tile t's first voxel
// is the sum of the head counts of tiles 0 .. t-1, which each work-group adds
// up itself; the last one also writes the voxel count.
__global__ __launch_bounds__(kVoxThreads) void voxel_starts_kernel(const uint32_t *ka,
                                                                   const uint32_t *kb, int64_t n,
                                                                   VoxGrid *grid,
                                                                   const uint32_t *tile_heads,
                                                                   int32_t *starts)
{
    __shared__ uint32_t wsum[kVoxWaves];
    const int32_t passes = grid->passes;  // not nvox: the last work-group writes it
    const uint32_t sentinel = grid->sentinel;
    const uint32_t *keys = sorted_keys(passes, ka, kb);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const uint64_t below = (uint64_t(1) << lane) - 1u;
    const int64_t base = int64_t(blockIdx.x) * kVoxTile;
    uint32_t before_tile = 0;
    for (uint32_t t = threadIdx.x; t < blockIdx.x; t += kVoxThreads) before_tile += tile_heads[t];
    uint32_t run;
    (void)vox_block_scan(before_tile, wsum, run);  // run = the block's sum
#pragma unroll
    for (int r = 0; r < kVoxItems; ++r) {
        const int64_t e = base + r * kVoxThreads + threadIdx.x;
        const bool h = is_head(keys, e, n, sentinel);
        const uint64_t bal = __ballot(h);
        if (lane == 0) wsum[w] = uint32_t(__popcll(bal));
        __syncthreads();
        uint32_t before = 0, total = 0;
        for (int k = 0; k < kVoxWaves; ++k) {
            before += k < w ? wsum[k] : 0u;
            total += wsum[k];
        }
        if (h) starts[run + before + uint32_t(__popcll(bal & below))] = int32_t(e);
        run += total;
        __syncthreads();
    }
    if (blockIdx.x == gridDim.x - 1 && threadIdx.x == 0) grid->nvox = run;
}

// Means of the voxels.  The sums run over each voxel's segment of the sorted
// points in order (= ascending point index), so each voxel's additions form
// one chain; what can run in parallel is the loading.
//   * Voxels of at most kVoxSmall points: one lane each, reading its segment
//     kChunk points at a time (one 16-byte load per point, all in flight).
//   * Larger voxels (near a LiDAR sensor: ~200 points at 0.2 m, ~6,000 at
//     1 m): one wave each (voxel_big_kernel).  Lanes walking such segments
//     would keep one chain per lane, but every load instruction of the wave
//     would touch 64 cache lines; a wave that stages one segment in coalesced
//     windows and runs its x, y and z chains in three lanes is ~10x faster on
//     them.  They go to a list as (voxel, segment start, segment end), in any
//     order (each result depends on its voxel alone); at over 64 points each,
//     the 16-byte entries fit in n int32 of workspace.
constexpr int kVoxSmall = 64;
constexpr int kVoxWin = 256;  // points per staged window

__global__ __launch_bounds__(kVoxThreads) void voxel_centroid_kernel(const float4 *sorted,
                                                                     const int32_t *starts,
                                                                     VoxGrid *grid, float *out,
                                                                     int32_t *counts,
                                                                     int4 *big)
{
    constexpr int kChunk = 32;
    const int lane = threadIdx.x & 63;
    const int64_t m = int64_t(grid->nvox);
    const int64_t n_finite = int64_t(grid->n_finite);
    for (int64_t v = int64_t(blockIdx.x) * kVoxThreads + threadIdx.x; v - lane < m;
         v += int64_t(gridDim.x) * kVoxThreads) {
        const bool own = v < m;
        const int64_t s = own ? int64_t(starts[v]) : 0;
        const int64_t e = own ? (v + 1 < m ? int64_t(starts[v + 1]) : n_finite) : 0;
        const bool large = e - s > kVoxSmall;
        const uint64_t bal = __ballot(large);
        if (bal) {  // wave-uniform: one atomic per wave
            uint32_t at = 0;
            if (lane == 0) at = atomicAdd(&grid->nbig, uint32_t(__popcll(bal)));
            at = uint32_t(__shfl(int(at), 0, 64));
            if (large)
                big[at + uint32_t(__popcll(bal & ((uint64_t(1) << lane) - 1u)))] =
                    make_int4(int32_t(v), int32_t(s), int32_t(e), 0);
        }
        if (!own || large) continue;
        double sx = 0.0, sy = 0.0, sz = 0.0;
        for (int64_t k0 = s; k0 < e; k0 += kChunk) {
            float4 q[kChunk];
#pragma unroll
            for (int j = 0; j < kChunk; ++j)
                q[j] = sorted[k0 + j < e ? k0 + j : e - 1];  // in bounds; unused past e
#pragma unroll
            for (int j = 0; j < kChunk; ++j) {
                if (k0 + j < e) {
                    sx += double(q[j].x);
                    sy += double(q[j].y);
                    sz += double(q[j].z);
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

// One wave (one work-group) per listed voxel.  Its segment is staged kVoxWin
// points at a time as x, y and z rows of doubles in LDS (the conversions done
// by all lanes); lane c < 3 then adds row c in order, while the loads of the
// next window are in flight.
__global__ __launch_bounds__(64) void voxel_big_kernel(const float4 *sorted,
                                                       const VoxGrid *grid, const int4 *big,
                                                       float *out, int32_t *counts)
{
    constexpr int kPer = kVoxWin / 64;  // points per lane and window
    __shared__ double row[3][kVoxWin];
    const int lane = threadIdx.x;
    const uint32_t nbig = grid->nbig;
    const double *mine = row[lane < 3 ? lane : 0];
    for (uint32_t i = blockIdx.x; i < nbig; i += gridDim.x) {
        const int4 job = big[i];
        const int64_t v = job.x, s = job.y, e = job.z;
        float4 q[kPer];
#pragma unroll
        for (int r = 0; r < kPer; ++r) {
            const int64_t k = s + r * 64 + lane;
            if (k < e) q[r] = sorted[k];
        }
        double acc = 0.0;
        for (int64_t w0 = s; w0 < e; w0 += kVoxWin) {
            const int len = int(e - w0 < kVoxWin ? e - w0 : kVoxWin);
#pragma unroll
            for (int r = 0; r < kPer; ++r) {
                const int k = r * 64 + lane;
                if (k < len) {
                    row[0][k] = double(q[r].x);
                    row[1][k] = double(q[r].y);
                    row[2][k] = double(q[r].z);
                }
            }
            __syncthreads();
#pragma unroll
            for (int r = 0; r < kPer; ++r) {  // the next window
                const int64_t k = w0 + kVoxWin + r * 64 + lane;
                if (k < e) q[r] = sorted[k];
            }
            if (lane < 3) {
                if (len == kVoxWin) {
#pragma unroll 32
                    for (int k = 0; k < kVoxWin; ++k) acc += mine[k];
                } else {
                    for (int k = 0; k < len; ++k) acc += mine[k];
                }
            }
            __syncthreads();  // the window is read before the next one is staged
        }
        if (lane < 3) out[3 * v + lane] = float(acc / double(e - s));
        if (lane == 0 && counts) counts[v] = int32_t(e - s);
    }
}

uint32_t grid_of(int64_t n, int64_t per, uint32_t cap)
{
    int64_t b = (n + per - 1) / per;
    if (b < 1) b = 1;
    if (b > int64_t(cap)) b = cap;
    return uint32_t(b);
}

}  // namespace

size_t voxel_ws_bytes(int64_t n)
{
    if (n <= 0) return 0;
    const size_t nn = size_t(n);
    const size_t nt = size_t(vox_tiles(n));
    return 4 * align256(nn * 4) + align256(size_t(kVoxBins) * nt * 4) +
           align256(size_t(kVoxBins) * 4) + align256(nt * 4) + align256(nn * 4) +
           align256(size_t(7) * kVoxBlocks * 4) + align256(sizeof(VoxGrid)) + align256(nn * 16);
}

VoxelWorkspace carve_voxel_workspace(void *ws, int64_t n)
{
    VoxelWorkspace w{};
    char *p = static_cast<char *>(ws);
    const size_t a = align256(size_t(n) * 4);
    const size_t nt = size_t(vox_tiles(n));
    w.keys_a = reinterpret_cast<uint32_t *>(p);
    w.keys_b = reinterpret_cast<uint32_t *>(p + a);
    w.vals_a = reinterpret_cast<int32_t *>(p + 2 * a);
    w.vals_b = reinterpret_cast<int32_t *>(p + 3 * a);
    p += 4 * a;
    w.hist = reinterpret_cast<uint32_t *>(p);
    p += align256(size_t(kVoxBins) * nt * 4);
    w.totals = reinterpret_cast<uint32_t *>(p);
    p += align256(size_t(kVoxBins) * 4);
    w.tile_heads = reinterpret_cast<uint32_t *>(p);
    p += align256(nt * 4);
    w.starts = reinterpret_cast<int32_t *>(p);
    p += a;
    w.bbox_part = reinterpret_cast<uint32_t *>(p);
    p += align256(size_t(7) * kVoxBlocks * 4);
    w.grid = reinterpret_cast<VoxGrid *>(p);
    p += align256(sizeof(VoxGrid));
    w.sorted = reinterpret_cast<float4 *>(p);
    return w;
}

hipError_t launch_voxel_filter(const float *xyz, int64_t n, double leaf, const VoxelWorkspace &w,
                               float *out, int32_t *counts, hipStream_t s)
{
    const uint32_t nb = grid_of(n, int64_t(kVoxThreads) * 4, kVoxBlocks);
    voxel_bbox_kernel<<<nb, kVoxThreads, 0, s>>>(xyz, n, w.bbox_part);
    VoxKeyArgs ka{};
    ka.xyz = xyz;
    ka.n = n;
    ka.leaf = leaf;
    ka.part = w.bbox_part;
    ka.nb = int32_t(nb);
    ka.grid = w.grid;
    ka.keys = w.keys_a;
    voxel_key_kernel<<<grid_of(n, int64_t(kVoxThreads) * 4, 1024), kVoxThreads, 0, s>>>(ka);
    const int32_t nt = vox_tiles(n);
    VoxPass p{};
    p.xyz = xyz;
    p.sorted = w.sorted;
    p.hist = w.hist;
    p.totals = w.totals;
    p.grid = w.grid;
    p.n = n;
    p.ntiles = nt;
    uint32_t *kin = w.keys_a, *kout = w.keys_b;
    int32_t *vin = w.vals_a, *vout = w.vals_b;
    for (int pass = 0; pass < kVoxMaxPasses; ++pass) {
        p.keys_in = kin;
        p.vals_in = vin;
        p.keys_out = kout;
        p.vals_out = vout;
        p.pass = pass;
        voxel_hist_kernel<<<nt, kVoxThreads, 0, s>>>(p);
        voxel_scan_kernel<<<kVoxBins, kVoxThreads, 0, s>>>(w.hist, nt, w.totals, w.grid, pass);
        voxel_scatter_kernel<<<nt, kVoxThreads, 0, s>>>(p);
        uint32_t *tk = kin; kin = kout; kout = tk;
        int32_t *tv = vin; vin = vout; vout = tv;
    }
    voxel_heads_kernel<<<nt, kVoxThreads, 0, s>>>(w.keys_a, w.keys_b, n, w.grid, w.tile_heads);
    voxel_starts_kernel<<<nt, kVoxThreads, 0, s>>>(w.keys_a, w.keys_b, n, w.grid, w.tile_heads,
                                                    w.starts);
    int4 *const big = reinterpret_cast<int4 *>(w.vals_a);  // free once the sort is done
    voxel_centroid_kernel<<<grid_of(n, kVoxThreads, 4096), kVoxThreads, 0, s>>>(
        w.sorted, w.starts, w.grid, out, counts, big);
    voxel_big_kernel<<<2048, 64, 0, s>>>(w.sorted, w.grid, big, out, counts);
    return hipGetLastError();
}

}  // namespace kdnn
