// Roofline micro-benchmarks for gfx950: the random-gather rate and the
// dependent-load latency of the memory level a working set of a given size
// lives in (L2, Infinity Cache, HBM).  They measure the ceilings the search
// kernels are compared against; nothing on the search path calls them.
//
//   gather_kernel<W4>: every lane reads `rounds` records of W4 consecutive
//     16-byte words at pseudo-random record indices, four records in flight
//     at a time (independent loads: a throughput ceiling).  W4 = 3 is the
//     shape of a child-pair box load, W4 = 16 that of a leaf chunk, W4 = 1 a
//     single point.
//   chase_kernel: every lane follows its own chain through a random cyclic
//     permutation of 64-byte records (each hop depends on the last: a latency
//     figure).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kdnn_internal.hpp"

namespace kdnn {

// Integer hash "lowbias32" (C. Wellons, "Prospecting for hash functions",
// 2018): a bijection on 32-bit words, used as a counter-based index stream.
__device__ __forceinline__ uint32_t lowbias32(uint32_t x)
{
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

constexpr int kGatherWG = 256;
constexpr int kInflight = 4;

template <int W4>
__global__ __launch_bounds__(kGatherWG) void gather_kernel(const uint4 *__restrict__ buf,
                                                           uint32_t nrec, uint32_t rounds,
                                                           uint32_t seed, uint32_t *sink)
{
    const uint32_t lane = blockIdx.x * kGatherWG + threadIdx.x;
    uint32_t acc = 0;
    for (uint32_t r = 0; r < rounds; r += kInflight) {
        uint4 v[kInflight][W4];
#pragma unroll
        for (int u = 0; u < kInflight; ++u) {
            const uint32_t h = lowbias32(lane * 0x9e3779b9u + (r + u) * 0x85ebca6bu + seed);
            const uint32_t idx = uint32_t((uint64_t(h) * nrec) >> 32);  // uniform in [0, nrec)
#pragma unroll
            for (int k = 0; k < W4; ++k) v[u][k] = buf[size_t(idx) * W4 + k];
        }
#pragma unroll
        for (int u = 0; u < kInflight; ++u)
#pragma unroll
            for (int k = 0; k < W4; ++k) acc ^= v[u][k].x ^ v[u][k].y ^ v[u][k].z ^ v[u][k].w;
    }
    if (acc == 0x5eed5eedu) sink[0] = acc;  // keeps the loads; practically never taken
}

__global__ __launch_bounds__(64) void chase_kernel(const uint32_t *__restrict__ next,
                                                   uint32_t nrec, uint32_t steps, uint32_t *sink)
{
    const uint32_t lane = blockIdx.x * 64 + threadIdx.x;
    uint32_t i = uint32_t((uint64_t(lowbias32(lane + 1u)) * nrec) >> 32);
    for (uint32_t s = 0; s < steps; ++s) {
        const uint32_t j = next[size_t(i) * 16];  // 64-byte records
        i = j < nrec ? j : nrec - 1;              // in bounds whatever the buffer holds
    }
    if (i == 0xFFFFFFFFu) sink[0] = i;
}

static bool timed(hipStream_t s, float *ms_out, void (*launch)(void *, hipStream_t), void *ctx)
{
    hipEvent_t a = nullptr, b = nullptr;
    bool ok = hipEventCreate(&a) == hipSuccess && hipEventCreate(&b) == hipSuccess &&
              hipEventRecord(a, s) == hipSuccess;
    if (ok) {
        launch(ctx, s);
        ok = hipGetLastError() == hipSuccess && hipEventRecord(b, s) == hipSuccess &&
             hipEventSynchronize(b) == hipSuccess && hipEventElapsedTime(ms_out, a, b) == hipSuccess;
    }
    if (a) (void)hipEventDestroy(a);
    if (b) (void)hipEventDestroy(b);
    return ok;
}

struct GatherCtx {
    const uint4 *buf;
    uint32_t nrec, rounds, seed, blocks;
    int words;
    uint32_t *sink;
};

static void launch_gather(void *p, hipStream_t s)
{
    const GatherCtx &c = *static_cast<const GatherCtx *>(p);
    const dim3 g(c.blocks);
    switch (c.words) {
    case 1: gather_kernel<1><<<g, kGatherWG, 0, s>>>(c.buf, c.nrec, c.rounds, c.seed, c.sink); break;
    case 3: gather_kernel<3><<<g, kGatherWG, 0, s>>>(c.buf, c.nrec, c.rounds, c.seed, c.sink); break;
    default: gather_kernel<16><<<g, kGatherWG, 0, s>>>(c.buf, c.nrec, c.rounds, c.seed, c.sink); break;
    }
}

struct ChaseCtx {
    const uint32_t *next;
    uint32_t nrec, steps, waves;
    uint32_t *sink;
};

static void launch_chase(void *p, hipStream_t s)
{
    const ChaseCtx &c = *static_cast<const ChaseCtx *>(p);
    chase_kernel<<<dim3(c.waves), 64, 0, s>>>(c.next, c.nrec, c.steps, c.sink);
}

bool run_gather_bench(const void *buf, int64_t n_records, int32_t words, int64_t lanes,
                      int32_t rounds, uint32_t seed, uint32_t *sink, float *ms, hipStream_t s)
{
    GatherCtx c{static_cast<const uint4 *>(buf), uint32_t(n_records), uint32_t(rounds), seed,
                uint32_t(lanes / kGatherWG), words, sink};
    return timed(s, ms, launch_gather, &c);
}

bool run_chase_bench(const uint32_t *next, int64_t n_records, int32_t waves, int32_t steps,
                     uint32_t *sink, float *ms, hipStream_t s)
{
    ChaseCtx c{next, uint32_t(n_records), uint32_t(steps), uint32_t(waves), sink};
    return timed(s, ms, launch_chase, &c);
}

}  // namespace kdnn
