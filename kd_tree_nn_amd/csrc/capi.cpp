// extern "C" entry points of libkdnn.so (declared and documented in kdnn.h).
// Argument checking, error reporting, tree lifetime, and the host ICP loop
// (CUDA-KDTree ICP article, §2.1 and §3.3: correspond, reduce, solve on the
// host, repeat; §4.6 convergence rule).  No exception crosses the ABI.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstddef>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "kdnn_internal.hpp"

using namespace kdnn;

namespace {

thread_local std::string g_err;

// nn_query's automatic Morton ordering: tree footprint above this many L2s.
// The ordering costs a radix sort per call (30-55 us at 0.1-1M queries); with
// each wave's queries spread over its XCD's segment, the search gains about
// that much only once the tree is several times the L2.
constexpr size_t kQuerySortL2Multiple = 4;

// Kernel timing (kdnn_timing_begin / kdnn_timing_end): event pairs for the
// next `cap` correspondence launches of this thread.
struct Timing {
    std::vector<hipEvent_t> ev;  // 2 per launch
    int32_t used = 0;
    bool on = false;
    void release()
    {
        for (hipEvent_t e : ev) (void)hipEventDestroy(e);
        ev.clear();
        used = 0;
        on = false;
    }
    ~Timing() { release(); }
    // next free pair, or null (off, or all used)
    const hipEvent_t *next()
    {
        if (!on || 2 * size_t(used) >= ev.size()) return nullptr;
        return &ev[2 * size_t(used++)];
    }
};
thread_local Timing g_timing;

kdnn_status fail(kdnn_status st, const std::string &msg)
{
    g_err = msg;
    return st;
}

kdnn_status hip_fail(hipError_t e, const char *what)
{
    return fail(KDNN_EDEVICE, std::string(what) + ": " + hipGetErrorString(e));
}

#define KDNN_GUARD_BEGIN try {
#define KDNN_GUARD_END                                                     \
    }                                                                      \
    catch (const std::bad_alloc &) { return fail(KDNN_ENOMEM, "out of host memory"); } \
    catch (...) { return fail(KDNN_EINVAL, "internal error"); }

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// A valid lane count, and at most one of the lanes / budget / LDS choices.
bool lanes_ok(uint32_t flags)
{
    const uint32_t g = (flags & KDNN_LANES_MASK) >> KDNN_LANES_SHIFT;
    const int chosen = int(g != 0) + int((flags & KDNN_BUDGET_MASK) != 0) +
                       int((flags & KDNN_TOP_LDS) != 0);
    return (g == 0 || g == 1 || g == 2 || g == 4 || g == 8 || g == 16) && chosen <= 1;
}

constexpr uint32_t kSchedMask = KDNN_LANES_MASK | KDNN_BUDGET_MASK | KDNN_TOP_LDS;

Schedule schedule_of(uint32_t flags)
{
    Schedule sc;
    sc.lanes = int((flags & KDNN_LANES_MASK) >> KDNN_LANES_SHIFT);
    sc.budget = (flags & KDNN_BUDGET_MASK) >> KDNN_BUDGET_SHIFT;
    sc.top_lds = (flags & KDNN_TOP_LDS) != 0;
    return sc;
}

double ms_since(std::chrono::steady_clock::time_point t0)
{
    return std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
}

void free_tree(kdnn_tree *t)
{
    if (!t) return;
    int cur = -1;
    if (hipGetDevice(&cur) == hipSuccess && cur != t->device) (void)hipSetDevice(t->device);
    if (t->d_nodes) (void)hipFree(t->d_nodes);
    if (t->d_boxes) (void)hipFree(t->d_boxes);
    if (t->d_points) (void)hipFree(t->d_points);
    if (t->d_slot_of) (void)hipFree(t->d_slot_of);
    if (t->d_paths) (void)hipFree(t->d_paths);
    if (t->h_pinned) (void)hipHostFree(t->h_pinned);
    if (t->h_loop) (void)hipHostFree(t->h_loop);
    if (t->d_loop) (void)hipFree(t->d_loop);
    if (cur >= 0 && cur != t->device) (void)hipSetDevice(cur);
    delete t;
}

kdnn_status check_points(const void *p, int64_t n, const char *name)
{
    if (n < 0 || n >= (int64_t(1) << 31)) return fail(KDNN_EINVAL, std::string(name) + ": count out of range");
    if (n > 0 && !p) return fail(KDNN_EINVAL, std::string(name) + ": null pointer");
    if (p && !aligned(p, 4)) return fail(KDNN_EINVAL, std::string(name) + ": not 4-byte aligned");
    return KDNN_OK;
}

kdnn_status check_ws(const void *ws, size_t have, size_t need)
{
    if (need == 0) return KDNN_OK;
    if (!ws) return fail(KDNN_EINVAL, "workspace: null pointer");
    if (!aligned(ws, 256)) return fail(KDNN_EINVAL, "workspace: not 256-byte aligned");
    if (have < need)
        return fail(KDNN_EINVAL, "workspace: " + std::to_string(have) + " bytes given, " +
                                     std::to_string(need) + " needed");
    return KDNN_OK;
}

void to_sums(const double *d, const double c[3], kdnn_icp_sums *o)
{
    o->n = int64_t(std::llround(d[16]));
    for (int k = 0; k < 3; ++k) {
        o->c[k] = c[k];
        o->sum_s[k] = d[k];
        o->sum_m[k] = d[3 + k];
    }
    for (int k = 0; k < 9; ++k) o->sum_sm[k] = d[6 + k];
    o->sum_d2 = d[15];
}

void rt_to_f32(const double *R, const double *t, float out[12])
{
    for (int k = 0; k < 9; ++k) out[k] = float(R[k]);
    for (int k = 0; k < 3; ++k) out[9 + k] = float(t[k]);
}

const double kI[9] = {1, 0, 0, 0, 1, 0, 0, 0, 1};
const double kZ[3] = {0, 0, 0};

// Resolve the ordering choice of ICP flags to KDNN_ICP_NO_SORT set or clear
// (KDNN_ICP_SORT cleared).
uint32_t icp_resolve_sort(const kdnn_tree *tree, uint32_t flags)
{
    const bool sort = (flags & KDNN_ICP_SORT) ||
                      (!(flags & KDNN_ICP_NO_SORT) && tree->auto_sort_icp);
    flags &= ~(KDNN_ICP_SORT | KDNN_ICP_NO_SORT);
    return sort ? flags : (flags | KDNN_ICP_NO_SORT);
}

// The fp32 squared-distance bound of a distance threshold: fl32(max_dist^2)
// (product in fp64, one rounding); no bound unless max_dist is finite and > 0.
float bound_of(double max_dist)
{
    return (max_dist > 0.0 && std::isfinite(max_dist)) ? float(max_dist * max_dist) : INFINITY;
}

kdnn_status check_reject(const kdnn_icp_reject *r, const char *where)
{
    if (r && !(r->reject_k >= 0.0 && std::isfinite(r->reject_k)))
        return fail(KDNN_EINVAL, std::string(where) + ": reject_k must be finite and >= 0");
    return KDNN_OK;
}

// The word of the tree's pinned slot that the reduction sets to the sequence
// number of the launch once its sums are there (the sums take words 0 .. 18).
constexpr int kDoneWord = 31;

// Wait until a reduction launched with sequence number seq has published its
// sums, i.e. set the pinned word w to seq: poll that word, and ask the stream
// every kStreamQueryInterval, so that a failed or finished stream ends the
// wait either way.  The stream is asked rarely: a hipStreamQuery every 20 us
// slowed the host-driven ICP loop from 33 to 44 us per Scene iteration.
constexpr std::chrono::microseconds kStreamQueryInterval(1000);
hipError_t wait_word(const volatile uint64_t *w, uint64_t seq, hipStream_t s)
{
    auto last = std::chrono::steady_clock::now();
    for (;;) {
        if (*w == seq) {
            std::atomic_thread_fence(std::memory_order_acquire);
            return hipSuccess;
        }
        const auto now = std::chrono::steady_clock::now();
        if (now - last < kStreamQueryInterval) continue;
        last = now;
        const hipError_t e = hipStreamQuery(s);
        if (e == hipErrorNotReady) continue;
        if (e != hipSuccess) return e;
        if (*w == seq) {  // the stream is idle: the word must be there now
            std::atomic_thread_fence(std::memory_order_acquire);
            return hipSuccess;
        }
        return hipErrorLaunchFailure;
    }
}

// The same for the tree's own pinned slot.
hipError_t wait_sums(const kdnn_tree *t, uint64_t seq, hipStream_t s)
{
    return wait_word(reinterpret_cast<const volatile uint64_t *>(t->h_pinned + kDoneWord), seq, s);
}

// Enqueue the traversal order (per flags) and the fused kernel.  done / seq:
// the reduction's completion word (device address) and value, or null.
kdnn_status icp_enqueue(const kdnn_tree *tree, const float *src, int64_t n, const double *R,
                        const double *t, double *sums_dev, int32_t *idx, float *d2,
                        uint32_t flags, const kdnn_icp_reject *rej, const IcpWorkspace &w,
                        hipStream_t s, uint64_t *done = nullptr, uint64_t seq = 0,
                        const IcpLoop *loop = nullptr, int hint_mode = 0)
{
    const float bound2 = rej ? bound_of(rej->max_dist) : INFINITY;
    const bool keep = rej && rej->reject_k > 0.0;
    const int32_t *perm = nullptr;
    hipError_t e = hipSuccess;
    if (flags & KDNN_ICP_NO_SORT) {
        // points in caller order
    } else if (flags & KDNN_ICP_REUSE_ORDER) {
        perm = w.sort.vals_a;
    } else {
        float rt[12];
        rt_to_f32(R, t, rt);
        e = launch_icp_order(tree->dev, src, n, rt, w, &perm, s);
    }
    if (e != hipSuccess) return hip_fail(e, "icp: order launch");
    e = launch_icp_fused(tree->dev, src, n, perm, R, t, w, sums_dev, idx, d2, schedule_of(flags),
                         bound2, keep, s, g_timing.next(), done, seq, loop, hint_mode);
    if (e != hipSuccess) return hip_fail(e, "icp: fused kernel launch");
    return KDNN_OK;
}

kdnn_status icp_check(const kdnn_tree *tree, const float *src, int64_t n, const double *R,
                      const double *t, uint32_t flags, void *ws, size_t ws_bytes)
{
    if (!tree) return fail(KDNN_EINVAL, "icp: null tree");
    if (n < 1) return fail(KDNN_EINVAL, "icp: n must be >= 1");
    kdnn_status st = check_points(src, n, "icp: src");
    if (st != KDNN_OK) return st;
    if (!R || !t) return fail(KDNN_EINVAL, "icp: null R or t");
    if ((flags & ~(KDNN_ICP_REUSE_ORDER | KDNN_ICP_NO_SORT | KDNN_ICP_SORT | kSchedMask)) ||
        !lanes_ok(flags))
        return fail(KDNN_EINVAL, "icp: unknown flag or lane count");
    if ((flags & KDNN_ICP_SORT) && (flags & KDNN_ICP_NO_SORT))
        return fail(KDNN_EINVAL, "icp: KDNN_ICP_SORT and KDNN_ICP_NO_SORT together");
    return check_ws(ws, ws_bytes, icp_ws_bytes(n));
}

// icp_align with the iterations kept on the device: the host enqueues the
// initial state, then per iteration the fused kernel and the step kernel
// (rigid solve, convergence rule, next transform on the device), and waits
// once -- after every 4 iterations when eps > 0, so that a converged
// registration stops soon.  The record the step kernels write (device memory,
// copied into the tree's pinned slot at the end) gives the outputs.  Caller
// holds the tree's ICP lock.
kdnn_status icp_align_on_device(kdnn_tree *mt, const float *src_dev, int64_t n, const double *R,
                                const double *t, int32_t max_iter, double eps, double *R_out,
                                double *t_out, double *E_hist, double *Rt_hist,
                                int32_t *iters_done, uint32_t flags, const kdnn_icp_reject *reject,
                                const IcpWorkspace &w, hipStream_t stream)
{
    constexpr int32_t kChunk = 4;
    hipError_t e = launch_icp_loop_init(w.loop, mt->d_loop, R, t, stream);
    if (e != hipSuccess) return hip_fail(e, "icp_align: loop start");
    const double reject_k = reject ? reject->reject_k : 0.0;
    IcpLoop L{w.loop, mt->d_loop, 0, eps, reject_k > 0.0 ? 1 : 0};
    const IcpLoopOut *out = mt->h_loop;
    constexpr size_t kHead = offsetof(IcpLoopOut, E);
    for (int32_t k = 0; k < max_iter; ++k) {
        L.iter = k;
        const uint32_t f = k == 0 ? flags : (flags | KDNN_ICP_REUSE_ORDER);
        L.mode = reject_k > 0.0 ? 1 : 0;
        const kdnn_status st = icp_enqueue(mt, src_dev, n, R, t, nullptr, nullptr, nullptr, f,
                                           reject, w, stream, nullptr, 0, &L, k == 0 ? 1 : 2);
        if (st != KDNN_OK) return st;
        if (reject_k > 0.0) {
            // residuals under the first solve, then the solve of the kept pairs
            L.mode = 2;
            e = launch_icp_reject(mt->dev, src_dev, n, R, t, reject_k * reject_k, w, nullptr,
                                  nullptr, nullptr, stream, nullptr, 0, &L);
            if (e != hipSuccess) return hip_fail(e, "icp_align: rejection launch");
        }
        if (eps > 0.0 && (k + 1) % kChunk == 0 && k + 1 < max_iter) {
            if ((e = hipMemcpyAsync(mt->h_loop, mt->d_loop, kHead, hipMemcpyDeviceToHost,
                                    stream)) != hipSuccess ||
                (e = hipStreamSynchronize(stream)) != hipSuccess)
                return hip_fail(e, "icp_align: synchronize");
            if (out->stopped) break;
        }
    }
    // the record: header and E_0.. always, the transforms used when asked for
    const size_t nrec = size_t(max_iter);
    if ((e = hipMemcpyAsync(mt->h_loop, mt->d_loop, kHead + nrec * sizeof(double),
                            hipMemcpyDeviceToHost, stream)) != hipSuccess ||
        (Rt_hist && (e = hipMemcpyAsync(mt->h_loop->rt_hist, mt->d_loop->rt_hist,
                                        nrec * sizeof(out->rt_hist[0]), hipMemcpyDeviceToHost,
                                        stream)) != hipSuccess) ||
        (e = hipStreamSynchronize(stream)) != hipSuccess)
        return hip_fail(e, "icp_align: synchronize");
    const int32_t done = int32_t(out->iters);
    const int32_t failed = int32_t(out->fail_iter);
    const int32_t recorded = failed >= 0 ? failed + 1 : done;
    for (int32_t k = 0; k < recorded && k < max_iter; ++k) {
        if (E_hist) E_hist[k] = out->E[k];
        if (Rt_hist)
            for (int j = 0; j < 12; ++j) Rt_hist[12 * k + j] = out->rt_hist[k][j];
    }
    for (int j = 0; j < 9; ++j) R_out[j] = out->rt[j];
    for (int j = 0; j < 3; ++j) t_out[j] = out->rt[9 + j];
    if (iters_done) *iters_done = done;
    if (failed >= 0)
        return fail(KDNN_EDEGENERATE, "icp_align: iteration " + std::to_string(failed) +
                                          (out->fail_phase ? " after rejection: " : ": ") +
                                          rigid_status_text(int32_t(out->status)));
    return KDNN_OK;
}

// icp_align_batch with the iterations kept on the device: each pair's state
// and record live in the workspace; per iteration the batched search and, per
// pair, a one-group step that reduces, solves and advances that pair's loop
// (converged or failed pairs' work-groups return at once).  The host waits
// once (every 4 iterations when eps > 0, stopping when every pair has).
kdnn_status batch_on_device(int32_t B, const kdnn_tree *const *trees, const float *const *src_dev,
                            const int64_t *n, const std::vector<double> &R,
                            const std::vector<double> &t, int32_t max_iter, double eps,
                            double *R_out, double *t_out, double *E_hist, int32_t *iters_done,
                            kdnn_status *status_out, const kdnn_icp_reject *reject, void *ws_dev,
                            int32_t total, const std::vector<int32_t> &part, hipStream_t stream)
{
    constexpr int32_t kChunk = 4;
    constexpr size_t kHead = offsetof(IcpLoopOut, E);
    // strides of the workspace's state and record arrays (256-byte aligned)
    const size_t sb = (sizeof(IcpLoopState) + 255) & ~size_t(255);
    const size_t rb = (sizeof(IcpLoopOut) + 255) & ~size_t(255);
    const size_t row = kHead + size_t(max_iter) * sizeof(double);
    // host staging (ordinary host memory; every copy below is followed by a
    // stream synchronisation before the buffer is read or released): B
    // states, then B record rows
    struct Staging {
        std::vector<char> h;
        hipStream_t s = nullptr;
        ~Staging() { (void)hipStreamSynchronize(s); }  // no copy outlives the buffer
    } pin;
    pin.s = stream;
    pin.h.assign(size_t(B) * (sb + row), 0);
    for (int32_t p = 0; p < B; ++p) {
        IcpLoopState *st = reinterpret_cast<IcpLoopState *>(pin.h.data() + size_t(p) * sb);
        std::memcpy(st->rt, &R[9 * size_t(p)], 9 * sizeof(double));
        std::memcpy(st->rt + 9, &t[3 * size_t(p)], 3 * sizeof(double));
    }
    hipError_t e;
    if ((e = hipMemcpyAsync(batch_loop_state(ws_dev, total, 0), pin.h.data(), size_t(B) * sb,
                            hipMemcpyHostToDevice, stream)) != hipSuccess ||
        (e = launch_batch_loop_init(B, ws_dev, total, stream)) != hipSuccess)
        return hip_fail(e, "icp_align_batch: loop start");
    const float bound2 = reject ? bound_of(reject->max_dist) : INFINITY;
    std::vector<BatchJob> jobs;
    for (int32_t k = 0; k < max_iter; ++k) {
        for (int32_t c0 = 0; c0 < B; c0 += batch_max_pairs()) {
            jobs.clear();
            for (int32_t p = c0; p < B && p < c0 + batch_max_pairs(); ++p) {
                BatchJob J{&trees[p]->dev, src_dev[p], n[p], &R[9 * size_t(p)],
                           &t[3 * size_t(p)], part[p], nullptr, nullptr};
                J.st = batch_loop_state(ws_dev, total, p);
                J.out = batch_loop_out(ws_dev, total, B, p);
                J.hint = batch_hint(ws_dev, total, B, n, p);
                J.hint_in = k > 0;
                jobs.push_back(J);
            }
            if ((e = launch_icp_batch(int32_t(jobs.size()), jobs.data(), bound2, ws_dev, total,
                                      stream, 0, k, eps)) != hipSuccess)
                return hip_fail(e, "icp_align_batch: launch");
        }
        if (eps > 0.0 && (k + 1) % kChunk == 0 && k + 1 < max_iter) {
            if ((e = hipMemcpyAsync(pin.h.data(), batch_loop_state(ws_dev, total, 0),
                                    size_t(B) * sb, hipMemcpyDeviceToHost, stream)) != hipSuccess ||
                (e = hipStreamSynchronize(stream)) != hipSuccess)
                return hip_fail(e, "icp_align_batch: synchronize");
            bool all = true;
            for (int32_t p = 0; p < B; ++p)
                all = all &&
                      reinterpret_cast<const IcpLoopState *>(pin.h.data() + size_t(p) * sb)->stop;
            if (all) break;
        }
    }
    char *rec = pin.h.data() + size_t(B) * sb;
    if ((e = hipMemcpy2DAsync(rec, row, batch_loop_out(ws_dev, total, B, 0), rb, row, size_t(B),
                              hipMemcpyDeviceToHost, stream)) != hipSuccess ||
        (e = hipStreamSynchronize(stream)) != hipSuccess)
        return hip_fail(e, "icp_align_batch: synchronize");
    bool any_failed = false;
    for (int32_t p = 0; p < B; ++p) {
        const IcpLoopOut *out = reinterpret_cast<const IcpLoopOut *>(rec + size_t(p) * row);
        std::memcpy(R_out + 9 * size_t(p), out->rt, 9 * sizeof(double));
        std::memcpy(t_out + 3 * size_t(p), out->rt + 9, 3 * sizeof(double));
        if (iters_done) iters_done[p] = int32_t(out->iters);
        const int64_t failed = out->fail_iter;
        const int64_t recorded = failed >= 0 ? failed + 1 : out->iters;
        if (E_hist)
            for (int64_t k = 0; k < recorded && k < max_iter; ++k)
                E_hist[size_t(p) * max_iter + size_t(k)] = out->E[k];
        if (failed >= 0) {
            if (status_out) status_out[p] = KDNN_EDEGENERATE;
            any_failed = true;
        }
    }
    if (any_failed) return fail(KDNN_EDEGENERATE, "icp_align_batch: a pair degenerated (status_out)");
    return KDNN_OK;
}

}  // namespace

extern "C" {

const char *kdnn_last_error(void) { return g_err.c_str(); }

kdnn_status kdnn_timing_begin(int32_t cap)
{
    KDNN_GUARD_BEGIN
    if (cap < 1 || cap > KDNN_TIMING_MAX)
        return fail(KDNN_EINVAL, "kdnn_timing_begin: cap out of range");
    g_timing.release();
    g_timing.ev.reserve(2 * size_t(cap));
    for (int32_t k = 0; k < 2 * cap; ++k) {
        hipEvent_t e;
        const hipError_t r = hipEventCreate(&e);
        if (r != hipSuccess) {
            g_timing.release();
            return hip_fail(r, "kdnn_timing_begin: hipEventCreate");
        }
        g_timing.ev.push_back(e);
    }
    g_timing.on = true;
    return KDNN_OK;
    KDNN_GUARD_END
}

kdnn_status kdnn_timing_end(float *ms_out, int32_t cap_out, int32_t *count_out)
{
    KDNN_GUARD_BEGIN
    if (!g_timing.on) return fail(KDNN_EINVAL, "kdnn_timing_end: timing not started");
    const int32_t used = g_timing.used;
    if (count_out) *count_out = used;
    if (ms_out && cap_out < used) {
        g_timing.release();
        return fail(KDNN_EINVAL, "kdnn_timing_end: cap_out smaller than the launch count");
    }
    for (int32_t k = 0; ms_out && k < used; ++k) {
        hipEvent_t a = g_timing.ev[2 * size_t(k)], b = g_timing.ev[2 * size_t(k) + 1];
        hipError_t r = hipEventSynchronize(b);
        if (r == hipSuccess) r = hipEventElapsedTime(&ms_out[k], a, b);
        if (r != hipSuccess) {
            g_timing.release();
            return hip_fail(r, "kdnn_timing_end: event");
        }
    }
    g_timing.release();
    return KDNN_OK;
    KDNN_GUARD_END
}

kdnn_status kdnn_gather_bench(const void *buf_dev, int64_t n_records, int32_t words, int64_t lanes,
                              int32_t rounds, uint32_t seed, uint32_t *sink_dev, float *ms_out,
                              hipStream_t stream)
{
    KDNN_GUARD_BEGIN
    if (!buf_dev || !aligned(buf_dev, 16) || !sink_dev || !aligned(sink_dev, 4) || !ms_out)
        return fail(KDNN_EINVAL, "kdnn_gather_bench: null or misaligned pointer");
    if (!(words == 1 || words == 3 || words == 16))
        return fail(KDNN_EINVAL, "kdnn_gather_bench: words must be 1, 3 or 16");
    if (n_records < 1 || n_records > int64_t(UINT32_MAX))
        return fail(KDNN_EINVAL, "kdnn_gather_bench: n_records out of range");
    if (lanes < 256 || lanes % 256 != 0 || lanes / 256 > int64_t(INT32_MAX))
        return fail(KDNN_EINVAL, "kdnn_gather_bench: lanes must be a positive multiple of 256");
    if (rounds < 4 || rounds % 4 != 0)
        return fail(KDNN_EINVAL, "kdnn_gather_bench: rounds must be a positive multiple of 4");
    if (!run_gather_bench(buf_dev, n_records, words, lanes, rounds, seed, sink_dev, ms_out, stream))
        return hip_fail(hipGetLastError(), "kdnn_gather_bench");
    return KDNN_OK;
    KDNN_GUARD_END
}

kdnn_status kdnn_chase_bench(const uint32_t *next_dev, int64_t n_records, int32_t waves,
                             int32_t steps, uint32_t *sink_dev, float *ms_out, hipStream_t stream)
{
    KDNN_GUARD_BEGIN
    if (!next_dev || !aligned(next_dev, 64) || !sink_dev || !aligned(sink_dev, 4) || !ms_out)
        return fail(KDNN_EINVAL, "kdnn_chase_bench: null or misaligned pointer");
    if (n_records < 1 || n_records > int64_t(UINT32_MAX))
        return fail(KDNN_EINVAL, "kdnn_chase_bench: n_records out of range");
    if (waves < 1 || steps < 1)
        return fail(KDNN_EINVAL, "kdnn_chase_bench: waves and steps must be >= 1");
    if (!run_chase_bench(next_dev, n_records, waves, steps, sink_dev, ms_out, stream))
        return hip_fail(hipGetLastError(), "kdnn_chase_bench");
    return KDNN_OK;
    KDNN_GUARD_END
}

size_t kdnn_replay_workspace_bytes(const kdnn_tree *tree, int64_t m, uint32_t flags)
{
    if (!tree || m < 1) return 0;
    try {
        const size_t q = (query_ws_bytes(m) + 255) & ~size_t(255);
        return q + replay_ws_bytes(tree->dev, m, (flags & KDNN_REPLAY_ICP) != 0);
    } catch (...) {
        return 0;
    }
}

kdnn_status kdnn_replay_bench(const kdnn_tree *tree, const float *q_dev, const float *q_prev_dev,
                              int64_t m, uint32_t flags, int32_t reps, void *ws_dev,
                              size_t ws_bytes, float *ms_out, kdnn_replay_info *info,
                              hipStream_t stream)
{
    KDNN_GUARD_BEGIN
    if (!tree) return fail(KDNN_EINVAL, "kdnn_replay_bench: null tree");
    if (m < 1) return fail(KDNN_EINVAL, "kdnn_replay_bench: m must be >= 1");
    kdnn_status st = check_points(q_dev, m, "kdnn_replay_bench: queries");
    if (st != KDNN_OK) return st;
    if (q_prev_dev && (st = check_points(q_prev_dev, m, "kdnn_replay_bench: previous queries")) !=
                          KDNN_OK)
        return st;
    if (reps < 1 || !ms_out || !info)
        return fail(KDNN_EINVAL, "kdnn_replay_bench: reps < 1 or null ms_out / info");
    if (flags & ~(KDNN_QUERY_NO_SORT | KDNN_QUERY_SORT | KDNN_REPLAY_ICP))
        return fail(KDNN_EINVAL, "kdnn_replay_bench: unknown flag");
    if ((flags & KDNN_QUERY_SORT) && (flags & KDNN_QUERY_NO_SORT))
        return fail(KDNN_EINVAL, "kdnn_replay_bench: KDNN_QUERY_SORT and KDNN_QUERY_NO_SORT together");
    const bool icp = (flags & KDNN_REPLAY_ICP) != 0;
    const size_t need = kdnn_replay_workspace_bytes(tree, m, flags);
    if (need == 0) return fail(KDNN_EINVAL, "kdnn_replay_bench: workspace size unavailable");
    if ((st = check_ws(ws_dev, ws_bytes, need)) != KDNN_OK) return st;
    const bool sort = (flags & KDNN_QUERY_SORT) ||
                      (!(flags & KDNN_QUERY_NO_SORT) && (icp ? tree->auto_sort_icp : tree->auto_sort));
    const QueryWorkspace qw = carve_query_workspace(ws_dev, m);
    const int32_t *perm = nullptr;
    hipError_t e = hipSuccess;
    if (sort && (e = launch_morton_order(tree->dev, q_dev, m, nullptr,
                                         icp ? kKeyBitsIcp : kKeyBitsQuery, qw.sort, &perm,
                                         stream)) != hipSuccess)
        return hip_fail(e, "kdnn_replay_bench: order launch");
    void *rws = static_cast<char *>(ws_dev) + ((query_ws_bytes(m) + 255) & ~size_t(255));
    *info = kdnn_replay_info{};
    if ((e = launch_replay(tree->dev, q_dev, m, perm, icp, q_prev_dev, rws, reps, ms_out, info,
                           stream)) != hipSuccess)
        return hip_fail(e, "kdnn_replay_bench");
    return KDNN_OK;
    KDNN_GUARD_END
}

int32_t kdnn_version(void) { return KDNN_VERSION; }

kdnn_status kdtree_layout(int64_t n, const kdnn_build_params *params, int32_t *depth_out,
                          int64_t *node_slots_out)
{
    KDNN_GUARD_BEGIN
    if (!depth_out || !node_slots_out) return fail(KDNN_EINVAL, "kdtree_layout: null output");
    std::string err;
    kdnn_status st = tree_layout(n, params, depth_out, node_slots_out, err);
    return st == KDNN_OK ? st : fail(st, err);
    KDNN_GUARD_END
}

kdnn_status kdtree_build_host(const float *xyz_host, int64_t n, const kdnn_build_params *params,
                              float *nodes_out, float *points_out)
{
    KDNN_GUARD_BEGIN
    if (!nodes_out || !points_out) return fail(KDNN_EINVAL, "kdtree_build_host: null output");
    HostTree ht;
    std::string err;
    kdnn_status st = build_host_tree(xyz_host, n, params, ht, err);
    if (st != KDNN_OK) return fail(st, err);
    std::memcpy(nodes_out, ht.nodes.data(), ht.nodes.size() * sizeof(float));
    std::memcpy(points_out, ht.points.data(), ht.points.size() * sizeof(float));
    return KDNN_OK;
    KDNN_GUARD_END
}

kdnn_status kdtree_build(const float *xyz_host, int64_t n, const kdnn_build_params *params,
                         kdnn_tree **out)
{
    KDNN_GUARD_BEGIN
    if (!out) return fail(KDNN_EINVAL, "kdtree_build: null output handle");
    HostTree ht;
    std::string err;
    const auto t0 = std::chrono::steady_clock::now();
    kdnn_status st = build_host_tree(xyz_host, n, params, ht, err);
    if (st != KDNN_OK) return fail(st, err);
    const double build_ms = ms_since(t0);

    const auto t1 = std::chrono::steady_clock::now();
    kdnn_tree *t = new kdnn_tree();
    hipError_t e = hipGetDevice(&t->device);
    if (e != hipSuccess) {
        delete t;
        return hip_fail(e, "kdtree_build: hipGetDevice");
    }
    // kPointPad sentinel points after the last one: +inf coordinates and index
    // 0xFFFFFFFF (never a hit), so a search may read whole chunks past a leaf.
    constexpr size_t kPointPad = 16;
    const size_t nb = ht.nodes.size() * sizeof(float), pb = ht.points.size() * sizeof(float);
    const size_t pad_bytes = kPointPad * 4 * sizeof(float);
    std::vector<float> pad(kPointPad * 4, INFINITY);
    for (size_t k = 0; k < kPointPad; ++k) {
        const uint32_t none = 0xFFFFFFFFu;
        std::memcpy(&pad[4 * k + 3], &none, 4);
    }
    std::vector<int32_t> slot_of(static_cast<size_t>(n));
    for (int64_t k = 0; k < n; ++k) {
        uint32_t j;
        std::memcpy(&j, &ht.points[4 * size_t(k) + 3], 4);
        slot_of[j] = int32_t(k);
    }
    // The boxes alone, 24 bytes per node slot, so that the two children of
    // node i are one 48-byte run (three 16-byte loads) for the search.
    const size_t slots = ht.nodes.size() / kNodeWords;
    std::vector<float> boxes(6 * slots);
    for (size_t r = 0; r < slots; ++r)
        std::memcpy(&boxes[6 * r], &ht.nodes[r * kNodeWords], 6 * sizeof(float));
    const size_t bb = boxes.size() * sizeof(float);
    const size_t ob = size_t(n) * sizeof(int32_t);
    // Each leaf's plane record (warm starts): for its ancestors at depths D-1,
    // D-2, .. (at most kPathLevels of them) the split axis and the near face,
    // along that axis, of the box of the child off the leaf's path (its lo
    // for a right child, its hi for a left one; at or beyond the split).
    const size_t leaves = size_t(1) << ht.depth;
    std::vector<uint32_t> paths(leaves * kPathWords, 0u);
    for (size_t j = 0; j < leaves; ++j) {
        uint32_t *rec = &paths[j * kPathWords];
        const size_t leaf = leaves + j;
        for (int k = 0; k < kPathLevels && k < ht.depth; ++k) {
            const float *w = &ht.nodes[(leaf >> (k + 1)) * kNodeWords];
            uint32_t ax;
            std::memcpy(&ax, &w[7], 4);
            ax &= 3u;
            const size_t sib = (leaf >> k) ^ 1u;
            const float *sb = &ht.nodes[sib * kNodeWords];
            const float face = (sib & 1u) ? sb[ax] : sb[3 + ax];
            rec[0] |= ax << (2 * k);
            std::memcpy(&rec[1 + k], &face, 4);
        }
    }
    const size_t rb = paths.size() * sizeof(uint32_t);
    if ((e = hipMalloc(&t->d_nodes, nb)) != hipSuccess ||
        (e = hipMalloc(&t->d_boxes, bb)) != hipSuccess ||
        (e = hipMalloc(&t->d_points, pb + pad_bytes)) != hipSuccess ||
        (e = hipMalloc(&t->d_slot_of, ob)) != hipSuccess ||
        (e = hipMalloc(&t->d_paths, rb)) != hipSuccess) {
        free_tree(t);
        return fail(KDNN_ENOMEM, std::string("kdtree_build: hipMalloc: ") + hipGetErrorString(e));
    }
    if ((e = hipHostMalloc(reinterpret_cast<void **>(&t->h_pinned), 256, hipHostMallocDefault)) !=
        hipSuccess) {
        free_tree(t);
        return fail(KDNN_ENOMEM, std::string("kdtree_build: hipHostMalloc: ") + hipGetErrorString(e));
    }
    std::memset(t->h_pinned, 0, 256);  // completion word 0: no launch yet
    // The fused kernel of the synchronous ICP calls writes its sums straight
    // into this slot (no separate copy launch per iteration).
    if ((e = hipHostGetDevicePointer(reinterpret_cast<void **>(&t->d_pinned), t->h_pinned, 0)) !=
        hipSuccess) {
        free_tree(t);
        return hip_fail(e, "kdtree_build: hipHostGetDevicePointer");
    }
    // the record the device-side ICP loop writes (per-iteration E and transform):
    // in device memory, copied once into pinned memory at the end of a
    // registration (writes to host memory would hold up every step kernel's
    // completion by a PCIe round trip)
    if ((e = hipMalloc(reinterpret_cast<void **>(&t->d_loop), sizeof(kdnn::IcpLoopOut))) !=
            hipSuccess ||
        (e = hipHostMalloc(reinterpret_cast<void **>(&t->h_loop), sizeof(kdnn::IcpLoopOut),
                           hipHostMallocDefault)) != hipSuccess) {
        free_tree(t);
        return fail(KDNN_ENOMEM, std::string("kdtree_build: loop record: ") + hipGetErrorString(e));
    }
    std::memset(static_cast<void *>(t->h_loop), 0, sizeof(kdnn::IcpLoopOut));
    if ((e = hipMemcpy(t->d_nodes, ht.nodes.data(), nb, hipMemcpyHostToDevice)) != hipSuccess ||
        (e = hipMemcpy(t->d_boxes, boxes.data(), bb, hipMemcpyHostToDevice)) != hipSuccess ||
        (e = hipMemcpy(t->d_points, ht.points.data(), pb, hipMemcpyHostToDevice)) != hipSuccess ||
        (e = hipMemcpy(static_cast<char *>(t->d_points) + pb, pad.data(), pad_bytes,
                       hipMemcpyHostToDevice)) != hipSuccess ||
        (e = hipMemcpy(t->d_slot_of, slot_of.data(), ob, hipMemcpyHostToDevice)) != hipSuccess ||
        (e = hipMemcpy(t->d_paths, paths.data(), rb, hipMemcpyHostToDevice)) != hipSuccess) {
        free_tree(t);
        return hip_fail(e, "kdtree_build: upload");
    }
    const double upload_ms = ms_since(t1);

    DeviceTree &d = t->dev;
    d.nodes = t->d_nodes;
    d.boxes = t->d_boxes;
    d.points = t->d_points;
    d.slot_of = t->d_slot_of;
    d.paths = t->d_paths;
    d.first_leaf = uint32_t(1) << ht.depth;
    d.depth = ht.depth;
    d.max_leaf = ht.max_leaf;
    d.n = n;
    for (int k = 0; k < 3; ++k) {
        d.box_lo[k] = ht.bbox_min[k];
        const float ext = ht.bbox_max[k] - ht.bbox_min[k];
        d.box_inv[k] = ext > 0.0f ? 1.0f / ext : 0.0f;
        d.center[k] = ht.center[k];
    }
    kdnn_tree_info &I = t->info;
    I.n = n;
    I.depth = ht.depth;
    I.leaf_size = ht.leaf_size;
    I.node_slots = int64_t(1) << (ht.depth + 1);
    I.leaves = int64_t(1) << ht.depth;
    I.min_leaf = ht.min_leaf;
    I.max_leaf = ht.max_leaf;
    for (int k = 0; k < 3; ++k) {
        I.bbox_min[k] = ht.bbox_min[k];
        I.bbox_max[k] = ht.bbox_max[k];
        I.center[k] = ht.center[k];
    }
    I.build_ms = build_ms;
    I.upload_ms = upload_ms;
    I.device_bytes = int64_t(nb + bb + pb + pad_bytes + ob + rb);
    int l2 = 0;
    if ((e = hipDeviceGetAttribute(&l2, hipDeviceAttributeL2CacheSize, t->device)) != hipSuccess) {
        free_tree(t);
        return hip_fail(e, "kdtree_build: L2 size query");
    }
    // nn_query pays the ordering on every call, ICP once per registration
    const size_t l2b = size_t(l2 > 0 ? l2 : 0);
    t->auto_sort = nb + pb > kQuerySortL2Multiple * l2b;
    t->auto_sort_icp = nb + pb > l2b;
    I.l2_bytes = l2;
    I.auto_sort = t->auto_sort ? 1 : 0;
    I.auto_sort_icp = t->auto_sort_icp ? 1 : 0;
    *out = t;
    return KDNN_OK;
    KDNN_GUARD_END
}

void kdtree_free(kdnn_tree *tree)
{
    try {
        free_tree(tree);
    } catch (...) {
    }
}

kdnn_status kdtree_info(const kdnn_tree *tree, kdnn_tree_info *out)
{
    if (!tree || !out) return fail(KDNN_EINVAL, "kdtree_info: null pointer");
    *out = tree->info;
    return KDNN_OK;
}

size_t nn_query_workspace_bytes(int64_t m) { return query_ws_bytes(m); }

static kdnn_status nn_query_impl(const kdnn_tree *tree, const float *q, int64_t m, int32_t *idx,
                                 float *d2, uint32_t *cn, uint32_t *cp, bool stats, uint32_t flags,
                                 float bound2, void *ws, size_t ws_bytes, hipStream_t s)
{
    if (!tree) return fail(KDNN_EINVAL, "nn_query: null tree");
    kdnn_status st = check_points(q, m, "nn_query: queries");
    if (st != KDNN_OK) return st;
    if (m == 0) return KDNN_OK;
    if (!idx || !d2) return fail(KDNN_EINVAL, "nn_query: null output");
    if (!aligned(idx, 4) || !aligned(d2, 4)) return fail(KDNN_EINVAL, "nn_query: misaligned output");
    if ((flags & ~(KDNN_QUERY_NO_SORT | KDNN_QUERY_SORT | kSchedMask)) || !lanes_ok(flags))
        return fail(KDNN_EINVAL, "nn_query: unknown flag or lane count");
    if ((flags & KDNN_QUERY_SORT) && (flags & KDNN_QUERY_NO_SORT))
        return fail(KDNN_EINVAL, "nn_query: KDNN_QUERY_SORT and KDNN_QUERY_NO_SORT together");
    if ((flags & KDNN_QUERY_SORT) && !ws)
        return fail(KDNN_EINVAL, "nn_query: the Morton ordering needs a workspace");
    if ((flags & KDNN_BUDGET_MASK) && !ws)
        return fail(KDNN_EINVAL, "nn_query: the two-pass schedule needs a workspace");
    const bool sort = (flags & KDNN_QUERY_SORT) ||
                      (!(flags & KDNN_QUERY_NO_SORT) && tree->auto_sort && ws);
    const int32_t *perm = nullptr;
    void *twopass = nullptr;
    if (ws) {
        st = check_ws(ws, ws_bytes, query_ws_bytes(m));
        if (st != KDNN_OK) return st;
        const QueryWorkspace w = carve_query_workspace(ws, m);
        twopass = w.twopass;
        if (sort) {
            hipError_t e = launch_morton_order(tree->dev, q, m, nullptr, kKeyBitsQuery, w.sort, &perm, s);
            if (e != hipSuccess) return hip_fail(e, "nn_query: order launch");
        }
    }
    hipError_t e = launch_nn(tree->dev, q, m, perm, idx, d2, cn, cp, stats, schedule_of(flags),
                             bound2, twopass, s, stats ? nullptr : g_timing.next());
    if (e != hipSuccess) return hip_fail(e, "nn_query: launch");
    return KDNN_OK;
}

kdnn_status nn_query(const kdnn_tree *tree, const float *q_dev, int64_t m, int32_t *idx_dev,
                     float *dist2_dev, uint32_t flags, void *ws_dev, size_t ws_bytes,
                     hipStream_t stream)
{
    KDNN_GUARD_BEGIN
    return nn_query_impl(tree, q_dev, m, idx_dev, dist2_dev, nullptr, nullptr, false, flags,
                         INFINITY, ws_dev, ws_bytes, stream);
    KDNN_GUARD_END
}

kdnn_status nn_query_radius(const kdnn_tree *tree, const float *q_dev, int64_t m, double max_dist,
                            int32_t *idx_dev, float *dist2_dev, uint32_t flags, void *ws_dev,
                            size_t ws_bytes, hipStream_t stream)
{
    KDNN_GUARD_BEGIN
    if (std::isnan(max_dist)) return fail(KDNN_EINVAL, "nn_query_radius: max_dist is NaN");
    return nn_query_impl(tree, q_dev, m, idx_dev, dist2_dev, nullptr, nullptr, false, flags,
                         bound_of(max_dist), ws_dev, ws_bytes, stream);
    KDNN_GUARD_END
}

kdnn_status nn_query_stats(const kdnn_tree *tree, const float *q_dev, int64_t m, int32_t *idx_dev,
                           float *dist2_dev, uint32_t *nodes_dev, uint32_t *points_dev,
                           uint32_t flags, void *ws_dev, size_t ws_bytes, hipStream_t stream)
{
    KDNN_GUARD_BEGIN
    return nn_query_impl(tree, q_dev, m, idx_dev, dist2_dev, nodes_dev, points_dev, true, flags,
                         INFINITY, ws_dev, ws_bytes, stream);
    KDNN_GUARD_END
}

kdnn_status transform_points(const float *in_dev, float *out_dev, int64_t n, const double *R_host,
                             const double *t_host, hipStream_t stream)
{
    KDNN_GUARD_BEGIN
    kdnn_status st = check_points(in_dev, n, "transform_points: in");
    if (st != KDNN_OK) return st;
    st = check_points(out_dev, n, "transform_points: out");
    if (st != KDNN_OK) return st;
    if (!R_host || !t_host) return fail(KDNN_EINVAL, "transform_points: null R or t");
    if (n == 0) return KDNN_OK;
    if (in_dev != out_dev) {
        const char *a = reinterpret_cast<const char *>(in_dev);
        const char *b = reinterpret_cast<const char *>(out_dev);
        const size_t len = size_t(n) * 12;
        if (a < b + len && b < a + len)
            return fail(KDNN_EINVAL, "transform_points: in and out partially overlap");
    }
    hipError_t e = launch_transform(in_dev, out_dev, n, R_host, t_host, stream);
    if (e != hipSuccess) return hip_fail(e, "transform_points: launch");
    return KDNN_OK;
    KDNN_GUARD_END
}

size_t icp_workspace_bytes(int64_t n) { return n > 0 ? icp_ws_bytes(n) : 0; }

kdnn_status icp_correspond_reduce_async(const kdnn_tree *tree, const float *src_dev, int64_t n,
                                        const double *R_host, const double *t_host,
                                        double *sums_dev, int32_t *idx_dev, float *dist2_dev,
                                        uint32_t flags, const kdnn_icp_reject *reject,
                                        void *ws_dev, size_t ws_bytes, hipStream_t stream)
{
    KDNN_GUARD_BEGIN
    kdnn_status st = icp_check(tree, src_dev, n, R_host, t_host, flags, ws_dev, ws_bytes);
    if (st != KDNN_OK) return st;
    if ((st = check_reject(reject, "icp_correspond_reduce_async")) != KDNN_OK) return st;
    if (!sums_dev || !aligned(sums_dev, 8)) return fail(KDNN_EINVAL, "icp: bad sums_dev");
    const IcpWorkspace w = carve_icp_workspace(ws_dev, n);
    return icp_enqueue(tree, src_dev, n, R_host, t_host, sums_dev, idx_dev, dist2_dev,
                       icp_resolve_sort(tree, flags), reject, w, stream);
    KDNN_GUARD_END
}

kdnn_status icp_correspond_reduce(const kdnn_tree *tree, const float *src_dev, int64_t n,
                                  const double *R_host, const double *t_host,
                                  kdnn_icp_sums *out_host, int32_t *idx_dev, float *dist2_dev,
                                  uint32_t flags, const kdnn_icp_reject *reject, void *ws_dev,
                                  size_t ws_bytes, hipStream_t stream)
{
    KDNN_GUARD_BEGIN
    kdnn_status st = icp_check(tree, src_dev, n, R_host, t_host, flags, ws_dev, ws_bytes);
    if (st != KDNN_OK) return st;
    if ((st = check_reject(reject, "icp_correspond_reduce")) != KDNN_OK) return st;
    if (!out_host) return fail(KDNN_EINVAL, "icp: null out_host");
    kdnn_tree *mt = const_cast<kdnn_tree *>(tree);
    std::lock_guard<std::mutex> lock(mt->icp_mu);
    const IcpWorkspace w = carve_icp_workspace(ws_dev, n);
    st = icp_enqueue(tree, src_dev, n, R_host, t_host, mt->d_pinned, idx_dev, dist2_dev,
                     icp_resolve_sort(tree, flags), reject, w, stream);
    if (st != KDNN_OK) return st;
    hipError_t e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "icp: synchronize");
    to_sums(mt->h_pinned, tree->dev.center, out_host);
    return KDNN_OK;
    KDNN_GUARD_END
}

kdnn_status icp_reject_reduce(const kdnn_tree *tree, const float *src_dev, int64_t n,
                              const double *R_host, const double *t_host, double reject_k,
                              kdnn_icp_sums *out_host, double *sigma2_out, uint8_t *kept_dev,
                              void *ws_dev, size_t ws_bytes, hipStream_t stream)
{
    KDNN_GUARD_BEGIN
    kdnn_status st = icp_check(tree, src_dev, n, R_host, t_host, 0, ws_dev, ws_bytes);
    if (st != KDNN_OK) return st;
    if (!(reject_k > 0.0 && std::isfinite(reject_k)))
        return fail(KDNN_EINVAL, "icp_reject_reduce: reject_k must be finite and > 0");
    if (!out_host) return fail(KDNN_EINVAL, "icp_reject_reduce: null out_host");
    kdnn_tree *mt = const_cast<kdnn_tree *>(tree);
    std::lock_guard<std::mutex> lock(mt->icp_mu);
    const IcpWorkspace w = carve_icp_workspace(ws_dev, n);
    hipError_t e = launch_icp_reject(tree->dev, src_dev, n, R_host, t_host, reject_k * reject_k, w,
                          mt->d_pinned, mt->d_pinned + KDNN_SUMS_DOUBLES, kept_dev, stream);
    if (e != hipSuccess) return hip_fail(e, "icp_reject_reduce: launch");
    if ((e = hipStreamSynchronize(stream)) != hipSuccess)
        return hip_fail(e, "icp_reject_reduce: synchronize");
    to_sums(mt->h_pinned, tree->dev.center, out_host);
    if (sigma2_out) *sigma2_out = mt->h_pinned[KDNN_SUMS_DOUBLES];
    return KDNN_OK;
    KDNN_GUARD_END
}

kdnn_status kdnn_moments(const kdnn_icp_sums *sums, kdnn_icp_moments *out)
{
    KDNN_GUARD_BEGIN
    if (!sums || !out) return fail(KDNN_EINVAL, "kdnn_moments: null pointer");
    moments_of_sums(*sums, *out);
    return KDNN_OK;
    KDNN_GUARD_END
}

kdnn_status kdnn_procrustes(const kdnn_icp_sums *sums, double *R_out, double *t_out)
{
    KDNN_GUARD_BEGIN
    if (!sums || !R_out || !t_out) return fail(KDNN_EINVAL, "kdnn_procrustes: null pointer");
    std::string err;
    double R[9], t[3];
    kdnn_status st = procrustes_from_sums(*sums, R, t, err);
    if (st != KDNN_OK) return fail(st, err);
    std::memcpy(R_out, R, sizeof R);
    std::memcpy(t_out, t, sizeof t);
    return KDNN_OK;
    KDNN_GUARD_END
}

kdnn_status icp_align(const kdnn_tree *tree, const float *src_dev, int64_t n, const double *R0_host,
                      const double *t0_host, int32_t max_iter, double eps, double *R_out,
                      double *t_out, double *E_hist, double *Rt_hist, int32_t *iters_done,
                      uint32_t flags, const kdnn_icp_reject *reject, void *ws_dev,
                      size_t ws_bytes, hipStream_t stream)
{
    KDNN_GUARD_BEGIN
    double R[9], t[3];
    std::memcpy(R, R0_host ? R0_host : kI, sizeof R);
    std::memcpy(t, t0_host ? t0_host : kZ, sizeof t);
    if (!R_out || !t_out) return fail(KDNN_EINVAL, "icp_align: null R_out or t_out");
    if (max_iter < 0) return fail(KDNN_EINVAL, "icp_align: max_iter < 0");
    if (!(eps >= 0.0)) return fail(KDNN_EINVAL, "icp_align: eps must be >= 0");
    if (flags & ~(KDNN_ICP_NO_SORT | KDNN_ICP_SORT | KDNN_ICP_HOST_LOOP | KDNN_ICP_DEVICE_LOOP |
                  kSchedMask))
        return fail(KDNN_EINVAL, "icp_align: unknown flag");
    if ((flags & KDNN_ICP_HOST_LOOP) && (flags & KDNN_ICP_DEVICE_LOOP))
        return fail(KDNN_EINVAL, "icp_align: KDNN_ICP_HOST_LOOP and KDNN_ICP_DEVICE_LOOP together");
    const bool device_loop = (flags & KDNN_ICP_DEVICE_LOOP) != 0;
    flags &= ~(KDNN_ICP_HOST_LOOP | KDNN_ICP_DEVICE_LOOP);
    if (device_loop) {
        const Schedule sc0 = schedule_of(flags);
        if (sc0.lanes > 1 || sc0.top_lds || sc0.budget != 0)
            return fail(KDNN_EINVAL, "icp_align: KDNN_ICP_DEVICE_LOOP needs one lane per query "
                                     "(no schedule flag or KDNN_LANES(1))");
        if (max_iter > kLoopMaxIter)
            return fail(KDNN_EINVAL, "icp_align: KDNN_ICP_DEVICE_LOOP records at most " +
                                         std::to_string(kLoopMaxIter) + " iterations");
    }
    kdnn_status st = icp_check(tree, src_dev, n, R, t, flags, ws_dev, ws_bytes);
    if (st != KDNN_OK) return st;
    if ((st = check_reject(reject, "icp_align")) != KDNN_OK) return st;
    flags = icp_resolve_sort(tree, flags);
    const double reject_k = reject ? reject->reject_k : 0.0;
    std::memcpy(R_out, R, sizeof R);
    std::memcpy(t_out, t, sizeof t);
    if (iters_done) *iters_done = 0;
    if (max_iter == 0) return KDNN_OK;

    kdnn_tree *mt = const_cast<kdnn_tree *>(tree);
    std::lock_guard<std::mutex> lock(mt->icp_mu);
    const IcpWorkspace w = carve_icp_workspace(ws_dev, n);
    if (device_loop)
        return icp_align_on_device(mt, src_dev, n, R, t, max_iter, eps, R_out, t_out, E_hist,
                                   Rt_hist, iters_done, flags, reject, w, stream);
    double prev_mse = 0.0;
    int small_steps = 0;
    for (int32_t k = 0; k < max_iter; ++k) {
        if (Rt_hist) {
            std::memcpy(Rt_hist + 12 * k, R, sizeof R);
            std::memcpy(Rt_hist + 12 * k + 9, t, sizeof t);
        }
        const uint32_t f = k == 0 ? flags : (flags | KDNN_ICP_REUSE_ORDER);
        const uint64_t seq = ++mt->seq;
        st = icp_enqueue(tree, src_dev, n, R, t, mt->d_pinned, nullptr, nullptr, f, reject, w,
                         stream, reinterpret_cast<uint64_t *>(mt->d_pinned + kDoneWord), seq,
                         nullptr, k == 0 ? 1 : 2);
        if (st != KDNN_OK) return st;
        hipError_t e = wait_sums(mt, seq, stream);
        if (e != hipSuccess) return hip_fail(e, "icp_align: wait for the sums");
        kdnn_icp_sums sums;
        to_sums(mt->h_pinned, tree->dev.center, &sums);
        if (E_hist) E_hist[k] = sums.sum_d2;
        std::string err;
        double Rn[9], tn[3];
        st = procrustes_from_sums(sums, Rn, tn, err);
        if (st != KDNN_OK) return fail(st, "icp_align: iteration " + std::to_string(k) + ": " + err);
        if (reject_k > 0.0) {
            // residual rejection under the first solve, then solve again
            const uint64_t rseq = ++mt->seq;
            e = launch_icp_reject(tree->dev, src_dev, n, Rn, tn, reject_k * reject_k, w,
                                  mt->d_pinned, nullptr, nullptr, stream,
                                  reinterpret_cast<uint64_t *>(mt->d_pinned + kDoneWord), rseq);
            if (e != hipSuccess) return hip_fail(e, "icp_align: rejection launch");
            if ((e = wait_sums(mt, rseq, stream)) != hipSuccess)
                return hip_fail(e, "icp_align: wait for the kept sums");
            kdnn_icp_sums kept;
            to_sums(mt->h_pinned, tree->dev.center, &kept);
            st = procrustes_from_sums(kept, Rn, tn, err);
            if (st != KDNN_OK)
                return fail(st, "icp_align: iteration " + std::to_string(k) + " after rejection: " + err);
        }
        std::memcpy(R, Rn, sizeof R);
        std::memcpy(t, tn, sizeof t);
        std::memcpy(R_out, R, sizeof R);
        std::memcpy(t_out, t, sizeof t);
        if (iters_done) *iters_done = k + 1;
        const double mse = sums.sum_d2 / double(sums.n);
        if (eps > 0.0 && k > 0) {
            small_steps = std::fabs(mse - prev_mse) < eps ? small_steps + 1 : 0;
            if (small_steps >= 2) break;
        }
        prev_mse = mse;
    }
    // the loop waited for the sums only; leave the stream idle, as documented
    const hipError_t e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "icp_align: synchronize");
    return KDNN_OK;
    KDNN_GUARD_END
}

kdnn_status icp_align_noalloc(const kdnn_tree *tree, const float *src_dev, int64_t n,
                              const double *R0_host, const double *t0_host, int32_t max_iter,
                              double eps, double *R_out, double *t_out, double *E_hist,
                              double *Rt_hist, int32_t *iters_done, uint32_t flags,
                              const kdnn_icp_reject *reject, hipStream_t stream)
{
    KDNN_GUARD_BEGIN
    if (!tree) return fail(KDNN_EINVAL, "icp_align_noalloc: null tree");
    if (n > KDNN_NOALLOC_MAX_POINTS)
        return fail(KDNN_EINVAL, "icp_align_noalloc: n = " + std::to_string(n) + " exceeds " +
                                     std::to_string(KDNN_NOALLOC_MAX_POINTS) +
                                     " (the scratch limit; use icp_align with a workspace)");
    const size_t need = icp_ws_bytes(n);
    if (need > size_t(KDNN_NOALLOC_SCRATCH_BYTES))
        return fail(KDNN_EINVAL, "icp_align_noalloc: workspace larger than the scratch");
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "icp_align_noalloc: hipGetDevice");
    if (tree->device != dev)
        return fail(KDNN_EINVAL, "icp_align_noalloc: the tree lives on another device");
    void *ptr = nullptr;
    std::mutex *call_mu = nullptr;
    if ((e = noalloc_scratch(dev, &ptr, &call_mu)) != hipSuccess)
        return hip_fail(e, "icp_align_noalloc: scratch address");
    std::lock_guard<std::mutex> lock(*call_mu);
    return icp_align(tree, src_dev, n, R0_host, t0_host, max_iter, eps, R_out, t_out, E_hist,
                     Rt_hist, iters_done, flags, reject, ptr, size_t(KDNN_NOALLOC_SCRATCH_BYTES),
                     stream);
    KDNN_GUARD_END
}

size_t voxel_downsample_workspace_bytes(int64_t n) { return voxel_ws_bytes(n); }

kdnn_status voxel_downsample(const float *xyz_dev, int64_t n, double leaf, float *out_dev,
                             int64_t *m_out, int32_t *counts_dev, void *ws_dev, size_t ws_bytes,
                             hipStream_t stream)
{
    KDNN_GUARD_BEGIN
    if (!m_out) return fail(KDNN_EINVAL, "voxel_downsample: null m_out");
    *m_out = 0;
    kdnn_status st = check_points(xyz_dev, n, "voxel_downsample: points");
    if (st != KDNN_OK) return st;
    if (!(leaf > 0.0 && std::isfinite(leaf)))
        return fail(KDNN_EINVAL, "voxel_downsample: leaf must be finite and > 0");
    if (n == 0) return KDNN_OK;
    if (!out_dev || !aligned(out_dev, 4)) return fail(KDNN_EINVAL, "voxel_downsample: bad out");
    if (counts_dev && !aligned(counts_dev, 4))
        return fail(KDNN_EINVAL, "voxel_downsample: misaligned counts");
    if ((st = check_ws(ws_dev, ws_bytes, voxel_ws_bytes(n))) != KDNN_OK) return st;
    const VoxelWorkspace w = carve_voxel_workspace(ws_dev, n);
    hipError_t e = launch_voxel_filter(xyz_dev, n, leaf, w, out_dev, counts_dev, stream);
    if (e != hipSuccess) return hip_fail(e, "voxel_downsample: launch");
    VoxGrid g{};
    if ((e = hipMemcpyAsync(&g, w.grid, sizeof g, hipMemcpyDeviceToHost, stream)) != hipSuccess ||
        (e = hipStreamSynchronize(stream)) != hipSuccess)
        return hip_fail(e, "voxel_downsample: synchronize");
    if (g.err == kVoxErrRange)
        return fail(KDNN_EINVAL, "voxel_downsample: leaf too small for the coordinates");
    if (g.err == kVoxErrCells)
        return fail(KDNN_EINVAL, "voxel_downsample: the voxel grid over the cloud's extent "
                                 "needs 2^32 cells or more (leaf too small)");
    const uint32_t m = g.n_finite == 0 ? 0u : g.nvox;
    *m_out = int64_t(m);
    return KDNN_OK;
    KDNN_GUARD_END
}

size_t icp_batch_workspace_bytes(int32_t B, const int64_t *n)
{
    if (B < 1 || !n) return 0;
    for (int32_t p = 0; p < B; ++p)
        if (n[p] < 1) return 0;
    return icp_batch_ws_bytes(B, n);
}

kdnn_status icp_align_batch(int32_t B, const kdnn_tree *const *trees, const float *const *src_dev,
                            const int64_t *n, const double *R0_host, const double *t0_host,
                            int32_t max_iter, double eps, double *R_out, double *t_out,
                            double *E_hist, int32_t *iters_done, kdnn_status *status_out,
                            uint32_t flags, const kdnn_icp_reject *reject, void *ws_dev,
                            size_t ws_bytes, hipStream_t stream)
{
    KDNN_GUARD_BEGIN
    if (B < 1 || !trees || !src_dev || !n || !R_out || !t_out)
        return fail(KDNN_EINVAL, "icp_align_batch: B < 1 or a null array");
    if (max_iter < 0) return fail(KDNN_EINVAL, "icp_align_batch: max_iter < 0");
    if (!(eps >= 0.0)) return fail(KDNN_EINVAL, "icp_align_batch: eps must be >= 0");
    if (flags & ~(KDNN_ICP_NO_SORT | KDNN_ICP_HOST_LOOP | KDNN_ICP_DEVICE_LOOP))
        return fail(KDNN_EINVAL, "icp_align_batch: only KDNN_ICP_NO_SORT, KDNN_ICP_HOST_LOOP and "
                                 "KDNN_ICP_DEVICE_LOOP are accepted (pairs are traversed in their "
                                 "given order, one lane each)");
    if ((flags & KDNN_ICP_HOST_LOOP) && (flags & KDNN_ICP_DEVICE_LOOP))
        return fail(KDNN_EINVAL,
                    "icp_align_batch: KDNN_ICP_HOST_LOOP and KDNN_ICP_DEVICE_LOOP together");
    if ((flags & KDNN_ICP_DEVICE_LOOP) && max_iter > kLoopMaxIter)
        return fail(KDNN_EINVAL, "icp_align_batch: KDNN_ICP_DEVICE_LOOP records at most " +
                                     std::to_string(kLoopMaxIter) + " iterations");
    kdnn_status st = check_reject(reject, "icp_align_batch");
    if (st != KDNN_OK) return st;
    if (reject && reject->reject_k > 0.0)
        return fail(KDNN_EINVAL, "icp_align_batch: residual rejection is not available in the "
                                 "batched call (max_dist is)");
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "icp_align_batch: hipGetDevice");
    for (int32_t p = 0; p < B; ++p) {
        if (!trees[p]) return fail(KDNN_EINVAL, "icp_align_batch: null tree");
        if (trees[p]->device != dev)
            return fail(KDNN_EINVAL, "icp_align_batch: a tree lives on another device");
        if (n[p] < 1) return fail(KDNN_EINVAL, "icp_align_batch: n must be >= 1");
        if ((st = check_points(src_dev[p], n[p], "icp_align_batch: src")) != KDNN_OK) return st;
    }
    if ((st = check_ws(ws_dev, ws_bytes, icp_batch_ws_bytes(B, n))) != KDNN_OK) return st;

    std::vector<double> R(size_t(9) * B), t(size_t(3) * B);
    for (int32_t p = 0; p < B; ++p) {
        std::memcpy(&R[9 * size_t(p)], R0_host ? R0_host + 9 * size_t(p) : kI, 9 * sizeof(double));
        std::memcpy(&t[3 * size_t(p)], t0_host ? t0_host + 3 * size_t(p) : kZ, 3 * sizeof(double));
        if (iters_done) iters_done[p] = 0;
        if (status_out) status_out[p] = KDNN_OK;
    }
    auto copy_out = [&]() {
        std::memcpy(R_out, R.data(), R.size() * sizeof(double));
        std::memcpy(t_out, t.data(), t.size() * sizeof(double));
    };
    copy_out();
    if (max_iter == 0) return KDNN_OK;

    // one partial column per work-group of every pair
    std::vector<int32_t> part(B);
    int32_t total = 0;
    for (int32_t p = 0; p < B; ++p) {
        part[p] = total;
        total += batch_groups(n[p]);
    }
    if (!(flags & KDNN_ICP_HOST_LOOP) && max_iter <= kLoopMaxIter)
        return batch_on_device(B, trees, src_dev, n, R, t, max_iter, eps, R_out, t_out, E_hist,
                               iters_done, status_out, reject, ws_dev, total, part, stream);

    // Each pair's reduction writes its 17 sums into its tree's pinned slot,
    // then the launch's sequence number into the slot's completion word, which
    // the host polls (the slots belong to the trees: nothing is allocated).
    // The users of those slots are serialised by the trees' locks, taken in
    // address order.  When one tree serves several pairs of the batch, its
    // single slot cannot: then every pair's sums go to its loop-state slot of
    // the workspace (unused by this path) and come back with one copy per
    // iteration.  On every return the stream is drained first (the Staging
    // destructor runs before the locks are released), since a launch of the
    // current iteration may still be writing.
    std::vector<kdnn_tree *> uniq;
    for (int32_t p = 0; p < B; ++p) uniq.push_back(const_cast<kdnn_tree *>(trees[p]));
    std::sort(uniq.begin(), uniq.end());
    uniq.erase(std::unique(uniq.begin(), uniq.end()), uniq.end());
    const bool shared_tree = int32_t(uniq.size()) != B;
    std::vector<std::unique_lock<std::mutex>> locks;
    for (kdnn_tree *u : uniq) locks.emplace_back(u->icp_mu);
    uint64_t seq0 = 0;
    for (kdnn_tree *u : uniq) seq0 = u->seq > seq0 ? u->seq : seq0;
    const size_t sb = (sizeof(IcpLoopState) + 255) & ~size_t(255);
    static_assert(sizeof(IcpLoopState) >= KDNN_SUMS_DOUBLES * sizeof(double),
                  "a loop-state slot holds one pair's sums");
    struct Staging {
        std::vector<double> h;
        hipStream_t s = nullptr;
        ~Staging() { (void)hipStreamSynchronize(s); }
    } pin;
    pin.s = stream;
    if (shared_tree) pin.h.assign(size_t(B) * (sb / sizeof(double)), 0.0);
    auto dev_sums = [&](int32_t p) {
        return shared_tree ? reinterpret_cast<double *>(batch_loop_state(ws_dev, total, p))
                           : trees[p]->d_pinned;
    };
    auto host_sums = [&](int32_t p) -> const double * {
        return shared_tree ? pin.h.data() + size_t(p) * (sb / sizeof(double)) : trees[p]->h_pinned;
    };

    const float bound2 = reject ? bound_of(reject->max_dist) : INFINITY;
    std::vector<char> done(B, 0);
    std::vector<double> prev_mse(B, 0.0);
    std::vector<int> small_steps(B, 0);
    std::vector<BatchJob> jobs;
    bool any_failed = false;
    for (int32_t k = 0; k < max_iter; ++k) {
        std::vector<int32_t> active;
        for (int32_t p = 0; p < B; ++p)
            if (!done[p]) active.push_back(p);
        if (active.empty()) break;
        // one sequence number for every tree of the batch (all of them locked)
        const uint64_t seq = seq0 + uint64_t(k) + 1;
        for (kdnn_tree *u : uniq) u->seq = seq;
        for (size_t c0 = 0; c0 < active.size(); c0 += size_t(batch_max_pairs())) {
            jobs.clear();
            for (size_t c = c0; c < active.size() && c < c0 + size_t(batch_max_pairs()); ++c) {
                const int32_t p = active[c];
                uint64_t *done_word =
                    shared_tree ? nullptr
                                : reinterpret_cast<uint64_t *>(trees[p]->d_pinned + kDoneWord);
                BatchJob J{&trees[p]->dev, src_dev[p], n[p], &R[9 * size_t(p)],
                           &t[3 * size_t(p)], part[p], dev_sums(p), done_word};
                J.hint = batch_hint(ws_dev, total, B, n, p);
                J.hint_in = k > 0;
                jobs.push_back(J);
            }
            e = launch_icp_batch(int32_t(jobs.size()), jobs.data(), bound2, ws_dev, total, stream,
                                 seq);
            if (e != hipSuccess) return hip_fail(e, "icp_align_batch: launch");
        }
        if (shared_tree) {
            // every pair's slot, active or not (one copy), then wait
            if ((e = hipMemcpyAsync(pin.h.data(), dev_sums(0), size_t(B) * sb,
                                    hipMemcpyDeviceToHost, stream)) != hipSuccess ||
                (e = hipStreamSynchronize(stream)) != hipSuccess)
                return hip_fail(e, "icp_align_batch: read back the sums");
        } else {
            for (const int32_t p : active)
                if ((e = wait_word(reinterpret_cast<const volatile uint64_t *>(
                                       trees[p]->h_pinned + kDoneWord),
                                   seq, stream)) != hipSuccess)
                    return hip_fail(e, "icp_align_batch: wait for the sums");
        }
        for (const int32_t p : active) {
            kdnn_icp_sums sums;
            to_sums(host_sums(p), trees[p]->dev.center, &sums);
            if (E_hist) E_hist[size_t(p) * max_iter + k] = sums.sum_d2;
            std::string err;
            double Rn[9], tn[3];
            const kdnn_status ps = procrustes_from_sums(sums, Rn, tn, err);
            if (ps != KDNN_OK) {
                if (status_out) status_out[p] = ps;
                done[p] = 1;
                any_failed = true;
                continue;
            }
            std::memcpy(&R[9 * size_t(p)], Rn, sizeof Rn);
            std::memcpy(&t[3 * size_t(p)], tn, sizeof tn);
            if (iters_done) iters_done[p] = k + 1;
            const double mse = sums.sum_d2 / double(sums.n);
            if (eps > 0.0 && k > 0) {
                small_steps[p] = std::fabs(mse - prev_mse[p]) < eps ? small_steps[p] + 1 : 0;
                if (small_steps[p] >= 2) done[p] = 1;
            }
            prev_mse[p] = mse;
        }
    }
    copy_out();
    // the loop waited for the sums only; leave the stream idle (and the pinned
    // buffer unused by the device) before returning
    if ((e = hipStreamSynchronize(stream)) != hipSuccess)
        return hip_fail(e, "icp_align_batch: synchronize");
    if (any_failed) return fail(KDNN_EDEGENERATE, "icp_align_batch: a pair degenerated (status_out)");
    return KDNN_OK;
    KDNN_GUARD_END
}

}  // extern "C"
