// Internal declarations shared by the host code and the HIP kernels of libkdnn.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <mutex>
#include <string>
#include <vector>

#include "kdnn.h"

namespace kdnn {

// ---------------------------------------------------------------- tree layout
//
// Nodes: a complete binary tree in heap order, 1-based (root = 1, children of
// i are 2i and 2i+1, so the node index spells the path from the root).  Slot
// 0 is unused so that every sibling pair shares one aligned 64-byte line.
// Each node is 32 bytes = two float4:
//   f4[2i]   = (lo.x, lo.y, lo.z, hi.x)
//   f4[2i+1] = (hi.y, hi.z, w6, w7)
// lo/hi: tight bounding box of the node's points (empty node: +inf / -inf).
// Internal node (i < 2^D): w6 = split value, w7 = axis as uint32.
// Leaf (i >= 2^D): w6 = first point slot (int32 bits), w7 = count (int32 bits).
//
// Points: one float4 per point in leaf order: (x, y, z, original index bits),
// so a leaf is one contiguous run read with 16-byte loads.
constexpr int kNodeWords = 8;
constexpr int kMaxDepth = 28;
// Per-leaf plane record: for the leaf's deepest kPathLevels ancestors, in one
// 64-byte record (16 words): word 0 their split axes, two bits each, deepest
// first; words 1 .. kPathLevels the near face, along that axis, of the box of
// each one's child off the leaf's path (at or beyond the split).
constexpr int kPathLevels = 14;
constexpr int kPathWords = 16;
// Morton prefix (of the 30-bit code) that orders the queries: nn_query pays
// the sort on every call and takes one 8-bit radix pass; the ICP entry points
// sort once per registration for 30 searches and take two.
constexpr int kKeyBitsQuery = 8;
constexpr int kKeyBitsIcp = 16;
constexpr int kMaxLeafSize = 1024;

struct HostTree {
    int32_t depth = 0;
    int32_t leaf_size = 0;
    int64_t n = 0;
    std::vector<float> nodes;   // (2^(D+1)) * 8 words
    std::vector<float> points;  // n * 4 words
    float bbox_min[3] = {0, 0, 0};
    float bbox_max[3] = {0, 0, 0};
    double center[3] = {0, 0, 0};
    int32_t min_leaf = 0, max_leaf = 0;
};

// Validate params and compute D and the node slot count (no allocation).
kdnn_status tree_layout(int64_t n, const kdnn_build_params *p, int32_t *depth, int64_t *slots,
                        std::string &err);
// Full host build into HostTree (validates finiteness).
kdnn_status build_host_tree(const float *xyz, int64_t n, const kdnn_build_params *p, HostTree &out,
                            std::string &err);

// Roofline micro-benchmarks (roofline.hip); each times one launch with events
// on s.  false on a HIP error.
bool run_gather_bench(const void *buf, int64_t n_records, int32_t words, int64_t lanes,
                      int32_t rounds, uint32_t seed, uint32_t *sink, float *ms, hipStream_t s);
bool run_chase_bench(const uint32_t *next, int64_t n_records, int32_t waves, int32_t steps,
                     uint32_t *sink, float *ms, hipStream_t s);

// Rigid solve from the 17 correspondence sums.
kdnn_status procrustes_from_sums(const kdnn_icp_sums &s, double R[9], double t[3], std::string &err);
// Centroids, H, E and E / n from the 17 correspondence sums (zero for n <= 0).
void moments_of_sums(const kdnn_icp_sums &s, kdnn_icp_moments &m);
// Message of a rigid_solve.hpp status code.
const char *rigid_status_text(int32_t st);

// ---------------------------------------------------------------- device side

struct DeviceTree {
    const void *nodes = nullptr;   // float4 array, 2 per node slot
    const void *boxes = nullptr;   // 6 floats per node slot: lo.xyz, hi.xyz (pairs 48 B)
    const void *points = nullptr;  // float4 array, 1 per point
    const void *slot_of = nullptr; // n int32: leaf-order slot of each original index
    const void *paths = nullptr;   // kPathWords words per leaf: its plane record
    uint32_t first_leaf = 1;       // 2^D
    int32_t depth = 0;             // D
    int32_t max_leaf = 0;          // points in the largest leaf
    int64_t n = 0;                 // target points
    float box_lo[3] = {0, 0, 0};   // target bbox (Morton normalisation)
    float box_inv[3] = {0, 0, 0};  // 1 / extent per axis (0 for a flat axis)
    double center[3] = {0, 0, 0};
};

// Workspace carving (all offsets 256-byte aligned).
struct SortWorkspace {
    uint32_t *keys_a, *keys_b;
    int32_t *vals_a, *vals_b;
    uint32_t *hist;    // [256][ntiles] tile counts per digit
    uint32_t *totals;  // [256] per-digit totals
    int32_t ntiles;
};
size_t sort_workspace_bytes(int64_t m);
SortWorkspace carve_sort_workspace(void *ws, int64_t m);

struct QueryWorkspace {
    SortWorkspace sort;
    void *twopass;  // two-pass list + per-group counts
};
size_t query_ws_bytes(int64_t m);
QueryWorkspace carve_query_workspace(void *ws, int64_t m);

// ICP iterations kept on the device (icp_align's default path): each
// iteration is the fused kernel followed by a one-group step kernel that sums
// the partials, solves the rigid transform (rigid_solve.hpp), applies the
// convergence rule and leaves the next transform here for the next fused
// kernel, so the host enqueues all iterations and waits once.
struct IcpLoopState {  // device memory (ICP workspace)
    double rt[12];     // (R row-major, t) of the next iteration
    double rt1[12];    // residual rejection: the iteration's first solve
    double prev_mse;   // mean squared distance of the last iteration
    double mse;        // residual rejection: this iteration's (first pass)
    int32_t small;     // consecutive iterations whose MSE changed by < eps
    uint32_t stop;     // nonzero: converged or failed, later iterations do nothing
};
constexpr int32_t kLoopMaxIter = 512;  // iterations the output record holds
struct IcpLoopOut {    // device memory, written by the step kernels (copied to the host at the end)
    double rt[12];     // last solved transform (the initial one until a solve)
    int64_t iters;     // iterations completed
    int64_t status;    // rigid_solve status of the failed iteration, 0 if none
    int64_t fail_iter; // that iteration, -1 if none
    int64_t fail_phase;// 1: the solve after residual rejection failed
    int64_t stopped;   // nonzero once state.stop is set
    double E[kLoopMaxIter];
    double rt_hist[kLoopMaxIter][12];  // transform used by each iteration
};
struct IcpLoop {
    IcpLoopState *state;  // device
    IcpLoopOut *out;      // device record
    int32_t iter;         // iteration index of this launch
    double eps;
    // 0: the iteration's only solve; with residual rejection, 1: the first
    // solve (into state.rt1, iteration not yet done), 2: the solve of the
    // kept pairs (ends the iteration)
    int32_t mode;
};

struct IcpWorkspace {
    SortWorkspace sort;
    double *partials;   // KDNN_SUMS_DOUBLES * max_blocks
    double *partials2;  // KDNN_SUMS_DOUBLES * pass-2 blocks
    uint64_t *pkey;     // [n] pass-1 best key per traversal slot
    uint32_t *pslot;    // [n]
    void *twopass;      // two-pass list + per-group counts
    int32_t *mslot;     // [n] original index of each source point's match (rejection)
    float *md2;         // [n] its squared distance
    double *stat;       // residual statistics of the rejection step
    double *sums;       // KDNN_SUMS_DOUBLES
    IcpLoopState *loop; // device-side ICP loop state
    uint32_t *hint;     // [n] heap index of the leaf that held each source point's
                        // last match (0: none), written by the fused kernel
    int32_t max_blocks;
};
size_t icp_ws_bytes(int64_t n);
IcpWorkspace carve_icp_workspace(void *ws, int64_t n);

// icp_align_noalloc's device scratch (noalloc.hip): the address of the
// current device's copy (found on the first call per device; `device` must
// be current) and the lock that keeps calls on that device from overlapping.
hipError_t noalloc_scratch(int device, void **ptr, std::mutex **call_mu);

// Kernel launchers (return the hipError_t of the launch).
// Morton-order the points moved by (R, t) (R == nullptr: not moved) by the
// top key_bits (8 or 16) bits of their code: on return *perm points at the
// int32 permutation (traversal slot -> point).
hipError_t launch_morton_order(const DeviceTree &t, const float *pts, int64_t m, const float *R12,
                               int key_bits, const SortWorkspace &ws, const int32_t **perm,
                               hipStream_t s);
// Same, for the ICP entry points (sort buffers carved from the ICP workspace).
hipError_t launch_icp_order(const DeviceTree &t, const float *pts, int64_t m, const float *R12,
                            const IcpWorkspace &ws, const int32_t **perm, hipStream_t s);
// Search schedule decoded from the KDNN_LANES / KDNN_BUDGET / KDNN_TOP_LDS
// flag fields (see kdnn.h).
struct Schedule {
    int lanes = 0;        // 0 = automatic, else single pass with this many lanes
    uint32_t budget = 0;  // 0 = default two-pass budget / automatic choice
    bool top_lds = false;
};
// timing: null, or two events the search kernel(s) stamp with their start and end.
hipError_t launch_nn(const DeviceTree &t, const float *q, int64_t m, const int32_t *perm,
                     int32_t *idx, float *d2, uint32_t *cnt_nodes, uint32_t *cnt_pts, bool stats,
                     const Schedule &sc, float bound2, void *twopass, hipStream_t s,
                     const hipEvent_t *timing = nullptr);
hipError_t launch_transform(const float *in, float *out, int64_t n, const double *R,
                            const double *t, hipStream_t s);
// Correspondence search + per-work-group partials, then the one-group
// reduction into sums_out.  timing: null, or two events the search
// kernel(s) stamp with their start and end.  done: null, or a word the
// reduction sets to seq (system-scope release) once the sums are written.
// loop: null, or one iteration of a device-side loop (one lane per query
// schedule only): the search takes its transform from loop->state (R, tv
// unused) and the step kernel replaces the reduction (sums_out unused).
// hint_mode (one lane per query schedule; other schedules ignore it): 0
// none, 1 record each source point's match leaf in ws.hint, 2 also start each
// search from the leaf recorded there by the previous launch over the same
// source (an ICP iteration after the first).
hipError_t launch_icp_fused(const DeviceTree &t, const float *src, int64_t n, const int32_t *perm,
                            const double *R, const double *tv, const IcpWorkspace &ws,
                            double *sums_out, int32_t *idx, float *d2, const Schedule &sc,
                            float bound2, bool keep_matches, hipStream_t s,
                            const hipEvent_t *timing = nullptr, uint64_t *done = nullptr,
                            uint64_t seq = 0, const IcpLoop *loop = nullptr,
                            int hint_mode = 0);
// Start a device-side ICP loop: state <- (R0, t0), counters cleared; the
// output record's transform <- (R0, t0), no iterations, no failure.
hipError_t launch_icp_loop_init(IcpLoopState *state, IcpLoopOut *out, const double *R0,
                                const double *t0, hipStream_t s);
// Voxel-grid filter (voxel.hip).
// The key grid of one call, computed on the device from the cloud's bounding
// box: voxel v = floor(p / leaf) - vmin, key = vx + dims[0] (vy + dims[1] vz);
// non-finite points take `sentinel` (the dims product, one past the last key).
struct VoxGrid {
    int64_t vmin[3];
    uint32_t dims[3];
    uint32_t sentinel;
    uint32_t n_finite;  // finite points
    int32_t passes;     // radix passes the keys need; 0: nothing to sort
    int32_t err;        // kVoxOk, kVoxErrRange or kVoxErrCells
    uint32_t nvox;      // voxels: the sum of the segment heads
    uint32_t nbig;      // voxels summed by a whole wave (their list: in vals_a)
};
constexpr int32_t kVoxOk = 0;
constexpr int32_t kVoxErrRange = 1;  // |floor(p / leaf)| >= 4e18 for a bounding-box corner
constexpr int32_t kVoxErrCells = 2;  // the grid over the extent needs 2^32 cells or more
struct VoxelWorkspace {
    uint32_t *keys_a, *keys_b;
    int32_t *vals_a, *vals_b;
    uint32_t *hist, *totals;  // [digits][tiles] tile counts, [digits] digit totals
    uint32_t *tile_heads;     // [tiles]
    int32_t *starts;          // [n] first sorted position of each voxel
    uint32_t *bbox_part;      // [7][blocks]: min xyz, max xyz (fp32 bits), finite count
    VoxGrid *grid;
    float4 *sorted;           // [n] the points' coordinates (x, y, z, 0) in sorted order
};
size_t voxel_ws_bytes(int64_t n);
VoxelWorkspace carve_voxel_workspace(void *ws, int64_t n);
// Every launch of the filter, none waiting on the host.  When the stream
// gets past them, *w.grid holds the grid, its error code and the voxel count,
// and out / counts their first nvox rows (none when err != kVoxOk).
hipError_t launch_voxel_filter(const float *xyz, int64_t n, double leaf, const VoxelWorkspace &w,
                               float *out, int32_t *counts, hipStream_t s);

// Batched correspondence steps: up to batch_max_pairs() (tree, source) pairs
// per launch, one pair per group of XCDs.  ws: icp_batch_ws_bytes layout
// (partials of `total` work-group columns).
struct BatchJob {
    const DeviceTree *tree;
    const float *src;
    int64_t n;
    const double *R;  // [9]
    const double *t;  // [3]
    int32_t part;     // first partial column
    double *sums;     // [KDNN_SUMS_DOUBLES] out (device-visible)
    uint64_t *done;   // null, or a device-visible word the reduction sets to seq
    IcpLoopState *st = nullptr;  // device loop: the pair's state (R, t unused), else null
    IcpLoopOut *out = nullptr;   // device loop: the pair's record
    uint32_t *hint = nullptr;    // [n] the pair's match leaves (warm start), or null
    bool hint_in = false;        // start the searches from them (an iteration after the first)
};
int batch_max_pairs();
int32_t batch_groups(int64_t n);  // work-groups (partial columns) of an n-point pair
// Workspace: the partial columns, then B loop states, then B loop records,
// then each pair's match leaves (n[p] words, 256-byte aligned).
size_t icp_batch_ws_bytes(int32_t B, const int64_t *n);
uint32_t *batch_hint(void *ws, int32_t total, int32_t B, const int64_t *n, int32_t p);
size_t batch_loop_bytes(int32_t B);
IcpLoopState *batch_loop_state(void *ws, int32_t total, int32_t p);
IcpLoopOut *batch_loop_out(void *ws, int32_t total, int32_t B, int32_t p);
// Each pair's record header from its state (states written by the host first).
hipError_t launch_batch_loop_init(int32_t B, void *ws, int32_t total, hipStream_t s);
// iter / eps: the device loop's (jobs with st set: the reduction also solves).
hipError_t launch_icp_batch(int32_t B, const BatchJob *jobs, float bound2, void *ws, int32_t total,
                            hipStream_t s, uint64_t seq = 0, int32_t iter = 0, double eps = 0.0);

// Residual rejection of the pairs the last fused launch stored (keep_matches):
// sums of the pairs with r^2 <= kk * mean r^2 under (R, t).
// Replay ceiling of a search launch (kdnn_replay_bench): workspace bytes and
// the launch (trace, pack, `reps` timed replays into ms_out[0 .. reps)).
// icp: the fused ICP kernel's launch shape, else nn_query's.  q_prev: null,
// or the previous ICP iteration's queries (each search then starts at the
// leaf of that query's nearest neighbour, as the ICP loop's searches do).
using ReplayTally = kdnn_replay_info;
size_t replay_ws_bytes(const DeviceTree &t, int64_t m, bool icp);
hipError_t launch_replay(const DeviceTree &t, const float *q, int64_t m, const int32_t *perm,
                         bool icp, const float *q_prev, void *ws, int32_t reps, float *ms_out,
                         ReplayTally *tally, hipStream_t s);

hipError_t launch_icp_reject(const DeviceTree &t, const float *src, int64_t n, const double *R,
                             const double *tv, double kk, const IcpWorkspace &ws, double *sums_out,
                             double *stat_out, uint8_t *kept, hipStream_t s,
                             uint64_t *done = nullptr, uint64_t seq = 0,
                             const IcpLoop *loop = nullptr);

}  // namespace kdnn

// The opaque handle of the C ABI.
struct kdnn_tree {
    int device = 0;
    kdnn::DeviceTree dev;
    void *d_nodes = nullptr;
    void *d_boxes = nullptr;
    void *d_points = nullptr;
    void *d_slot_of = nullptr;
    void *d_paths = nullptr;
    kdnn_tree_info info{};
    double *h_pinned = nullptr;  // host readback slot for the ICP sums (32 doubles;
                                 // the last word: completion sequence number)
    uint64_t seq = 0;            // last sequence number handed to the reduction
    double *d_pinned = nullptr;  // the same slot as the device addresses it
    kdnn::IcpLoopOut *d_loop = nullptr;  // device-side ICP loop record (device memory)
    kdnn::IcpLoopOut *h_loop = nullptr;  // its pinned copy, read after a registration
    bool auto_sort = false;      // nn_query orders queries unless told otherwise
    bool auto_sort_icp = false;  // the ICP entry points order the source unless told otherwise
    std::mutex icp_mu;           // serialises users of h_pinned
};
