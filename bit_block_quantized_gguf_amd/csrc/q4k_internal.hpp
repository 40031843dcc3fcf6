// q4k_internal.hpp — host-side declarations shared by the library's sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q4k.h"

namespace q4k {

// ---------------------------------------------------------------- errors
int fail(int code, const char *fmt, ...);
void clear_error();
int hip_fail(hipError_t e, const char *what);

#define Q4K_HIP(call)                                                   \
    do {                                                                \
        hipError_t e_ = (call);                                         \
        if (e_ != hipSuccess) return ::q4k::hip_fail(e_, #call);        \
    } while (0)

// ---------------------------------------------------------------- workspace
// Split-K partial sums and arrival counters.  They live in the caller's
// workspace (a stack plan allocates its own at creation).  Counters start at
// zero and every kernel that uses one returns it to zero, so no clearing work
// is ever enqueued on the hot path (and none is recorded into a graph).
struct Workspace {
    float *partials = nullptr;
    size_t partial_floats = 0;
    unsigned *counters = nullptr;
    size_t n_counters = 0;
};

// Every workspace layout starts with the same counter region of
// kMaxCounters arrival counters (a GEMV grid has at most that many
// workgroups), and no call writes data there: a workspace shared by calls of
// different kinds keeps its counters at zero.  The call's own data follow.
constexpr size_t kMaxCounters = 16384;
constexpr size_t kCounterBytes = kMaxCounters * sizeof(unsigned);
// Bytes of the counter region plus `partial_floats` floats; carve() splits a
// base pointer into the two.
size_t region_bytes(size_t partial_floats);
Workspace carve(void *base, size_t partial_floats);

// Allocate a zeroed workspace owned by a stack plan (plan creation only).
int alloc_workspace(size_t partial_floats, size_t n_counters, Workspace *out);
void free_workspace(Workspace *ws);

// ---------------------------------------------------------------- GEMV
enum GemvEpilogue : int {
    EPI_PLAIN = 0,   // y = W x
    EPI_SCALE = 1,   // y = (W x) / rms(x)
    EPI_RESID = 2,   // y = resid + (W x) / rms(x)
    EPI_SWIGLU = 3,  // g = (Wg x)/rms(x), v = (Wu x)/rms(x), y = silu(g) * v
};

struct GemvParams {
    const uint8_t *w0;      // first matrix (M x K super-blocks)
    const uint8_t *w1;      // second matrix (EPI_SWIGLU), same shape
    const float *x;         // [nv][K], vector stride x_stride floats
    int64_t x_stride;
    float *y;               // [nv][M], vector stride y_stride floats
    int64_t y_stride;
    float *y_g;             // EPI_SWIGLU: scaled gate output [M] (null: not written)
    float *y_v;             // EPI_SWIGLU: scaled up output [M] (null: not written)
    int32_t M, K, nb;       // nb = K / 256
    int64_t row_bytes;      // nb * 144
    int32_t ks;             // unused by the GEMV (the launch carries the grid)
    float *ws;              // partials of tiles split between workgroups [groups][2][nv][64]
    unsigned *cnt;          // per-tile arrival counters of split tiles (zero between launches)
    const float *in_sq;     // EPI_SCALE/RESID/SWIGLU: per-32-element sums of squares of x
                            // (null: no 1/rms scaling)
    int32_t in_sq_n;        // number of partials to add (ceil(K/32))
    int32_t in_len;         // divisor of the mean (K)
    const float *resid;     // EPI_RESID: residual [M]
    float *out_sq;          // EPI != PLAIN: per-32-row sums of squares of y (null: not written)
    float eps;
};

struct GemvLaunch {
    int wk;  // waves per workgroup (= super-blocks per unit), fixed at 4
    int ks;  // workgroups in the grid (each takes a contiguous range of units)
};

// Launch shape for a GEMV: as many workgroups as fit on the current device
// (from the kernel's occupancy), capped by the number of work units.
GemvLaunch choose_gemv_launch(int64_t M, int64_t K, int nv, int nmat, int epi = EPI_PLAIN);

// Workspace needs of a launch: partial sums of the cut tiles (two slots of
// nv x 64 floats per workgroup) and one arrival counter per workgroup (the
// counter of a cut tile is that of the workgroup owning its first unit: a
// workgroup owns the first unit of at most one cut tile).
size_t gemv_partial_floats(const GemvLaunch &L, int nv);
size_t gemv_counters(const GemvLaunch &L);

// Enqueue one GEMV kernel.  nv in {1,2,4,8,16} for EPI_PLAIN; nv = 1 otherwise.
int launch_gemv(const GemvParams &p, int nv, int nmat, int epi, const GemvLaunch &L,
                hipStream_t stream);

// Q8_0 GEMV (one vector, plain output): launch shape and launch.  p.nb is the
// number of 32-weight blocks per row (K / 32) and p.row_bytes = nb * 34.
GemvLaunch choose_gemv_q8_launch(int64_t M, int64_t K);
int launch_gemv_q8(const GemvParams &p, const GemvLaunch &L, hipStream_t stream);

// Q6_K GEMV (one vector, plain output): launch shape and launch.  p.nb is the
// number of 256-weight blocks per row (a multiple of 4), p.row_bytes nb * 210.
GemvLaunch choose_gemv_q6_launch(int64_t M, int64_t K);
int launch_gemv_q6(const GemvParams &p, const GemvLaunch &L, hipStream_t stream);

// q4k_gemv with its split-tile scratch in a fixed per-device array instead of
// a caller workspace (q4k_noalloc.hip).
int gemv_noalloc(const void *w, const float *x, float *y, int64_t M, int64_t K,
                 hipStream_t stream);

// Arrival counters per node of the persistent decode kernel: workgroup g
// counts into counter g mod kStackSyncLanes, so the arrivals at a node
// boundary spread over that many addresses; the node's wait reads them all.
constexpr int kStackSyncLanes = 16;

// Persistent decode kernel (q4k_gemv.hip): grid size (co-resident
// workgroups, at most two per CU), node descriptor size, filling one node
// descriptor (host memory), and the cooperative launch over n_nodes nodes.
int stack_groups(int *G);
size_t stack_node_bytes();
int fill_stack_node(void *dst, const GemvParams &p, int nmat, int epi, int G);
int launch_stack_kernel(const void *nodes, int n_nodes, unsigned *done, unsigned epoch,
                        unsigned *err, int spin_limit, int G, hipStream_t stream);

// Per-32-element sums of squares of v[0..n) (used to seed the stack).
int launch_sumsq(const float *v, int64_t n, float *out, hipStream_t stream);

// xg = x * (1 + w) elementwise (skipped when w is null) and the per-32-element
// sums of squares of x (the RMS of the un-gained input).
int launch_norm_gain(const float *x, const float *w, int64_t n, float *xg, float *sq,
                     hipStream_t stream);

// Tuning override for benchmarks: workgroup count (0 = occupancy-based).
void set_gemv_override(int groups);

// ---------------------------------------------------------------- token mixers
struct GdnShape {
    int Hk, Hv;   // key heads, value heads (head dimension 128 for both)
    float eps;
};
struct AttnShape {
    int Hq, Hkv, R;  // query heads, key/value heads (head dimension 256), rotary dims
    float theta, eps;
};
// scratch: gdn_scratch_floats(Hk, Hv) floats (the heads' outputs before
// their norm); cnt: Hv + Hk arrival counters (value heads, then key heads),
// zero before the call and after it.  out_sq (may be null): per-32-element
// sums of squares of out.
size_t gdn_scratch_floats(int Hk, int Hv);
int launch_gdn_step(const GdnShape &s, const float *u, const float *conv_w, const float *a_log,
                    const float *dt_bias, const float *norm_w, float *conv_state, float *S,
                    float *out, float *out_sq, float *scratch, unsigned *cnt,
                    hipStream_t stream);
// pos_dev, when not null, holds the position (read on the device); else pos.
// Attention step scratch: the split-KV partials
// (floats; depends on the cache capacity through the chunk count).
size_t attn_scratch_floats(int Hq, int Hkv, int64_t cap);
// out_sq (may be null): per-32-element sums of squares of out.
int launch_attn_step(const AttnShape &s, const float *u, const float *q_norm_w,
                     const float *k_norm_w, float *k_cache, float *v_cache, int64_t cap,
                     int64_t pos, const int64_t *pos_dev, float *out, float *out_sq,
                     float *scratch, hipStream_t stream);

// ---------------------------------------------------------------- dequant
int launch_dequant(const uint8_t *w, float *out, int64_t M, int64_t K, hipStream_t stream);

// ---------------------------------------------------------------- GEMM
struct GemmLaunch {
    int ks;  // workgroups of the stream-K grid
    int r;   // 32-token groups per tile (tile = 256 W rows x 32r tokens)
};
GemmLaunch choose_gemm_launch(int64_t M, int64_t K, int64_t P);

// Host-side checks of the work partitions (q4k_check_partition): the
// kernels' own range arithmetic run for every workgroup, against the
// workspace a launch reserves and the bounds of its operands.  groups or
// tile_tokens 0: the launch heuristics' choice.
int check_gemv_partition(int64_t M, int64_t K, int nv, int nmat, int groups);
int check_gemv_q8_partition(int64_t M, int64_t K, int groups);
int check_gemv_q6_partition(int64_t M, int64_t K, int groups);
int check_gemm_partition(int64_t M, int64_t K, int64_t P, int tile_tokens, int groups);
// Workspace: split partials (rounded up to 64 floats) followed by the bf16 copy of X.
size_t gemm_partial_floats(const GemmLaunch &L, int64_t M, int64_t P);
size_t gemm_xb_floats(int64_t K, int64_t P);
size_t gemm_counters(int64_t M, int64_t P);
int launch_gemm(const uint8_t *w, const float *X, float *Y, int64_t M, int64_t K, int64_t P,
                const GemmLaunch &L, const Workspace &ws, hipStream_t stream);
void set_gemm_override(int token_groups, int workgroups);

}  // namespace q4k
