// q4k_api.hip — C ABI entry points of libq4k: argument validation, error
// reporting, the split-K workspace cache, and dispatch to the kernels.
#include "q4k_internal.hpp"

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

namespace q4k {

namespace {

thread_local std::string t_error;

std::mutex g_ws_mutex;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;

std::mutex g_dev_mutex;
std::map<int, bool> g_dev_ok;

}  // namespace

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    t_error = buf;
    return code;
}

void clear_error() { t_error.clear(); }

int hip_fail(hipError_t e, const char *what) {
    return fail(Q4K_EHIP, "%s failed: %s", what, hipGetErrorString(e));
}

void free_workspace(Workspace *ws) {
    if (ws->partials) (void)hipFree(ws->partials);
    if (ws->counters) (void)hipFree(ws->counters);
    *ws = Workspace();
}

int alloc_workspace(size_t partial_floats, size_t n_counters, Workspace *out) {
    Workspace ws;
    if (partial_floats) {
        if (hipMalloc(&ws.partials, partial_floats * sizeof(float)) != hipSuccess) {
            (void)hipGetLastError();
            return fail(Q4K_ENOMEM, "workspace: cannot allocate %zu floats", partial_floats);
        }
        ws.partial_floats = partial_floats;
    }
    if (n_counters) {
        if (hipMalloc(&ws.counters, n_counters * sizeof(unsigned)) != hipSuccess) {
            (void)hipGetLastError();
            free_workspace(&ws);
            return fail(Q4K_ENOMEM, "workspace: cannot allocate %zu counters", n_counters);
        }
        ws.n_counters = n_counters;
        hipError_t e = hipMemset(ws.counters, 0, n_counters * sizeof(unsigned));
        if (e == hipSuccess) e = hipDeviceSynchronize();
        if (e != hipSuccess) {
            free_workspace(&ws);
            return hip_fail(e, "hipMemset(workspace counters)");
        }
    }
    *out = ws;
    return Q4K_OK;
}

int stream_workspace(hipStream_t stream, size_t partial_floats, size_t n_counters,
                     Workspace *out) {
    int dev = 0;
    Q4K_HIP(hipGetDevice(&dev));
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    Workspace &ws = g_ws[std::make_pair(dev, stream)];
    if (ws.partial_floats >= partial_floats && ws.n_counters >= n_counters) {
        *out = ws;
        return Q4K_OK;
    }
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    Q4K_HIP(hipStreamIsCapturing(stream, &cap));
    if (cap != hipStreamCaptureStatusNone)
        return fail(Q4K_EUNSUPPORTED,
                    "workspace must grow during graph capture: make one call of this size on "
                    "the stream before capturing");
    // Work already queued on this stream may still use the old buffers.
    Q4K_HIP(hipStreamSynchronize(stream));
    Workspace grown;
    int rc = alloc_workspace(std::max(partial_floats, ws.partial_floats),
                             std::max(n_counters, ws.n_counters), &grown);
    if (rc) return rc;
    free_workspace(&ws);
    ws = grown;
    *out = ws;
    return Q4K_OK;
}

}  // namespace q4k

using namespace q4k;

namespace {

constexpr int64_t kMaxDim = 0x7FFFFFFF;

int check_device() {
    int dev = 0;
    Q4K_HIP(hipGetDevice(&dev));
    std::lock_guard<std::mutex> lock(g_dev_mutex);
    auto it = g_dev_ok.find(dev);
    if (it == g_dev_ok.end()) {
        hipDeviceProp_t prop;
        Q4K_HIP(hipGetDeviceProperties(&prop, dev));
        const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        it = g_dev_ok.emplace(dev, ok).first;
        if (!ok) return fail(Q4K_EUNSUPPORTED, "device %d is %s, this library targets gfx950", dev,
                             prop.gcnArchName);
    }
    return it->second ? Q4K_OK : fail(Q4K_EUNSUPPORTED, "device %d is not gfx950", dev);
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int check_mk(int64_t M, int64_t K) {
    if (M < 0 || K <= 0 || K % 256 != 0)
        return fail(Q4K_ESHAPE, "need M >= 0 and K a positive multiple of 256 (M=%lld K=%lld)",
                    (long long)M, (long long)K);
    if (M > kMaxDim || K > kMaxDim) return fail(Q4K_EUNSUPPORTED, "dimension beyond 2^31-1");
    return Q4K_OK;
}

int check_ptr(const void *p, const char *name) {
    if (!p) return fail(Q4K_EINVAL, "%s is NULL", name);
    if (!aligned16(p)) return fail(Q4K_EALIGN, "%s is not 16-byte aligned", name);
    return Q4K_OK;
}

#define Q4K_TRY(expr)            \
    do {                         \
        int rc_ = (expr);        \
        if (rc_) return rc_;     \
    } while (0)

int gemv_multi(const void *w, const float *X, float *Y, int64_t M, int64_t K, int64_t N,
               hipStream_t stream) {
    // Pick the largest supported vector count at each step (16, 8, 4, 2, 1).
    int64_t done = 0;
    size_t need_partials = 0;
    const size_t need_counters = gemv_counters(M);
    for (int nv = 16; nv >= 1; nv >>= 1) {
        const GemvLaunch L = choose_gemv_launch(M, K, nv, 1);
        need_partials = std::max(need_partials, gemv_partial_floats(L, M, nv, 1));
    }
    Workspace ws;
    Q4K_TRY(stream_workspace(stream, need_partials, need_counters, &ws));
    while (done < N) {
        int nv = 16;
        while (nv > N - done) nv >>= 1;
        GemvParams p = {};
        p.w0 = (const uint8_t *)w;
        p.x = X + done * K;
        p.x_stride = K;
        p.y = Y + done * M;
        p.y_stride = M;
        p.M = (int32_t)M;
        p.K = (int32_t)K;
        p.nb = (int32_t)(K / 256);
        p.row_bytes = (K / 256) * 144;
        const GemvLaunch L = choose_gemv_launch(M, K, nv, 1);
        p.ks = L.ks;
        p.ws = ws.partials;
        p.cnt = ws.counters;
        Q4K_TRY(launch_gemv(p, nv, 1, EPI_PLAIN, L, stream));
        done += nv;
    }
    return Q4K_OK;
}

}  // namespace

extern "C" {

const char *q4k_last_error(void) { return t_error.c_str(); }

int q4k_version(void) { return 10000; }

int q4k_dequant(const void *w, float *out, int64_t M, int64_t K, void *stream) {
    clear_error();
    Q4K_TRY(check_mk(M, K));
    if (M == 0) return Q4K_OK;
    Q4K_TRY(check_ptr(w, "w"));
    Q4K_TRY(check_ptr(out, "out"));
    Q4K_TRY(check_device());
    return launch_dequant((const uint8_t *)w, out, M, K, (hipStream_t)stream);
}

int q4k_gemv(const void *w, const float *x, float *y, int64_t M, int64_t K, void *stream) {
    clear_error();
    Q4K_TRY(check_mk(M, K));
    if (M == 0) return Q4K_OK;
    Q4K_TRY(check_ptr(w, "w"));
    Q4K_TRY(check_ptr(x, "x"));
    Q4K_TRY(check_ptr(y, "y"));
    Q4K_TRY(check_device());
    return gemv_multi(w, x, y, M, K, 1, (hipStream_t)stream);
}

int q4k_gemv_batch(const void *w, const float *X, float *Y, int64_t M, int64_t K, int64_t N,
                   void *stream) {
    clear_error();
    Q4K_TRY(check_mk(M, K));
    if (N < 0) return fail(Q4K_ESHAPE, "N must be >= 0");
    if (N > kMaxDim) return fail(Q4K_EUNSUPPORTED, "N beyond 2^31-1");
    if (M == 0 || N == 0) return Q4K_OK;
    Q4K_TRY(check_ptr(w, "w"));
    Q4K_TRY(check_ptr(X, "X"));
    Q4K_TRY(check_ptr(Y, "Y"));
    Q4K_TRY(check_device());
    return gemv_multi(w, X, Y, M, K, N, (hipStream_t)stream);
}

int q4k_gemm(const void *w, const float *X, float *Y, int64_t M, int64_t K, int64_t P,
             void *stream) {
    clear_error();
    Q4K_TRY(check_mk(M, K));
    if (P < 0) return fail(Q4K_ESHAPE, "P must be >= 0");
    if (P > kMaxDim) return fail(Q4K_EUNSUPPORTED, "P beyond 2^31-1");
    if (M == 0 || P == 0) return Q4K_OK;
    Q4K_TRY(check_ptr(w, "w"));
    Q4K_TRY(check_ptr(X, "X"));
    Q4K_TRY(check_ptr(Y, "Y"));
    Q4K_TRY(check_device());
    const GemmLaunch L = choose_gemm_launch(M, K, P);
    Workspace ws;
    Q4K_TRY(stream_workspace((hipStream_t)stream,
                             gemm_partial_floats(L, M, P) + gemm_xb_floats(K, P),
                             gemm_counters(M, P), &ws));
    return launch_gemm((const uint8_t *)w, X, Y, M, K, P, L, ws, (hipStream_t)stream);
}

int q4k_gemv_q6_k(const void *w, const float *x, float *y, int64_t M, int64_t K, void *stream) {
    clear_error();
    Q4K_TRY(check_mk(M, K));
    if (K % 1024 != 0)
        return fail(Q4K_ESHAPE, "q4k_gemv_q6_k: K must be a multiple of 1024 (K=%lld)", (long long)K);
    if (M == 0) return Q4K_OK;
    Q4K_TRY(check_ptr(w, "w"));
    Q4K_TRY(check_ptr(x, "x"));
    Q4K_TRY(check_ptr(y, "y"));
    Q4K_TRY(check_device());
    const GemvLaunch L = choose_gemv_q6_launch(M, K);
    Workspace ws;
    Q4K_TRY(stream_workspace((hipStream_t)stream, gemv_partial_floats(L, M, 1, 1),
                             gemv_counters(M), &ws));
    GemvParams p = {};
    p.w0 = (const uint8_t *)w;
    p.x = x;
    p.x_stride = K;
    p.y = y;
    p.y_stride = M;
    p.M = (int32_t)M;
    p.K = (int32_t)K;
    p.nb = (int32_t)(K / 256);
    p.row_bytes = (K / 256) * 210;
    p.ks = L.ks;
    p.ws = ws.partials;
    p.cnt = ws.counters;
    return launch_gemv_q6(p, L, (hipStream_t)stream);
}

int q4k_gemv_q8_0(const void *w, const float *x, float *y, int64_t M, int64_t K, void *stream) {
    clear_error();
    Q4K_TRY(check_mk(M, K));
    if (M == 0) return Q4K_OK;
    Q4K_TRY(check_ptr(w, "w"));
    Q4K_TRY(check_ptr(x, "x"));
    Q4K_TRY(check_ptr(y, "y"));
    Q4K_TRY(check_device());
    const GemvLaunch L = choose_gemv_q8_launch(M, K);
    Workspace ws;
    Q4K_TRY(stream_workspace((hipStream_t)stream, gemv_partial_floats(L, M, 1, 1),
                             gemv_counters(M), &ws));
    GemvParams p = {};
    p.w0 = (const uint8_t *)w;
    p.x = x;
    p.x_stride = K;
    p.y = y;
    p.y_stride = M;
    p.M = (int32_t)M;
    p.K = (int32_t)K;
    p.nb = (int32_t)(K / 32);
    p.row_bytes = (K / 32) * 34;
    p.ks = L.ks;
    p.ws = ws.partials;
    p.cnt = ws.counters;
    return launch_gemv_q8(p, L, (hipStream_t)stream);
}

int q4k_mlp(const void *w_gate, const void *w_up, const void *w_down, int64_t hidden,
            int64_t inter, const float *x, const float *norm_w, float eps, const float *resid,
            float *y, float *act, void *stream) {
    clear_error();
    Q4K_TRY(check_mk(inter, hidden));  // gate and up: inter x hidden
    Q4K_TRY(check_mk(hidden, inter));  // down: hidden x inter
    if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(Q4K_EINVAL, "eps must be finite and >= 0");
    Q4K_TRY(check_ptr(w_gate, "w_gate"));
    Q4K_TRY(check_ptr(w_up, "w_up"));
    Q4K_TRY(check_ptr(w_down, "w_down"));
    Q4K_TRY(check_ptr(x, "x"));
    Q4K_TRY(check_ptr(y, "y"));
    if (act) Q4K_TRY(check_ptr(act, "act"));
    Q4K_TRY(check_device());
    const hipStream_t st = (hipStream_t)stream;
    const int epi_down = resid ? EPI_RESID : EPI_PLAIN;
    const GemvLaunch Lg = choose_gemv_launch(inter, hidden, 1, 2, EPI_SWIGLU);
    const GemvLaunch Ld = choose_gemv_launch(hidden, inter, 1, 1, epi_down);
    auto round64 = [](size_t n) { return (n + 63) / 64 * 64; };
    // workspace: [GEMV partials][x * (1 + w)][sums of squares of x][activation]
    const size_t off_xg = round64(std::max(gemv_partial_floats(Lg, inter, 1, 2),
                                           gemv_partial_floats(Ld, hidden, 1, 1)));
    const size_t off_sq = off_xg + round64((size_t)hidden);
    const size_t off_act = off_sq + round64((size_t)((hidden + 31) / 32));
    const size_t total = off_act + (act ? 0 : round64((size_t)inter));
    Workspace ws;
    Q4K_TRY(stream_workspace(st, total, std::max(gemv_counters(inter), gemv_counters(hidden)),
                             &ws));
    float *xg = ws.partials + off_xg, *sq = ws.partials + off_sq;
    float *a = act ? act : ws.partials + off_act;
    Q4K_TRY(launch_norm_gain(x, norm_w, hidden, xg, sq, st));
    // a = silu(W_gate n) * (W_up n), n = x / rms(x) * (1 + w): the gain goes on
    // the input, the 1/rms on the outputs
    GemvParams p = {};
    p.w0 = (const uint8_t *)w_gate;
    p.w1 = (const uint8_t *)w_up;
    p.x = norm_w ? xg : x;
    p.x_stride = hidden;
    p.y = a;
    p.y_stride = inter;
    p.M = (int32_t)inter;
    p.K = (int32_t)hidden;
    p.nb = (int32_t)(hidden / 256);
    p.row_bytes = (hidden / 256) * 144;
    p.ks = Lg.ks;
    p.ws = ws.partials;
    p.cnt = ws.counters;
    p.in_sq = sq;
    p.in_sq_n = (int32_t)((hidden + 31) / 32);
    p.in_len = (int32_t)hidden;
    p.eps = eps;
    Q4K_TRY(launch_gemv(p, 1, 2, EPI_SWIGLU, Lg, st));
    // y = resid + W_down a (the activation is not normalised)
    GemvParams q = {};
    q.w0 = (const uint8_t *)w_down;
    q.x = a;
    q.x_stride = inter;
    q.y = y;
    q.y_stride = hidden;
    q.M = (int32_t)hidden;
    q.K = (int32_t)inter;
    q.nb = (int32_t)(inter / 256);
    q.row_bytes = (inter / 256) * 144;
    q.ks = Ld.ks;
    q.ws = ws.partials;
    q.cnt = ws.counters;
    q.resid = resid;
    return launch_gemv(q, 1, 1, epi_down, Ld, st);
}

void q4k_release_workspaces(void) {
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    if (g_ws.empty()) return;
    (void)hipDeviceSynchronize();
    for (auto &kv : g_ws) free_workspace(&kv.second);
    g_ws.clear();
}

/* Benchmark knobs: force the GEMV workgroup count and the GEMM tile width and
 * workgroup count (0 restores the shape heuristics).  Not thread-safe with
 * respect to concurrent calls; meant for sweeps. */
int q4k_tune_gemv(int32_t waves_per_group, int32_t workgroups) {
    clear_error();
    if (waves_per_group != 0 && waves_per_group != 4)
        return fail(Q4K_EINVAL, "waves_per_group must be 0 or 4");
    if (workgroups < 0 || workgroups > (1 << 20))
        return fail(Q4K_EINVAL, "workgroups must be in 0..2^20");
    set_gemv_override(workgroups);
    return Q4K_OK;
}

int q4k_tune_gemm(int32_t tile_tokens, int32_t workgroups) {
    clear_error();
    if (tile_tokens != 0 && tile_tokens != 32 && tile_tokens != 64 && tile_tokens != 128 &&
        tile_tokens != 256)
        return fail(Q4K_EINVAL, "tile_tokens must be 0, 32, 64, 128 or 256");
    if (workgroups < 0 || workgroups > 4096)
        return fail(Q4K_EINVAL, "workgroups must be in 0..4096");
    set_gemm_override(tile_tokens / 32, workgroups);
    return Q4K_OK;
}

/* Launch configuration the heuristics pick for a shape (for reports). */
int q4k_gemv_config(int64_t M, int64_t K, int64_t N, int32_t *waves_per_group,
                    int32_t *workgroups) {
    clear_error();
    Q4K_TRY(check_mk(M, K));
    if (!waves_per_group || !workgroups) return fail(Q4K_EINVAL, "NULL output");
    int nv = 16;
    while (nv > 1 && nv > N) nv >>= 1;
    const GemvLaunch L = choose_gemv_launch(M, K, nv, 1);
    *waves_per_group = L.wk;
    *workgroups = L.ks;
    return Q4K_OK;
}

int q4k_gemm_config(int64_t M, int64_t K, int64_t P, int32_t *tile_tokens, int32_t *workgroups) {
    clear_error();
    Q4K_TRY(check_mk(M, K));
    if (!tile_tokens || !workgroups) return fail(Q4K_EINVAL, "NULL output");
    const GemmLaunch L = choose_gemm_launch(M, K, P);
    *tile_tokens = 32 * L.r;
    // the launch caps the count at the number of work items
    const int64_t tiles = ((M + 255) / 256) * ((P + 32 * L.r - 1) / (32 * L.r));
    *workgroups = (int32_t)std::max<int64_t>(1, std::min<int64_t>(L.ks, tiles * (K / 256)));
    return Q4K_OK;
}

}  // extern "C"
