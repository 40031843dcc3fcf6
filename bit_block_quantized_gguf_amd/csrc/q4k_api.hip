// q4k_api.hip — C ABI entry points of libq4k: argument validation, error
// reporting, workspace layout, and dispatch to the kernels.  Hot calls never
// allocate or synchronise: the scratch memory they need comes from the
// caller's workspace, whose size q4k_workspace_size() reports.
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

std::mutex g_dev_mutex;
std::map<int, bool> g_dev_ok;

size_t round256(size_t bytes) { return (bytes + 255) / 256 * 256; }

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

size_t region_bytes(size_t partial_floats) {
    return kCounterBytes + round256(partial_floats * sizeof(float));
}

Workspace carve(void *base, size_t partial_floats) {
    Workspace ws;
    char *b = static_cast<char *>(base);
    ws.counters = reinterpret_cast<unsigned *>(b);
    ws.n_counters = kMaxCounters;
    ws.partials = reinterpret_cast<float *>(b + kCounterBytes);
    ws.partial_floats = partial_floats;
    return ws;
}

void free_workspace(Workspace *ws) {
    // counters and partials share one allocation that starts at the counters
    if (ws->counters) (void)hipFree(ws->counters);
    *ws = Workspace();
}

int alloc_workspace(size_t partial_floats, size_t n_counters, Workspace *out) {
    if (n_counters > kMaxCounters) return fail(Q4K_EUNSUPPORTED, "more than %zu workgroups", kMaxCounters);
    const size_t bytes = region_bytes(partial_floats);
    void *base = nullptr;
    if (hipMalloc(&base, bytes) != hipSuccess) {
        (void)hipGetLastError();
        return fail(Q4K_ENOMEM, "workspace: cannot allocate %zu bytes", bytes);
    }
    hipError_t e = hipMemset(base, 0, bytes);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
        (void)hipFree(base);
        return hip_fail(e, "hipMemset(workspace)");
    }
    *out = carve(base, partial_floats);
    return Q4K_OK;
}

}  // namespace q4k

using namespace q4k;

namespace {

constexpr int64_t kMaxRows = (int64_t)1 << 30;   // M
constexpr int64_t kMaxCols = (int64_t)1 << 24;   // K: 63 row strides + a row run stay below 2^32
constexpr int64_t kMaxDim = 0x7FFFFFFF;          // N, P

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

// Shape limits.  Inside a 64-row tile the kernels address weights with
// 32-bit offsets (row * row_bytes + chunk, row < 64) and the GEMM addresses
// its bf16 X slice with a 32-bit byte offset of at most 16 * 2K; K <= 2^24
// keeps both far below 2^31 for every block format (Q8_0's 34/32 bytes per
// weight is the widest).  M <= 2^30 keeps tile indices times rows in int.
int check_mk(int64_t M, int64_t K) {
    if (M < 0 || K <= 0 || K % 256 != 0)
        return fail(Q4K_ESHAPE, "need M >= 0 and K a positive multiple of 256 (M=%lld K=%lld)",
                    (long long)M, (long long)K);
    if (M > kMaxRows) return fail(Q4K_EUNSUPPORTED, "M=%lld beyond 2^30", (long long)M);
    if (K > kMaxCols) return fail(Q4K_EUNSUPPORTED, "K=%lld beyond 2^24", (long long)K);
    return Q4K_OK;
}

int check_ptr(const void *p, const char *name) {
    if (!p) return fail(Q4K_EINVAL, "%s is NULL", name);
    if (!aligned16(p)) return fail(Q4K_EALIGN, "%s is not 16-byte aligned", name);
    return Q4K_OK;
}

int check_ws(const void *ws, size_t ws_bytes, size_t need, const char *what) {
    if (need == 0) return Q4K_OK;
    if (!ws) return fail(Q4K_EINVAL, "%s: workspace is NULL (needs %zu bytes)", what, need);
    if (((uintptr_t)ws & 255u) != 0)
        return fail(Q4K_EALIGN, "%s: workspace is not 256-byte aligned", what);
    if (ws_bytes < need)
        return fail(Q4K_EINVAL, "%s: workspace of %zu bytes, needs %zu (q4k_workspace_size)", what,
                    ws_bytes, need);
    return Q4K_OK;
}

#define Q4K_TRY(expr)            \
    do {                         \
        int rc_ = (expr);        \
        if (rc_) return rc_;     \
    } while (0)

// ---- workspace sizes (bytes) -------------------------------------------

// A batched call splits N greedily into launches of 16, 8, 4, 2 and 1
// vectors; its workspace covers the largest of them.
size_t gemv_ws_bytes(int64_t M, int64_t K, int64_t N) {
    size_t partials = 0;
    for (int nv = 16; nv >= 1; nv >>= 1) {
        if (nv > N) continue;
        const GemvLaunch L = choose_gemv_launch(M, K, nv, 1);
        partials = std::max(partials, gemv_partial_floats(L, nv));
    }
    return region_bytes(partials);
}

size_t q8_ws_bytes(int64_t M, int64_t K) {
    const GemvLaunch L = choose_gemv_q8_launch(M, K);
    return region_bytes(gemv_partial_floats(L, 1));
}

size_t q6_ws_bytes(int64_t M, int64_t K) {
    const GemvLaunch L = choose_gemv_q6_launch(M, K);
    return region_bytes(gemv_partial_floats(L, 1));
}

// MLP workspace: [counters][partials][x * (1 + w)][sums of squares of x][activation]
struct MlpLayout {
    GemvLaunch Lg, Ld;
    size_t partials, off_xg, off_sq, off_act, total;  // offsets in bytes
};

MlpLayout mlp_layout(int64_t hidden, int64_t inter, bool resid) {
    MlpLayout m;
    m.Lg = choose_gemv_launch(inter, hidden, 1, 2, EPI_SWIGLU);
    m.Ld = choose_gemv_launch(hidden, inter, 1, 1, resid ? EPI_RESID : EPI_PLAIN);
    m.partials = std::max(gemv_partial_floats(m.Lg, 1), gemv_partial_floats(m.Ld, 1));
    m.off_xg = region_bytes(m.partials);
    m.off_sq = m.off_xg + round256((size_t)hidden * sizeof(float));
    m.off_act = m.off_sq + round256((size_t)((hidden + 31) / 32) * sizeof(float));
    m.total = m.off_act + round256((size_t)inter * sizeof(float));
    return m;
}

// GEMM workspace: [counter region, unused][partial tiles][bf16 copy of X]
size_t gemm_ws_bytes(int64_t M, int64_t K, int64_t P) {
    const GemmLaunch L = choose_gemm_launch(M, K, P);
    return region_bytes(gemm_partial_floats(L, M, P) + gemm_xb_floats(K, P));
}

// GDN step workspace: [counter region: per-value-head and per-key-head
// arrival counters][head outputs before their norm]
size_t gdn_ws_bytes(int Hk, int Hv) { return region_bytes(gdn_scratch_floats(Hk, Hv)); }

// Attention step workspace: [counter region, unused][split-KV partials]
size_t attn_ws_bytes(int Hq, int Hkv, int64_t cap) {
    return region_bytes(attn_scratch_floats(Hq, Hkv, cap));
}

// The caller has checked the workspace against gemv_ws_bytes(M, K, N).
int gemv_multi(const void *w, const float *X, float *Y, int64_t M, int64_t K, int64_t N,
               void *wsp, size_t ws_bytes, hipStream_t stream) {
    (void)ws_bytes;
    // Pick the largest supported vector count at each step (16, 8, 4, 2, 1).
    int64_t done = 0;
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
        const Workspace ws = carve(wsp, gemv_partial_floats(L, nv));
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

int q4k_version(void) { return 10100; }

int q4k_workspace_size(int32_t op, int64_t M, int64_t K, int64_t N, size_t *bytes) {
    clear_error();
    if (!bytes) return fail(Q4K_EINVAL, "NULL output");
    *bytes = 0;
    switch (op) {
        case Q4K_OP_GEMV:
            Q4K_TRY(check_mk(M, K));
            if (M > 0) *bytes = gemv_ws_bytes(M, K, 1);
            return Q4K_OK;
        case Q4K_OP_GEMV_BATCH:
            Q4K_TRY(check_mk(M, K));
            if (N < 0) return fail(Q4K_ESHAPE, "N must be >= 0");
            if (N > kMaxDim) return fail(Q4K_EUNSUPPORTED, "N beyond 2^31-1");
            if (M > 0 && N > 0) *bytes = gemv_ws_bytes(M, K, N);
            return Q4K_OK;
        case Q4K_OP_GEMV_Q8_0:
            Q4K_TRY(check_mk(M, K));
            if (M > 0) *bytes = q8_ws_bytes(M, K);
            return Q4K_OK;
        case Q4K_OP_GEMV_Q6_K:
            Q4K_TRY(check_mk(M, K));
            if (K % 1024 != 0)
                return fail(Q4K_ESHAPE, "q4k_gemv_q6_k: K must be a multiple of 1024");
            if (M > 0) *bytes = q6_ws_bytes(M, K);
            return Q4K_OK;
        case Q4K_OP_GEMM:
            Q4K_TRY(check_mk(M, K));
            if (N < 0) return fail(Q4K_ESHAPE, "P must be >= 0");
            if (N > kMaxDim) return fail(Q4K_EUNSUPPORTED, "P beyond 2^31-1");
            if (M > 0 && N > 0) *bytes = gemm_ws_bytes(M, K, N);
            return Q4K_OK;
        case Q4K_OP_MLP:
            Q4K_TRY(check_mk(M, K));  // inter x hidden
            Q4K_TRY(check_mk(K, M));  // hidden x inter
            if (M == 0) return fail(Q4K_ESHAPE, "inter must be positive");
            // sized for the residual variant, which needs at least as much
            *bytes = std::max(mlp_layout(K, M, true).total, mlp_layout(K, M, false).total);
            return Q4K_OK;
        case Q4K_OP_GDN_STEP:
            if (M <= 0 || K <= 0 || K % M != 0 || M > 4096 || K > 4096)
                return fail(Q4K_ESHAPE, "gdn: key heads %lld, value heads %lld", (long long)M,
                            (long long)K);
            *bytes = gdn_ws_bytes((int)M, (int)K);
            return Q4K_OK;
        case Q4K_OP_ATTN_STEP:
            if (M <= 0 || K <= 0 || M % K != 0 || M > 65536)
                return fail(Q4K_ESHAPE, "attention: query heads %lld, kv heads %lld", (long long)M,
                            (long long)K);
            if (N <= 0 || N > ((int64_t)1 << 40) / 256 / K)
                return fail(Q4K_ESHAPE, "attention: capacity %lld", (long long)N);
            *bytes = attn_ws_bytes((int)M, (int)K, N);
            return Q4K_OK;
        default:
            return fail(Q4K_EINVAL, "unknown op %d", op);
    }
}

int q4k_dequant(const void *w, float *out, int64_t M, int64_t K, void *stream) {
    clear_error();
    Q4K_TRY(check_mk(M, K));
    if (M == 0) return Q4K_OK;
    Q4K_TRY(check_ptr(w, "w"));
    Q4K_TRY(check_ptr(out, "out"));
    Q4K_TRY(check_device());
    return launch_dequant((const uint8_t *)w, out, M, K, (hipStream_t)stream);
}

int q4k_gemv(const void *w, const float *x, float *y, int64_t M, int64_t K, void *ws,
             size_t ws_bytes, void *stream) {
    clear_error();
    Q4K_TRY(check_mk(M, K));
    if (M == 0) return Q4K_OK;
    Q4K_TRY(check_ptr(w, "w"));
    Q4K_TRY(check_ptr(x, "x"));
    Q4K_TRY(check_ptr(y, "y"));
    Q4K_TRY(check_ws(ws, ws_bytes, gemv_ws_bytes(M, K, 1), "gemv"));
    Q4K_TRY(check_device());
    return gemv_multi(w, x, y, M, K, 1, ws, ws_bytes, (hipStream_t)stream);
}

int q4k_gemv_noalloc(const void *w, const float *x, float *y, int64_t M, int64_t K,
                     void *stream) {
    clear_error();
    Q4K_TRY(check_mk(M, K));
    if (M == 0) return Q4K_OK;
    Q4K_TRY(check_ptr(w, "w"));
    Q4K_TRY(check_ptr(x, "x"));
    Q4K_TRY(check_ptr(y, "y"));
    Q4K_TRY(check_device());
    return gemv_noalloc(w, x, y, M, K, (hipStream_t)stream);
}

int q4k_gemv_batch(const void *w, const float *X, float *Y, int64_t M, int64_t K, int64_t N,
                   void *ws, size_t ws_bytes, void *stream) {
    clear_error();
    Q4K_TRY(check_mk(M, K));
    if (N < 0) return fail(Q4K_ESHAPE, "N must be >= 0");
    if (N > kMaxDim) return fail(Q4K_EUNSUPPORTED, "N beyond 2^31-1");
    if (M == 0 || N == 0) return Q4K_OK;
    Q4K_TRY(check_ptr(w, "w"));
    Q4K_TRY(check_ptr(X, "X"));
    Q4K_TRY(check_ptr(Y, "Y"));
    Q4K_TRY(check_ws(ws, ws_bytes, gemv_ws_bytes(M, K, N), "gemv_batch"));
    Q4K_TRY(check_device());
    return gemv_multi(w, X, Y, M, K, N, ws, ws_bytes, (hipStream_t)stream);
}

int q4k_gemm(const void *w, const float *X, float *Y, int64_t M, int64_t K, int64_t P, void *ws,
             size_t ws_bytes, void *stream) {
    clear_error();
    Q4K_TRY(check_mk(M, K));
    if (P < 0) return fail(Q4K_ESHAPE, "P must be >= 0");
    if (P > kMaxDim) return fail(Q4K_EUNSUPPORTED, "P beyond 2^31-1");
    if (M == 0 || P == 0) return Q4K_OK;
    Q4K_TRY(check_ptr(w, "w"));
    Q4K_TRY(check_ptr(X, "X"));
    Q4K_TRY(check_ptr(Y, "Y"));
    const GemmLaunch L = choose_gemm_launch(M, K, P);
    Q4K_TRY(check_ws(ws, ws_bytes, gemm_ws_bytes(M, K, P), "gemm"));
    Q4K_TRY(check_device());
    const Workspace w2 = carve(ws, gemm_partial_floats(L, M, P) + gemm_xb_floats(K, P));
    return launch_gemm((const uint8_t *)w, X, Y, M, K, P, L, w2, (hipStream_t)stream);
}

int q4k_gemv_q6_k(const void *w, const float *x, float *y, int64_t M, int64_t K, void *ws,
                  size_t ws_bytes, void *stream) {
    clear_error();
    Q4K_TRY(check_mk(M, K));
    if (K % 1024 != 0)
        return fail(Q4K_ESHAPE, "q4k_gemv_q6_k: K must be a multiple of 1024 (K=%lld)", (long long)K);
    if (M == 0) return Q4K_OK;
    Q4K_TRY(check_ptr(w, "w"));
    Q4K_TRY(check_ptr(x, "x"));
    Q4K_TRY(check_ptr(y, "y"));
    const GemvLaunch L = choose_gemv_q6_launch(M, K);
    Q4K_TRY(check_ws(ws, ws_bytes, q6_ws_bytes(M, K), "gemv_q6_k"));
    Q4K_TRY(check_device());
    const Workspace w2 = carve(ws, gemv_partial_floats(L, 1));
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
    p.ws = w2.partials;
    p.cnt = w2.counters;
    return launch_gemv_q6(p, L, (hipStream_t)stream);
}

int q4k_gemv_q8_0(const void *w, const float *x, float *y, int64_t M, int64_t K, void *ws,
                  size_t ws_bytes, void *stream) {
    clear_error();
    Q4K_TRY(check_mk(M, K));
    if (M == 0) return Q4K_OK;
    Q4K_TRY(check_ptr(w, "w"));
    Q4K_TRY(check_ptr(x, "x"));
    Q4K_TRY(check_ptr(y, "y"));
    const GemvLaunch L = choose_gemv_q8_launch(M, K);
    Q4K_TRY(check_ws(ws, ws_bytes, q8_ws_bytes(M, K), "gemv_q8_0"));
    Q4K_TRY(check_device());
    const Workspace w2 = carve(ws, gemv_partial_floats(L, 1));
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
    p.ws = w2.partials;
    p.cnt = w2.counters;
    return launch_gemv_q8(p, L, (hipStream_t)stream);
}

int q4k_mlp(const void *w_gate, const void *w_up, const void *w_down, int64_t hidden,
            int64_t inter, const float *x, const float *norm_w, float eps, const float *resid,
            float *y, float *act, void *ws, size_t ws_bytes, void *stream) {
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
    const hipStream_t st = (hipStream_t)stream;
    const int epi_down = resid ? EPI_RESID : EPI_PLAIN;
    const MlpLayout m = mlp_layout(hidden, inter, resid != nullptr);
    Q4K_TRY(check_ws(ws, ws_bytes, m.total, "mlp"));
    Q4K_TRY(check_device());
    char *base = static_cast<char *>(ws);
    const Workspace w2 = carve(base, m.partials);
    float *xg = reinterpret_cast<float *>(base + m.off_xg);
    float *sq = reinterpret_cast<float *>(base + m.off_sq);
    float *a = act ? act : reinterpret_cast<float *>(base + m.off_act);
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
    p.ks = m.Lg.ks;
    p.ws = w2.partials;
    p.cnt = w2.counters;
    p.in_sq = sq;
    p.in_sq_n = (int32_t)((hidden + 31) / 32);
    p.in_len = (int32_t)hidden;
    p.eps = eps;
    Q4K_TRY(launch_gemv(p, 1, 2, EPI_SWIGLU, m.Lg, st));
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
    q.ks = m.Ld.ks;
    q.ws = w2.partials;
    q.cnt = w2.counters;
    q.resid = resid;
    return launch_gemv(q, 1, 1, epi_down, m.Ld, st);
}

int q4k_gdn_step(const q4k_gdn_params *p, const float *u, float *conv_state, float *state,
                 float *out, void *ws, size_t ws_bytes, void *stream) {
    clear_error();
    if (!p) return fail(Q4K_EINVAL, "NULL parameters");
    if (p->key_heads <= 0 || p->value_heads <= 0 || p->value_heads % p->key_heads != 0 ||
        p->key_heads > 4096 || p->value_heads > 4096)
        return fail(Q4K_ESHAPE, "gdn: need value heads a positive multiple of key heads");
    if (p->key_dim != 128 || p->value_dim != 128)
        return fail(Q4K_ESHAPE, "gdn: key and value head dimensions must be 128");
    if (!(p->eps >= 0.f) || !std::isfinite(p->eps)) return fail(Q4K_EINVAL, "eps must be finite and >= 0");
    Q4K_TRY(check_ptr(u, "u"));
    Q4K_TRY(check_ptr(conv_state, "conv_state"));
    Q4K_TRY(check_ptr(state, "state"));
    Q4K_TRY(check_ptr(out, "out"));
    Q4K_TRY(check_ptr(p->conv_w, "conv_w"));
    Q4K_TRY(check_ptr(p->a_log, "a_log"));
    Q4K_TRY(check_ptr(p->dt_bias, "dt_bias"));
    Q4K_TRY(check_ptr(p->norm_w, "norm_w"));
    Q4K_TRY(check_ws(ws, ws_bytes, gdn_ws_bytes(p->key_heads, p->value_heads), "gdn_step"));
    Q4K_TRY(check_device());
    GdnShape sh{p->key_heads, p->value_heads, p->eps};
    float *scratch = reinterpret_cast<float *>(static_cast<char *>(ws) + kCounterBytes);
    static_assert(kMaxCounters >= 8192, "a counter per value head and per key head");
    return launch_gdn_step(sh, u, p->conv_w, p->a_log, p->dt_bias, p->norm_w, conv_state, state,
                           out, nullptr, scratch, static_cast<unsigned *>(ws),
                           (hipStream_t)stream);
}

int q4k_attn_step(const q4k_attn_params *p, const float *u, float *k_cache, float *v_cache,
                  int64_t capacity, int64_t pos, float *out, void *ws, size_t ws_bytes,
                  void *stream) {
    clear_error();
    if (!p) return fail(Q4K_EINVAL, "NULL parameters");
    if (p->head_dim != 256) return fail(Q4K_ESHAPE, "attention: head dimension must be 256");
    if (p->q_heads <= 0 || p->kv_heads <= 0 || p->q_heads % p->kv_heads != 0 ||
        p->q_heads > 65536)
        return fail(Q4K_ESHAPE, "attention: need query heads a positive multiple of kv heads");
    if (p->rope_dim < 0 || p->rope_dim > 256 || p->rope_dim % 2 != 0)
        return fail(Q4K_ESHAPE, "attention: rope_dim must be even and in 0..256");
    if (capacity <= 0 || pos < 0 || pos >= capacity)
        return fail(Q4K_ESHAPE, "attention: position %lld outside the cache of %lld",
                    (long long)pos, (long long)capacity);
    if (capacity > ((int64_t)1 << 40) / 256 / p->kv_heads)
        return fail(Q4K_EUNSUPPORTED, "attention: cache too large");
    if (!(p->eps >= 0.f) || !std::isfinite(p->eps) || !(p->rope_theta > 0.f))
        return fail(Q4K_EINVAL, "eps must be >= 0 and rope_theta > 0");
    Q4K_TRY(check_ptr(u, "u"));
    Q4K_TRY(check_ptr(k_cache, "k_cache"));
    Q4K_TRY(check_ptr(v_cache, "v_cache"));
    Q4K_TRY(check_ptr(out, "out"));
    Q4K_TRY(check_ptr(p->q_norm_w, "q_norm_w"));
    Q4K_TRY(check_ptr(p->k_norm_w, "k_norm_w"));
    Q4K_TRY(check_ws(ws, ws_bytes, attn_ws_bytes(p->q_heads, p->kv_heads, capacity), "attn_step"));
    Q4K_TRY(check_device());
    AttnShape sh{p->q_heads, p->kv_heads, p->rope_dim, p->rope_theta, p->eps};
    float *scratch = reinterpret_cast<float *>(static_cast<char *>(ws) + kCounterBytes);
    return launch_attn_step(sh, u, p->q_norm_w, p->k_norm_w, k_cache, v_cache, capacity, pos,
                            nullptr, out, nullptr, scratch, (hipStream_t)stream);
}

int q4k_check_partition(int32_t op, int64_t M, int64_t K, int64_t N, int32_t workgroups) {
    clear_error();
    if (workgroups < 0 || workgroups > (int32_t)kMaxCounters)
        return fail(Q4K_EINVAL, "workgroups must be in 0..%zu", kMaxCounters);
    if (M <= 0 || K <= 0 || M > kMaxRows || K > kMaxCols)
        return fail(Q4K_ESHAPE, "bad shape %lld x %lld", (long long)M, (long long)K);
    switch (op) {
        case Q4K_OP_GEMV: return check_gemv_partition(M, K, 1, 1, workgroups);
        case Q4K_OP_GEMV_BATCH:
            if (N < 1) return fail(Q4K_ESHAPE, "N must be >= 1");
            return check_gemv_partition(M, K, (int)std::min<int64_t>(N, 16), 1, workgroups);
        case Q4K_OP_MLP: {  // M = intermediate, K = hidden
            const int rc = check_gemv_partition(M, K, 1, 2, workgroups);
            return rc ? rc : check_gemv_partition(K, M, 1, 1, workgroups);
        }
        case Q4K_OP_GEMM:
            if (N < 1) return fail(Q4K_ESHAPE, "P must be >= 1");
            return check_gemm_partition(M, K, N, 0, workgroups);
        case Q4K_OP_GEMV_Q8_0: return check_gemv_q8_partition(M, K, workgroups);
        case Q4K_OP_GEMV_Q6_K: return check_gemv_q6_partition(M, K, workgroups);
        default: return fail(Q4K_EINVAL, "op %d has no partition to check", op);
    }
}

/* Benchmark knobs: force the GEMV workgroup count and the GEMM tile width and
 * workgroup count (0 restores the shape heuristics).  Not thread-safe with
 * respect to concurrent calls; meant for sweeps. */
int q4k_tune_gemv(int32_t waves_per_group, int32_t workgroups) {
    clear_error();
    if (waves_per_group != 0 && waves_per_group != 4)
        return fail(Q4K_EINVAL, "waves_per_group must be 0 or 4");
    if (workgroups < 0 || workgroups > (int32_t)kMaxCounters)
        return fail(Q4K_EINVAL, "workgroups must be in 0..%zu", kMaxCounters);
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
