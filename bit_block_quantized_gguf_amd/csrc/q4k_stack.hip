// q4k_stack.hip — the per-token decode matmul chain as one hipGraph.
//
// The diagnosis page ("Mac Qwen3.6-27B Metal Q4_K perf diagnosis", TL;DR and
// §4) finds decode dominated not by arithmetic but by one submission and one
// host round trip per matmul (~336 per token), and names the fix: keep the
// activation on the device and submit the whole token once.  Here the chain
// is captured once into a hipGraph and each token is a single
// hipGraphLaunch; the activations never leave the device.
//
// Node list per token (4 GEMV kernels per layer, gate and up fused):
//   sumsq(h0)
//   for each layer:  u     = W_in rmsn(h)                 (EPI_SCALE)
//                    h_mid = h + W_out rmsn(u[:K_out])    (EPI_RESID)
//                    g, v, a = silu(g) * v                (EPI_SWIGLU, gate|up in one pass)
//                    h'    = h_mid + W_down rmsn(a)       (EPI_RESID)
//   logits = W_lm rmsn(h)                                 (EPI_SCALE)
// Every GEMV's epilogue writes the per-32-row sums of squares of its
// output; the consumer adds them in a fixed order to get its input's RMS, so
// RMS normalisation costs no extra pass and no extra node.
#include "q4k_internal.hpp"

#include <string.h>

#include <algorithm>
#include <new>
#include <vector>

using namespace q4k;

struct q4k_stack {
    int device = 0;
    int64_t hidden = 0;
    int32_t n_layers = 0;
    float eps = 1e-6f;
    std::vector<q4k_layer> layers;
    q4k_mat lm_head{};
    float *arena = nullptr;
    size_t arena_floats = 0;
    std::vector<int64_t> off_h, off_u, off_hmid, off_g, off_v, off_a;
    int64_t off_logits = 0;
    float *sq = nullptr;  // per-tile sums of squares
    size_t sq_floats = 0;
    std::vector<int64_t> sq_h, sq_u, sq_hmid, sq_a;
    int64_t sq_logits = 0;
    Workspace ws;
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    int64_t n_nodes = 0;
};

namespace {

int check_mat(const q4k_mat &m, const char *name, int layer) {
    if (!m.w) return fail(Q4K_EINVAL, "layer %d %s: NULL weights", layer, name);
    if (((uintptr_t)m.w & 15u) != 0)
        return fail(Q4K_EALIGN, "layer %d %s: weights not 16-byte aligned", layer, name);
    if (m.M <= 0 || m.K <= 0 || m.K % 256 != 0 || m.M > 0x7FFFFFFF || m.K > 0x7FFFFFFF)
        return fail(Q4K_ESHAPE, "layer %d %s: bad shape %lld x %lld", layer, name,
                    (long long)m.M, (long long)m.K);
    return Q4K_OK;
}

// number of 32-element sum-of-squares granules of a vector
int64_t tiles_of(int64_t n) { return (n + 31) / 32; }

GemvParams base_params(const q4k_mat &m) {
    GemvParams p = {};
    p.w0 = (const uint8_t *)m.w;
    p.M = (int32_t)m.M;
    p.K = (int32_t)m.K;
    p.nb = (int32_t)(m.K / 256);
    p.row_bytes = (m.K / 256) * 144;
    p.x_stride = m.K;
    p.y_stride = m.M;
    return p;
}

// Enqueue the whole token on `cs` (under capture).
int enqueue_token(q4k_stack *s, hipStream_t cs, int64_t *nodes) {
    float *A = s->arena;
    float *SQ = s->sq;
    int64_t n = 0;
    int rc = launch_sumsq(A + s->off_h[0], s->hidden, SQ + s->sq_h[0], cs);
    if (rc) return rc;
    ++n;
    auto run = [&](GemvParams p, int nmat, int epi, int64_t M, int64_t K) -> int {
        const GemvLaunch L = choose_gemv_launch(M, K, 1, nmat, epi);
        p.ks = L.ks;
        p.ws = s->ws.partials;
        p.cnt = s->ws.counters;
        p.eps = s->eps;
        ++n;
        return launch_gemv(p, 1, nmat, epi, L, cs);
    };
    for (int32_t l = 0; l < s->n_layers; ++l) {
        const q4k_layer &L = s->layers[l];
        // mixer-in: u = W_in rmsn(h)
        GemvParams p = base_params(L.mix_in);
        p.x = A + s->off_h[l];
        p.y = A + s->off_u[l];
        p.in_sq = SQ + s->sq_h[l];
        p.in_sq_n = (int32_t)tiles_of(s->hidden);
        p.in_len = (int32_t)s->hidden;
        p.out_sq = SQ + s->sq_u[l];
        if ((rc = run(p, 1, EPI_SCALE, L.mix_in.M, L.mix_in.K))) return rc;
        // mixer-out: h_mid = h + W_out rmsn(u[:K_out])
        p = base_params(L.mix_out);
        p.x = A + s->off_u[l];
        p.y = A + s->off_hmid[l];
        p.in_sq = SQ + s->sq_u[l];
        p.in_sq_n = (int32_t)tiles_of(L.mix_out.K);
        p.in_len = (int32_t)L.mix_out.K;
        p.resid = A + s->off_h[l];
        p.out_sq = SQ + s->sq_hmid[l];
        if ((rc = run(p, 1, EPI_RESID, L.mix_out.M, L.mix_out.K))) return rc;
        // gate|up: a = silu(W_gate rmsn(h_mid)) * (W_up rmsn(h_mid))
        p = base_params(L.gate);
        p.w1 = (const uint8_t *)L.up.w;
        p.x = A + s->off_hmid[l];
        p.y = A + s->off_a[l];
        p.y_g = A + s->off_g[l];
        p.y_v = A + s->off_v[l];
        p.in_sq = SQ + s->sq_hmid[l];
        p.in_sq_n = (int32_t)tiles_of(s->hidden);
        p.in_len = (int32_t)s->hidden;
        p.out_sq = SQ + s->sq_a[l];
        if ((rc = run(p, 2, EPI_SWIGLU, L.gate.M, L.gate.K))) return rc;
        // down: h' = h_mid + W_down rmsn(a)
        p = base_params(L.down);
        p.x = A + s->off_a[l];
        p.y = A + s->off_h[l + 1];
        p.in_sq = SQ + s->sq_a[l];
        p.in_sq_n = (int32_t)tiles_of(L.down.K);
        p.in_len = (int32_t)L.down.K;
        p.resid = A + s->off_hmid[l];
        p.out_sq = SQ + s->sq_h[l + 1];
        if ((rc = run(p, 1, EPI_RESID, L.down.M, L.down.K))) return rc;
    }
    GemvParams p = base_params(s->lm_head);
    p.x = A + s->off_h[s->n_layers];
    p.y = A + s->off_logits;
    p.in_sq = SQ + s->sq_h[s->n_layers];
    p.in_sq_n = (int32_t)tiles_of(s->hidden);
    p.in_len = (int32_t)s->hidden;
    p.out_sq = SQ + s->sq_logits;
    if ((rc = run(p, 1, EPI_SCALE, s->lm_head.M, s->lm_head.K))) return rc;
    *nodes = n;
    return Q4K_OK;
}

void release(q4k_stack *s) {
    if (!s) return;
    (void)hipSetDevice(s->device);
    (void)hipDeviceSynchronize();
    if (s->exec) (void)hipGraphExecDestroy(s->exec);
    if (s->graph) (void)hipGraphDestroy(s->graph);
    if (s->arena) (void)hipFree(s->arena);
    if (s->sq) (void)hipFree(s->sq);
    free_workspace(&s->ws);
    delete s;
}

}  // namespace

extern "C" {

int q4k_decode_stack_create(const q4k_stack_desc *d, void *stream, q4k_stack **out) {
    clear_error();
    if (!d || !out) return fail(Q4K_EINVAL, "NULL descriptor or output");
    *out = nullptr;
    if (d->flags != 0) return fail(Q4K_EINVAL, "flags must be 0");
    if (d->n_layers < 0 || d->hidden <= 0 || d->hidden % 256 != 0)
        return fail(Q4K_ESHAPE, "need n_layers >= 0 and hidden a positive multiple of 256");
    if (d->n_layers > 0 && !d->layers) return fail(Q4K_EINVAL, "NULL layers");
    if (!(d->eps >= 0.0f)) return fail(Q4K_EINVAL, "eps must be >= 0");
    const int64_t H = d->hidden;
    int rc;
    for (int32_t l = 0; l < d->n_layers; ++l) {
        const q4k_layer &L = d->layers[l];
        if ((rc = check_mat(L.mix_in, "mix_in", l)) || (rc = check_mat(L.mix_out, "mix_out", l)) ||
            (rc = check_mat(L.gate, "gate", l)) || (rc = check_mat(L.up, "up", l)) ||
            (rc = check_mat(L.down, "down", l)))
            return rc;
        if (L.mix_in.K != H || L.gate.K != H || L.up.K != H)
            return fail(Q4K_ESHAPE, "layer %d: mix_in/gate/up K must equal hidden", l);
        if (L.mix_out.M != H || L.down.M != H)
            return fail(Q4K_ESHAPE, "layer %d: mix_out/down M must equal hidden", l);
        if (L.mix_out.K > L.mix_in.M)
            return fail(Q4K_ESHAPE, "layer %d: mix_out K exceeds mix_in M", l);
        if (L.gate.M != L.up.M || L.down.K != L.gate.M)
            return fail(Q4K_ESHAPE, "layer %d: gate/up M must equal down K", l);
    }
    if ((rc = check_mat(d->lm_head, "lm_head", -1))) return rc;
    if (d->lm_head.K != H) return fail(Q4K_ESHAPE, "lm_head K must equal hidden");

    q4k_stack *s = new (std::nothrow) q4k_stack();
    if (!s) return fail(Q4K_ENOMEM, "plan allocation failed");
    if (hipGetDevice(&s->device) != hipSuccess) {
        delete s;
        return fail(Q4K_EHIP, "hipGetDevice failed");
    }
    {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, s->device) != hipSuccess ||
            strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
            delete s;
            return fail(Q4K_EUNSUPPORTED, "decode stack needs a gfx950 device");
        }
    }
    s->hidden = H;
    s->n_layers = d->n_layers;
    s->eps = d->eps;
    s->layers.assign(d->layers, d->layers + d->n_layers);
    s->lm_head = d->lm_head;

    // arena layout
    size_t off = 0, sqo = 0;
    auto take = [](size_t &o, int64_t n) {
        const int64_t r = (int64_t)o;
        o += (size_t)((n + 63) / 64 * 64);  // keep every buffer 256-byte aligned
        return r;
    };
    size_t max_partials = 0, max_counters = 0;
    auto need = [&](int64_t M, int64_t K, int nmat, int epi) {
        const GemvLaunch L = choose_gemv_launch(M, K, 1, nmat, epi);
        max_partials = std::max(max_partials, gemv_partial_floats(L, 1));
        max_counters = std::max(max_counters, gemv_counters(L));
    };
    for (int32_t l = 0; l <= s->n_layers; ++l) {
        s->off_h.push_back(take(off, H));
        s->sq_h.push_back(take(sqo, tiles_of(H)));
        if (l == s->n_layers) break;
        const q4k_layer &L = s->layers[l];
        s->off_u.push_back(take(off, L.mix_in.M));
        s->off_hmid.push_back(take(off, H));
        s->off_g.push_back(take(off, L.gate.M));
        s->off_v.push_back(take(off, L.gate.M));
        s->off_a.push_back(take(off, L.gate.M));
        s->sq_u.push_back(take(sqo, tiles_of(L.mix_in.M)));
        s->sq_hmid.push_back(take(sqo, tiles_of(H)));
        s->sq_a.push_back(take(sqo, tiles_of(L.gate.M)));
        need(L.mix_in.M, L.mix_in.K, 1, EPI_SCALE);
        need(L.mix_out.M, L.mix_out.K, 1, EPI_RESID);
        need(L.gate.M, L.gate.K, 2, EPI_SWIGLU);
        need(L.down.M, L.down.K, 1, EPI_RESID);
    }
    s->off_logits = take(off, s->lm_head.M);
    s->sq_logits = take(sqo, tiles_of(s->lm_head.M));
    need(s->lm_head.M, s->lm_head.K, 1, EPI_SCALE);
    s->arena_floats = off;
    s->sq_floats = sqo;

    if (hipMalloc(&s->arena, off * sizeof(float)) != hipSuccess ||
        hipMalloc(&s->sq, sqo * sizeof(float)) != hipSuccess) {
        (void)hipGetLastError();
        release(s);
        return fail(Q4K_ENOMEM, "decode stack: arena allocation failed");
    }
    if ((rc = alloc_workspace(max_partials, max_counters, &s->ws))) {
        release(s);
        return rc;
    }
    if (hipMemset(s->arena, 0, off * sizeof(float)) != hipSuccess ||
        hipMemset(s->sq, 0, sqo * sizeof(float)) != hipSuccess ||
        hipDeviceSynchronize() != hipSuccess) {
        release(s);
        return fail(Q4K_EHIP, "decode stack: arena clear failed");
    }

    // capture on a private stream (default priority)
    hipStream_t cs = nullptr;
    if (hipStreamCreateWithFlags(&cs, hipStreamNonBlocking) != hipSuccess) {
        release(s);
        return fail(Q4K_EHIP, "decode stack: stream creation failed");
    }
    hipError_t e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
    int64_t nodes = 0;
    if (e == hipSuccess) {
        rc = enqueue_token(s, cs, &nodes);
        hipGraph_t g = nullptr;
        hipError_t e2 = hipStreamEndCapture(cs, &g);
        if (rc == Q4K_OK && e2 != hipSuccess) rc = hip_fail(e2, "hipStreamEndCapture");
        s->graph = g;
    } else {
        rc = hip_fail(e, "hipStreamBeginCapture");
    }
    (void)hipStreamDestroy(cs);
    if (rc == Q4K_OK) {
        e = hipGraphInstantiate(&s->exec, s->graph, nullptr, nullptr, 0);
        if (e != hipSuccess) rc = hip_fail(e, "hipGraphInstantiate");
    }
    if (rc == Q4K_OK) {
        // upload the executable graph now so the first token pays no setup
        e = hipGraphUpload(s->exec, (hipStream_t)stream);
        if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
        if (e != hipSuccess) rc = hip_fail(e, "hipGraphUpload");
    }
    if (rc != Q4K_OK) {
        release(s);
        return rc;
    }
    s->n_nodes = nodes;
    *out = s;
    return Q4K_OK;
}

int q4k_decode_stack(q4k_stack *s, const float *h_in, float *logits, void *stream) {
    clear_error();
    if (!s || !h_in) return fail(Q4K_EINVAL, "NULL plan or input");
    if (((uintptr_t)h_in & 15u) || ((uintptr_t)logits & 15u))
        return fail(Q4K_EALIGN, "h_in/logits not 16-byte aligned");
    hipStream_t st = (hipStream_t)stream;
    Q4K_HIP(hipMemcpyAsync(s->arena + s->off_h[0], h_in, (size_t)s->hidden * sizeof(float),
                           hipMemcpyDeviceToDevice, st));
    Q4K_HIP(hipGraphLaunch(s->exec, st));
    if (logits)
        Q4K_HIP(hipMemcpyAsync(logits, s->arena + s->off_logits,
                               (size_t)s->lm_head.M * sizeof(float), hipMemcpyDeviceToDevice, st));
    return Q4K_OK;
}

int q4k_decode_stack_buffer(q4k_stack *s, int32_t layer, int32_t which, const float **ptr,
                            int64_t *n) {
    clear_error();
    if (!s || !ptr || !n) return fail(Q4K_EINVAL, "NULL argument");
    if (which == Q4K_BUF_LOGITS) {
        *ptr = s->arena + s->off_logits;
        *n = s->lm_head.M;
        return Q4K_OK;
    }
    const int32_t max_layer = which == Q4K_BUF_H ? s->n_layers : s->n_layers - 1;
    if (layer < 0 || layer > max_layer) return fail(Q4K_EINVAL, "layer %d out of range", layer);
    switch (which) {
        case Q4K_BUF_H: *ptr = s->arena + s->off_h[layer]; *n = s->hidden; break;
        case Q4K_BUF_U: *ptr = s->arena + s->off_u[layer]; *n = s->layers[layer].mix_in.M; break;
        case Q4K_BUF_HMID: *ptr = s->arena + s->off_hmid[layer]; *n = s->hidden; break;
        case Q4K_BUF_G: *ptr = s->arena + s->off_g[layer]; *n = s->layers[layer].gate.M; break;
        case Q4K_BUF_V: *ptr = s->arena + s->off_v[layer]; *n = s->layers[layer].gate.M; break;
        case Q4K_BUF_A: *ptr = s->arena + s->off_a[layer]; *n = s->layers[layer].gate.M; break;
        default: return fail(Q4K_EINVAL, "unknown buffer %d", which);
    }
    return Q4K_OK;
}

int q4k_decode_stack_nodes(q4k_stack *s, int64_t *n_nodes) {
    clear_error();
    if (!s || !n_nodes) return fail(Q4K_EINVAL, "NULL argument");
    *n_nodes = s->n_nodes;
    return Q4K_OK;
}

void q4k_decode_stack_destroy(q4k_stack *s) { release(s); }

}  // extern "C"
