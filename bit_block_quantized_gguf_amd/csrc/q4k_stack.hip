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
//   for each layer:  u     = W_in rmsn(h)                 (EPI_SCALE)
//                    h_mid = h + W_out rmsn(u[:K_out])    (EPI_RESID)
//                    g, v, a = silu(g) * v                (EPI_SWIGLU, gate|up in one pass)
//                    h'    = h_mid + W_down rmsn(a)       (EPI_RESID)
//   logits = W_lm rmsn(h)                                 (EPI_SCALE)
// Every GEMV's epilogue writes the per-32-row sums of squares of its
// output; the consumer adds them in a fixed order to get its input's RMS, so
// RMS normalisation costs no extra pass and no extra node.  The first GEMV
// adds the squares of h0 itself.
//
// A persistent plan (Q4K_STACK_PERSISTENT) runs the same GEMV nodes, with
// the same parameters and the same unit split, inside one cooperative
// kernel per token (stack_kernel in q4k_gemv.hip).
//
// With the real token mixers ("Qwen3.6-27B on Apple M3 Pro — the llama.cpp
// parity bar", architecture list; §4 of the diagnosis page asks for the GDN
// recurrence and the attention on the device too), each layer runs
//   u = W_in rmsn(h);  o = GDN step(u) or attention step(u, pos);
//   sumsq(o);  h_mid = h + W_out rmsn(o);  then the MLP as above,
// and a last one-thread node advances the device-side position.  The plan
// owns the recurrent states and KV caches.
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
    std::vector<int64_t> off_h, off_u, off_hmid, off_g, off_v, off_a, off_o;
    int64_t off_logits = 0;
    float *sq = nullptr;  // per-tile sums of squares
    size_t sq_floats = 0;
    std::vector<int64_t> sq_h, sq_u, sq_hmid, sq_a, sq_o;
    int64_t sq_logits = 0;
    Workspace ws;
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    int64_t n_nodes = 0;
    // token mixers
    bool mixers = false;
    std::vector<q4k_mixer> mix;
    int64_t cap = 0;                  // KV-cache positions
    float *states = nullptr;          // every layer's conv state, S or K/V caches
    size_t state_floats = 0;
    std::vector<int64_t> st_a, st_b;  // per layer: conv state / K cache, S / V cache
    float *mix_scratch = nullptr;     // GDN head outputs; attention partials
    unsigned *mix_cnt = nullptr;      // GDN arrival counters (zero between calls)
    int64_t *pos_dev = nullptr;       // device-side position
    int64_t host_pos = 0;             // tokens launched since creation or reset
    // persistent plan
    bool persistent = false;
    int pgroups = 0;                  // co-resident workgroups of the kernel
    void *pnodes = nullptr;           // node descriptors (device)
    unsigned *psync = nullptr;        // kStackSyncLanes arrival counters per node, then the error word
    unsigned epoch = 0;               // tokens launched (each node's counters grow by pgroups in all)
    int spin = 1 << 20;               // polls before a wait gives up
};

namespace {

constexpr int MD = 128;   // GDN head dimension
constexpr size_t kMixCounters = 8192;  // GDN arrival counters: per value head and key head
constexpr int AHD = 256;  // attention head dimension

int check_mat(const q4k_mat &m, const char *name, int layer) {
    if (!m.w) return fail(Q4K_EINVAL, "layer %d %s: NULL weights", layer, name);
    if (((uintptr_t)m.w & 15u) != 0)
        return fail(Q4K_EALIGN, "layer %d %s: weights not 16-byte aligned", layer, name);
    if (m.M <= 0 || m.K <= 0 || m.K % 256 != 0 || m.M > ((int64_t)1 << 30) ||
        m.K > ((int64_t)1 << 24))
        return fail(Q4K_ESHAPE, "layer %d %s: bad shape %lld x %lld", layer, name,
                    (long long)m.M, (long long)m.K);
    return Q4K_OK;
}

bool al16(const void *p) { return p && ((uintptr_t)p & 15u) == 0; }

int check_mixer(const q4k_layer &L, const q4k_mixer &m, int l) {
    if (L.kind == 0) {
        const q4k_gdn_params &g = m.gdn;
        if (g.key_heads <= 0 || g.value_heads <= 0 || g.value_heads % g.key_heads != 0 ||
            g.key_dim != MD || g.value_dim != MD || g.key_heads > 4096 || g.value_heads > 4096)
            return fail(Q4K_ESHAPE, "layer %d: GDN heads must be 128-dim, value heads a multiple "
                        "of key heads", l);
        if (!(g.eps >= 0.f)) return fail(Q4K_EINVAL, "layer %d: GDN eps", l);
        if (!al16(g.conv_w) || !al16(g.a_log) || !al16(g.dt_bias) || !al16(g.norm_w))
            return fail(Q4K_EINVAL, "layer %d: GDN parameter NULL or not 16-byte aligned", l);
        const int64_t Min = (int64_t)(2 * g.key_heads + 2 * g.value_heads) * MD + 2 * g.value_heads;
        if (L.mix_in.M != Min || L.mix_out.K != (int64_t)g.value_heads * MD)
            return fail(Q4K_ESHAPE, "layer %d: GDN needs mix_in.M %lld and mix_out.K %lld", l,
                        (long long)Min, (long long)g.value_heads * MD);
    } else if (L.kind == 1) {
        const q4k_attn_params &a = m.attn;
        if (a.head_dim != AHD || a.q_heads <= 0 || a.kv_heads <= 0 ||
            a.q_heads % a.kv_heads != 0 || a.rope_dim < 0 || a.rope_dim > AHD ||
            a.rope_dim % 2 != 0 || a.q_heads > 65536)
            return fail(Q4K_ESHAPE, "layer %d: attention heads must be 256-dim, q heads a "
                        "multiple of kv heads, rope_dim even", l);
        if (!(a.eps >= 0.f) || !(a.rope_theta > 0.f))
            return fail(Q4K_EINVAL, "layer %d: attention eps / theta", l);
        if (!al16(a.q_norm_w) || !al16(a.k_norm_w))
            return fail(Q4K_EINVAL, "layer %d: attention norm weights NULL or not aligned", l);
        const int64_t Min = (int64_t)(2 * a.q_heads + 2 * a.kv_heads) * AHD;
        if (L.mix_in.M != Min || L.mix_out.K != (int64_t)a.q_heads * AHD)
            return fail(Q4K_ESHAPE, "layer %d: attention needs mix_in.M %lld and mix_out.K %lld",
                        l, (long long)Min, (long long)a.q_heads * AHD);
    } else {
        return fail(Q4K_EINVAL, "layer %d: kind must be 0 or 1 with mixers", l);
    }
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

__global__ void advance_position_kernel(int64_t *pos) { *pos += 1; }

__global__ __launch_bounds__(256) void zero_kernel(float *p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0.f;
}

// Enqueue the whole token on `cs` (under capture), or, with `pn`, append the
// GEMV nodes' descriptors for the persistent kernel instead (no mixers then).
int enqueue_token(q4k_stack *s, hipStream_t cs, int64_t *nodes, std::vector<uint8_t> *pn) {
    float *A = s->arena;
    float *SQ = s->sq;
    int64_t n = 0;
    int rc;
    // the first GEMV reads h0 and adds its squares itself
    auto h_sq = [&](int32_t l) -> const float * { return l == 0 ? nullptr : SQ + s->sq_h[l]; };
    auto run = [&](GemvParams p, int nmat, int epi, int64_t M, int64_t K) -> int {
        p.ws = s->ws.partials;
        p.cnt = s->ws.counters;
        p.eps = s->eps;
        ++n;
        if (pn) {
            const size_t at = pn->size();
            pn->resize(at + stack_node_bytes());
            return fill_stack_node(pn->data() + at, p, nmat, epi, s->pgroups);
        }
        const GemvLaunch L = choose_gemv_launch(M, K, 1, nmat, epi);
        p.ks = L.ks;
        return launch_gemv(p, 1, nmat, epi, L, cs);
    };
    for (int32_t l = 0; l < s->n_layers; ++l) {
        const q4k_layer &L = s->layers[l];
        // mixer-in: u = W_in rmsn(h)
        GemvParams p = base_params(L.mix_in);
        p.x = A + s->off_h[l];
        p.y = A + s->off_u[l];
        p.in_sq = h_sq(l);
        p.in_sq_n = (int32_t)tiles_of(s->hidden);
        p.in_len = (int32_t)s->hidden;
        p.out_sq = SQ + s->sq_u[l];
        if ((rc = run(p, 1, EPI_SCALE, L.mix_in.M, L.mix_in.K))) return rc;
        // mixer-out: h_mid = h + W_out rmsn(m), m = the mixer output (or u[:K_out])
        const float *mo = A + s->off_u[l];
        const float *mo_sq = SQ + s->sq_u[l];
        if (s->mixers) {
            if (pn) return fail(Q4K_EUNSUPPORTED, "persistent plans have no token mixers");
            const q4k_mixer &m = s->mix[l];
            float *o = A + s->off_o[l];
            if (L.kind == 0) {
                const GdnShape sh{m.gdn.key_heads, m.gdn.value_heads, m.gdn.eps};
                if ((rc = launch_gdn_step(sh, A + s->off_u[l], m.gdn.conv_w, m.gdn.a_log,
                                          m.gdn.dt_bias, m.gdn.norm_w, s->states + s->st_a[l],
                                          s->states + s->st_b[l], o, SQ + s->sq_o[l],
                                          s->mix_scratch, s->mix_cnt, cs)))
                    return rc;
                n += 1;
            } else {
                const AttnShape sh{m.attn.q_heads, m.attn.kv_heads, m.attn.rope_dim,
                                   m.attn.rope_theta, m.attn.eps};
                if ((rc = launch_attn_step(sh, A + s->off_u[l], m.attn.q_norm_w, m.attn.k_norm_w,
                                           s->states + s->st_a[l], s->states + s->st_b[l], s->cap,
                                           0, s->pos_dev, o, SQ + s->sq_o[l], s->mix_scratch,
                                           cs)))
                    return rc;
                n += 2;
            }
            mo = o;
            mo_sq = SQ + s->sq_o[l];
        }
        p = base_params(L.mix_out);
        p.x = mo;
        p.y = A + s->off_hmid[l];
        p.in_sq = mo_sq;
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
    p.in_sq = h_sq(s->n_layers);
    p.in_sq_n = (int32_t)tiles_of(s->hidden);
    p.in_len = (int32_t)s->hidden;
    p.out_sq = SQ + s->sq_logits;
    if ((rc = run(p, 1, EPI_SCALE, s->lm_head.M, s->lm_head.K))) return rc;
    if (s->mixers) {
        hipLaunchKernelGGL(advance_position_kernel, dim3(1), dim3(1), 0, cs, s->pos_dev);
        Q4K_HIP(hipGetLastError());
        ++n;
    }
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
    if (s->states) (void)hipFree(s->states);
    if (s->mix_scratch) (void)hipFree(s->mix_scratch);
    if (s->mix_cnt) (void)hipFree(s->mix_cnt);
    if (s->pos_dev) (void)hipFree(s->pos_dev);
    if (s->pnodes) (void)hipFree(s->pnodes);
    if (s->psync) (void)hipFree(s->psync);
    free_workspace(&s->ws);
    delete s;
}

int zero_states(q4k_stack *s, hipStream_t st) {
    if (!s->mixers) return Q4K_OK;
    if (s->state_floats) {
        hipLaunchKernelGGL(zero_kernel, dim3((unsigned)((s->state_floats + 255) / 256)), dim3(256),
                           0, st, s->states, (int64_t)s->state_floats);
        Q4K_HIP(hipGetLastError());
    }
    // the position too, by a kernel (a plan may be reset inside a captured graph)
    hipLaunchKernelGGL(zero_kernel, dim3(1), dim3(256), 0, st, reinterpret_cast<float *>(s->pos_dev),
                       (int64_t)(sizeof(int64_t) / sizeof(float)));
    Q4K_HIP(hipGetLastError());
    // and the GDN arrival counters (zero after every complete token; cleared
    // here in case a token did not run to completion)
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)((kMixCounters + 255) / 256)), dim3(256), 0, st,
                       reinterpret_cast<float *>(s->mix_cnt), (int64_t)kMixCounters);
    Q4K_HIP(hipGetLastError());
    s->host_pos = 0;
    return Q4K_OK;
}

}  // namespace

extern "C" {

int q4k_decode_stack_create(const q4k_stack_desc *d, void *stream, q4k_stack **out) {
    clear_error();
    if (!d || !out) return fail(Q4K_EINVAL, "NULL descriptor or output");
    *out = nullptr;
    if (d->flags != 0 && d->flags != Q4K_STACK_MIXERS && d->flags != Q4K_STACK_PERSISTENT)
        return fail(Q4K_EINVAL, "flags must be 0, Q4K_STACK_MIXERS or Q4K_STACK_PERSISTENT");
    const bool mixers = d->flags == Q4K_STACK_MIXERS;
    const bool persistent = d->flags == Q4K_STACK_PERSISTENT;
    if (persistent && d->spin_limit < 0) return fail(Q4K_EINVAL, "spin_limit must be >= 0");
    if (d->n_layers < 0 || d->hidden <= 0 || d->hidden % 256 != 0)
        return fail(Q4K_ESHAPE, "need n_layers >= 0 and hidden a positive multiple of 256");
    if (d->n_layers > 0 && !d->layers) return fail(Q4K_EINVAL, "NULL layers");
    if (!(d->eps >= 0.0f)) return fail(Q4K_EINVAL, "eps must be >= 0");
    if (mixers && d->n_layers > 0 && !d->mixers) return fail(Q4K_EINVAL, "NULL mixers");
    const int64_t H = d->hidden;
    int rc;
    bool any_attn = false;
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
        if (mixers) {
            if ((rc = check_mixer(L, d->mixers[l], l))) return rc;
            any_attn |= L.kind == 1;
        }
    }
    if (mixers && any_attn && (d->attn_capacity <= 0 || d->attn_capacity > ((int64_t)1 << 24)))
        return fail(Q4K_ESHAPE, "attn_capacity must be in 1..2^24");
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
    s->mixers = mixers;
    s->persistent = persistent;
    if (persistent) {
        if (d->spin_limit > 0) s->spin = d->spin_limit;
        if ((rc = stack_groups(&s->pgroups))) {
            delete s;
            return rc;
        }
    }
    if (mixers) {
        s->mix.assign(d->mixers, d->mixers + d->n_layers);
        s->cap = d->attn_capacity;
    }

    // arena layout
    size_t off = 0, sqo = 0, sto = 0, scratch = 0;
    auto take = [](size_t &o, int64_t n) {
        const int64_t r = (int64_t)o;
        o += (size_t)((n + 63) / 64 * 64);  // keep every buffer 256-byte aligned
        return r;
    };
    size_t max_partials = 0, max_counters = 0;
    auto need = [&](int64_t M, int64_t K, int nmat, int epi) {
        GemvLaunch L = choose_gemv_launch(M, K, 1, nmat, epi);
        if (persistent) L.ks = s->pgroups;  // every node spans the whole grid
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
        s->off_o.push_back(mixers ? take(off, L.mix_out.K) : -1);
        s->sq_u.push_back(take(sqo, tiles_of(L.mix_in.M)));
        s->sq_hmid.push_back(take(sqo, tiles_of(H)));
        s->sq_a.push_back(take(sqo, tiles_of(L.gate.M)));
        s->sq_o.push_back(mixers ? take(sqo, tiles_of(L.mix_out.K)) : -1);
        if (mixers && L.kind == 0) {
            const q4k_gdn_params &g = s->mix[l].gdn;
            const int64_t C = (int64_t)(2 * g.key_heads + g.value_heads) * MD;
            s->st_a.push_back(take(sto, 3 * C));
            s->st_b.push_back(take(sto, (int64_t)g.value_heads * MD * MD));
            scratch = std::max(scratch, gdn_scratch_floats(g.key_heads, g.value_heads));
        } else if (mixers) {
            const q4k_attn_params &a = s->mix[l].attn;
            const int64_t n = (int64_t)a.kv_heads * s->cap * AHD;
            s->st_a.push_back(take(sto, n));
            s->st_b.push_back(take(sto, n));
            scratch = std::max(scratch, attn_scratch_floats(a.q_heads, a.kv_heads, s->cap));
        } else {
            s->st_a.push_back(-1);
            s->st_b.push_back(-1);
        }
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
    s->state_floats = sto;

    bool ok = hipMalloc(&s->arena, off * sizeof(float)) == hipSuccess &&
              hipMalloc(&s->sq, sqo * sizeof(float)) == hipSuccess;
    if (ok && mixers) {
        ok = (sto == 0 || hipMalloc(&s->states, sto * sizeof(float)) == hipSuccess) &&
             hipMalloc(&s->mix_scratch, std::max<size_t>(scratch, 64) * sizeof(float)) ==
                 hipSuccess &&
             hipMalloc(&s->mix_cnt, kMixCounters * sizeof(unsigned)) == hipSuccess &&
             hipMalloc(&s->pos_dev, sizeof(int64_t)) == hipSuccess;
    }
    if (!ok) {
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
        (s->states && hipMemset(s->states, 0, sto * sizeof(float)) != hipSuccess) ||
        (s->pos_dev && hipMemset(s->pos_dev, 0, sizeof(int64_t)) != hipSuccess) ||
        (s->mix_cnt && hipMemset(s->mix_cnt, 0, kMixCounters * sizeof(unsigned)) != hipSuccess) ||
        hipDeviceSynchronize() != hipSuccess) {
        release(s);
        return fail(Q4K_EHIP, "decode stack: arena clear failed");
    }

    if (persistent) {
        // node descriptors built once on the host, then uploaded; counters
        // and the error word start at zero
        std::vector<uint8_t> pn;
        int64_t nodes = 0;
        if ((rc = enqueue_token(s, nullptr, &nodes, &pn))) {
            release(s);
            return rc;
        }
        const size_t sync_bytes = ((size_t)nodes * kStackSyncLanes + 1) * sizeof(unsigned);
        if (hipMalloc(&s->pnodes, pn.size()) != hipSuccess ||
            hipMalloc(&s->psync, sync_bytes) != hipSuccess) {
            (void)hipGetLastError();
            release(s);
            return fail(Q4K_ENOMEM, "decode stack: node table allocation failed");
        }
        if (hipMemcpy(s->pnodes, pn.data(), pn.size(), hipMemcpyHostToDevice) != hipSuccess ||
            hipMemset(s->psync, 0, sync_bytes) != hipSuccess ||
            hipDeviceSynchronize() != hipSuccess) {
            release(s);
            return fail(Q4K_EHIP, "decode stack: node table upload failed");
        }
        s->n_nodes = nodes;
        *out = s;
        return Q4K_OK;
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
        rc = enqueue_token(s, cs, &nodes, nullptr);
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
    if (s->mixers && s->cap > 0 && s->host_pos >= s->cap)
        return fail(Q4K_EINVAL, "attention cache full (%lld positions): q4k_decode_stack_reset",
                    (long long)s->cap);
    hipStream_t st = (hipStream_t)stream;
    Q4K_HIP(hipMemcpyAsync(s->arena + s->off_h[0], h_in, (size_t)s->hidden * sizeof(float),
                           hipMemcpyDeviceToDevice, st));
    if (s->persistent) {
        const int rc = launch_stack_kernel(s->pnodes, (int)s->n_nodes, s->psync, s->epoch,
                                           s->psync + s->n_nodes * kStackSyncLanes, s->spin,
                                           s->pgroups, st);
        if (rc) return rc;
        ++s->epoch;
    } else {
        Q4K_HIP(hipGraphLaunch(s->exec, st));
    }
    if (logits)
        Q4K_HIP(hipMemcpyAsync(logits, s->arena + s->off_logits,
                               (size_t)s->lm_head.M * sizeof(float), hipMemcpyDeviceToDevice, st));
    ++s->host_pos;
    return Q4K_OK;
}

int q4k_decode_stack_reset(q4k_stack *s, void *stream) {
    clear_error();
    if (!s) return fail(Q4K_EINVAL, "NULL plan");
    return zero_states(s, (hipStream_t)stream);
}

int q4k_decode_stack_position(q4k_stack *s, int64_t *pos) {
    clear_error();
    if (!s || !pos) return fail(Q4K_EINVAL, "NULL argument");
    *pos = s->host_pos;
    return Q4K_OK;
}

int q4k_decode_stack_status(q4k_stack *s, void *stream, int32_t *status) {
    clear_error();
    if (!s || !status) return fail(Q4K_EINVAL, "NULL argument");
    *status = 0;
    if (!s->persistent) return Q4K_OK;
    hipStream_t st = (hipStream_t)stream;
    unsigned word = 0;
    Q4K_HIP(hipStreamSynchronize(st));
    unsigned *errw = s->psync + s->n_nodes * kStackSyncLanes;
    Q4K_HIP(hipMemcpy(&word, errw, sizeof word, hipMemcpyDeviceToHost));
    if (word) {
        // A workgroup that gave up may have run into the next node while its
        // tiles were still being finished, leaving split-tile counters off
        // zero: clear them with the record, so later tokens are sound.
        Q4K_HIP(hipMemset(errw, 0, sizeof word));
        Q4K_HIP(hipMemset(s->ws.counters, 0, kCounterBytes));
    }
    Q4K_HIP(hipDeviceSynchronize());
    *status = word ? 1 : 0;
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
    if (which >= Q4K_BUF_MIX && !s->mixers) return fail(Q4K_EINVAL, "plan has no mixers");
    const int kind = which >= Q4K_BUF_MIX ? s->layers[layer].kind : -1;
    switch (which) {
        case Q4K_BUF_H: *ptr = s->arena + s->off_h[layer]; *n = s->hidden; break;
        case Q4K_BUF_U: *ptr = s->arena + s->off_u[layer]; *n = s->layers[layer].mix_in.M; break;
        case Q4K_BUF_HMID: *ptr = s->arena + s->off_hmid[layer]; *n = s->hidden; break;
        case Q4K_BUF_G: *ptr = s->arena + s->off_g[layer]; *n = s->layers[layer].gate.M; break;
        case Q4K_BUF_V: *ptr = s->arena + s->off_v[layer]; *n = s->layers[layer].gate.M; break;
        case Q4K_BUF_A: *ptr = s->arena + s->off_a[layer]; *n = s->layers[layer].gate.M; break;
        case Q4K_BUF_MIX:
            *ptr = s->arena + s->off_o[layer];
            *n = s->layers[layer].mix_out.K;
            break;
        case Q4K_BUF_CONV_STATE:
        case Q4K_BUF_GDN_STATE: {
            if (kind != 0) return fail(Q4K_EINVAL, "layer %d is not a GDN layer", layer);
            const q4k_gdn_params &g = s->mix[layer].gdn;
            const int64_t C = (int64_t)(2 * g.key_heads + g.value_heads) * MD;
            if (which == Q4K_BUF_CONV_STATE) {
                *ptr = s->states + s->st_a[layer];
                *n = 3 * C;
            } else {
                *ptr = s->states + s->st_b[layer];
                *n = (int64_t)g.value_heads * MD * MD;
            }
            break;
        }
        case Q4K_BUF_K_CACHE:
        case Q4K_BUF_V_CACHE:
            if (kind != 1) return fail(Q4K_EINVAL, "layer %d is not an attention layer", layer);
            *ptr = s->states + (which == Q4K_BUF_K_CACHE ? s->st_a[layer] : s->st_b[layer]);
            *n = (int64_t)s->mix[layer].attn.kv_heads * s->cap * AHD;
            break;
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
