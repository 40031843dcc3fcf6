// q4k_mixer.hip — the two token mixers of the hybrid model for one decode
// token, on the GPU: the Gated DeltaNet recurrence and gated full attention.
//
// "Qwen3.6-27B on Apple M3 Pro — the llama.cpp parity bar", architecture
// list: Gated DeltaNet layers with a depthwise causal conv of kernel 4, 16
// key heads and 48 value heads of 128, swish output gate, f32 recurrent
// state; full-attention layers with 24 query and 4 key/value heads of 256,
// output gate, partial rotary over a quarter of each head, theta 1e7, q/k
// RMSNorm in the (1 + w) form.  The decode profile of "Mac Qwen3.6-27B Metal
// Q4_K perf diagnosis" (§2) puts the recurrence at 5.9% of a token and the
// attention, conv, norms and gates at 6.8%; §4 asks for them on the device so
// that a token is one submission.
//
// Gated DeltaNet step (per token; u = [q | k | v | z | b | a]), one kernel,
// gdn_step_kernel, four workgroups per value head:
//   conv         — silu of the 4-tap causal conv over (state, input) of the
//                  q and k channels of the head's key head and of the v
//                  channels of the workgroup's rows, the conv state shifted
//                  once per channel; beta = sigmoid(b) and
//                  alpha = exp(-exp(A_log) softplus(a + dt_bias));
//   recurrence   — q and k L2-normalised (q also by 1/sqrt(128)); on the
//                  workgroup's 32 rows of the head's 128 x 128 state
//                  (value-dimension major, S[dv][dk]) S <- alpha S,
//                  delta = beta (v - S^T k), S <- S + k delta^T, o = S^T q.
//                  Thread t holds float4 t + 256 m of the slice: rows
//                  t/32 + 8m, key dims 4 (t%32) .. +3, so every load and
//                  store instruction moves 4 KB of contiguous state and each
//                  row's dot products reduce over the 32 lanes that hold it;
//   gated norm   — out = norm_w * o / rms(o) * silu(z) over the head's 128
//                  outputs, by the last of its four workgroups.
// Gated attention step (position pos; u = [per head: q | gate] x Hq, k, v):
//   attn_chunk_kernel   — (1 + w) RMSNorm and rotary (first R dims, angle
//                         and its reduction in double) of q and k, k and v
//                         written to the cache at
//                         pos, then a split-KV online softmax over chunks of
//                         positions, each key/value row read once per group
//                         of query heads that share it;
//   attn_combine_kernel — merges the chunks per query head, sigmoid gate.
#include "q4k_device.hpp"
#include "q4k_internal.hpp"

#include <algorithm>

#include <math.h>

namespace q4k {
namespace {

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + expf(-x)); }
__device__ __forceinline__ float siluf_(float x) { return x / (1.0f + expf(-x)); }
__device__ __forceinline__ float softplusf_(float x) { return x > 30.f ? x : log1pf(expf(x)); }

// Cross-lane steps through DPP (no LDS round trip, unlike __shfl_xor):
// quad_perm [1,0,3,2] = lane ^ 1, [2,3,0,1] = lane ^ 2, row_half_mirror =
// lane 7 - i within each 8 lanes, row_mirror = lane 15 - i within each 16.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_f(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
// sum over each group of 8 lanes (8i .. 8i+7), in every lane of the group
__device__ __forceinline__ float sum8_dpp(float v) {
    v += dpp_f<0xB1>(v);
    v += dpp_f<0x4E>(v);
    v += dpp_f<0x141>(v);
    return v;
}
// sum / maximum over the wave, in every lane: groups of 16 by DPP, then the
// four groups' values read out in a fixed order
__device__ __forceinline__ float wave_sum_dpp(float v) {
    v = sum8_dpp(v);
    v += dpp_f<0x140>(v);
    return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}
__device__ __forceinline__ float wave_max_dpp(float v) {
    v = fmaxf(v, dpp_f<0xB1>(v));
    v = fmaxf(v, dpp_f<0x4E>(v));
    v = fmaxf(v, dpp_f<0x141>(v));
    v = fmaxf(v, dpp_f<0x140>(v));
    return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}

// sum over the 32 lanes of each half-wave (every lane ends with its half's sum)
__device__ __forceinline__ float half_sum32(float v) {
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 8);
    v += __shfl_xor(v, 4);
    v += __shfl_xor(v, 2);
    v += __shfl_xor(v, 1);
    return v;
}

// Workgroup barrier for hand-offs through LDS only: it waits for this
// wave's LDS (and scalar) operations, not for its global loads in flight,
// which __syncthreads() would also drain.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Block (256 threads) sum; every thread gets the total.  red: 4 floats of LDS.
__device__ __forceinline__ float block_sum256(float v, float *red) {
    v = wave_sum_dpp(v);
    const int w = threadIdx.x >> 6;
    lds_barrier();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    lds_barrier();
    return (red[0] + red[1]) + (red[2] + red[3]);
}

constexpr int GD = 128;  // key and value head dimension of the recurrence

// One GDN decode step in one kernel.  The recurrence of a value head is
// independent per row dv of its state, so each head's 128 rows are split over
// GRS workgroups (GRR rows each, 16 KB of state): 4 x 48 = 192 workgroups for
// the model's 48 heads.  Each workgroup
//   * issues its state loads first;
//   * forms the causal conv + SiLU of the q and k channels of its key head
//     (256 channels, one per thread) and of the v channels of its rows from
//     the old conv state, and beta and the decay of its head;
//   * L2-normalises q and k and runs the delta rule on its rows;
//   * publishes its rows' outputs with device-coherent stores and counts
//     itself in on the head's arrival counter; the last of the GRS applies
//     the gated RMSNorm (in a fixed order, whoever arrives last) and resets
//     the counter.
// Conv state: a v channel is read by one workgroup only, which shifts it in
// place.  A q or k channel is read by the GRS workgroups of every value head
// of its key head; each counts itself in on the key head's counter after its
// reads have returned, and the last one shifts those 256 channels' state and
// resets the counter, so no workgroup reads a state another has shifted.
constexpr int GRS = 4;         // workgroups per value head
constexpr int GRR = GD / GRS;  // state rows per workgroup

__device__ __forceinline__ float conv4(const float4 w, float s0, float s1, float s2, float x) {
    return siluf_(fmaf(w.w, x, fmaf(w.z, s2, fmaf(w.y, s1, w.x * s0))));
}

__global__ __launch_bounds__(256) void gdn_step_kernel(
    const float *__restrict__ u, const float *__restrict__ conv_w, float *conv_state, int Hk,
    int Hv, const float *__restrict__ a_log, const float *__restrict__ dt_bias,
    const float *__restrict__ norm_w, float eps, float *__restrict__ S, float *__restrict__ out,
    float *__restrict__ out_sq, float *obuf, unsigned *cnt_v, unsigned *cnt_k) {
    __shared__ float kq[2][GD];
    __shared__ float vv[GRR];
    __shared__ float ov[GRR];
    __shared__ float gab[2];
    __shared__ float red[4];
    __shared__ unsigned last_s;
    const int h = blockIdx.x / GRS, part = blockIdx.x - h * GRS, t = threadIdx.x;
    const int rep = Hv / Hk, j = h / rep;  // key head of this value head
    const int64_t nq = (int64_t)Hk * GD;
    // this workgroup's state rows: their loads fly while the inputs are formed
    // thread t holds key dims 8 (t % 16) .. +7 of rows t / 16 + 16 m of the
    // slice (two float4 per row): every load instruction pair moves 2 KB of
    // contiguous state, and a row's dot products reduce over 16 lanes
    float4 *Sh = reinterpret_cast<float4 *>(S + ((int64_t)h * GD + part * GRR) * GD);
    constexpr int NM = GRR / 16;  // rows per thread
    float4 s[NM][2];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        s[m][0] = Sh[2 * t + 512 * m];
        s[m][1] = Sh[2 * t + 1 + 512 * m];
    }
    // conv of the q (threads 0..127) and k (128..255) channels of key head j
    const int64_t chqk = t < GD ? (int64_t)j * GD + t : nq + (int64_t)j * GD + (t - GD);
    const float4 wqk = *reinterpret_cast<const float4 *>(conv_w + 4 * chqk);
    const float q0 = conv_state[3 * chqk], q1 = conv_state[3 * chqk + 1],
                q2 = conv_state[3 * chqk + 2], xqk = u[chqk];
    const float qk = conv4(wqk, q0, q1, q2, xqk);
    // conv of the v channels of this workgroup's rows (their only reader)
    if (t < GRR) {
        const int64_t ch = 2 * nq + (int64_t)h * GD + part * GRR + t;
        const float4 w = *reinterpret_cast<const float4 *>(conv_w + 4 * ch);
        float *st = conv_state + 3 * ch;
        const float v0 = st[0], v1 = st[1], v2 = st[2], x = u[ch];
        vv[t] = conv4(w, v0, v1, v2, x);
        st[0] = v1;
        st[1] = v2;
        st[2] = x;
    }
    if (t == 0) {
        const int64_t off = 2 * nq + 2 * (int64_t)Hv * GD;  // b after q, k, v and z
        const float b = u[off + h], a = u[off + Hv + h];
        gab[0] = sigmoidf_(b);
        gab[1] = expf(-expf(a_log[h]) * softplusf_(a + dt_bias[h]));
    }
    // L2 norms of q and k
    float ssq = t < GD ? qk * qk : 0.f, ssk = t < GD ? 0.f : qk * qk;
    ssq = block_sum256(ssq, red);
    ssk = block_sum256(ssk, red);
    if (t < GD) kq[1][t] = qk / sqrtf(ssq + eps) / sqrtf((float)GD);
    else kq[0][t - GD] = qk / sqrtf(ssk + eps);
    lds_barrier();
    // every thread's conv-state reads have returned (their values are used
    // above): count in on the key head now; the answer (is this the last
    // reader, which shifts the state?) is only needed at the end
    unsigned k_old = 0;
    if (t == 0)
        k_old = __hip_atomic_fetch_add(&cnt_k[j], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const float alpha = gab[1], beta = gab[0];
    const int lane16 = t & 15, row0 = t >> 4;
    const float4 k0 = *reinterpret_cast<const float4 *>(&kq[0][8 * lane16]);
    const float4 k1 = *reinterpret_cast<const float4 *>(&kq[0][8 * lane16 + 4]);
    const float4 q0v = *reinterpret_cast<const float4 *>(&kq[1][8 * lane16]);
    const float4 q1v = *reinterpret_cast<const float4 *>(&kq[1][8 * lane16 + 4]);
    auto dot8 = [](const float4 &a0, const float4 &a1, const float4 &b0, const float4 &b1) {
        return fmaf(a0.x, b0.x, fmaf(a0.y, b0.y, fmaf(a0.z, b0.z, fmaf(a0.w, b0.w,
               fmaf(a1.x, b1.x, fmaf(a1.y, b1.y, fmaf(a1.z, b1.z, a1.w * b1.w)))))));
    };
    auto axpy4 = [](float4 &r, const float4 &k, float d) {
        r.x = fmaf(k.x, d, r.x);
        r.y = fmaf(k.y, d, r.y);
        r.z = fmaf(k.z, d, r.z);
        r.w = fmaf(k.w, d, r.w);
    };
    auto scale4 = [](float4 &r, float a) {
        r.x *= a;
        r.y *= a;
        r.z *= a;
        r.w *= a;
    };
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        const int dv = row0 + 16 * m;  // row within this workgroup's slice
        float4 r0 = s[m][0], r1 = s[m][1];
        scale4(r0, alpha);
        scale4(r1, alpha);
        float kv = dot8(r0, r1, k0, k1);
        kv = sum8_dpp(kv);
        kv += dpp_f<0x140>(kv);  // sum over the row's 16 lanes
        const float delta = beta * (vv[dv] - kv);
        axpy4(r0, k0, delta);
        axpy4(r1, k1, delta);
        float o = dot8(r0, r1, q0v, q1v);
        o = sum8_dpp(o);
        o += dpp_f<0x140>(o);
        if (lane16 == 0) ov[dv] = o;
        s[m][0] = r0;
        s[m][1] = r1;
    }
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        Sh[2 * t + 512 * m] = s[m][0];
        Sh[2 * t + 1 + 512 * m] = s[m][1];
    }
    lds_barrier();
    float *ob = obuf + (int64_t)h * GD;
    if (t < GRR)
        __hip_atomic_store(&ob[part * GRR + t], ov[t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's stores have completed
    lds_barrier();
    if (t == 0) {
        const bool v_last = __hip_atomic_fetch_add(&cnt_v[h], 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT) == (unsigned)(GRS - 1);
        const bool k_last = k_old == (unsigned)(rep * GRS - 1);
        last_s = (v_last ? 1u : 0u) | (k_last ? 2u : 0u);
    }
    lds_barrier();
    if (last_s & 2u) {  // the last reader of key head j's q and k channels
        float *st = conv_state + 3 * chqk;
        st[0] = q1;
        st[1] = q2;
        st[2] = xqk;
        if (t == 0) __hip_atomic_store(&cnt_k[j], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (!(last_s & 1u)) return;
    if (t == 0) __hip_atomic_store(&cnt_v[h], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // gated RMSNorm of the head's output
    const float o = t < GD ? __hip_atomic_load(&ob[t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                           : 0.f;
    const float ms = block_sum256(o * o, red);
    if (t < GD) {
        const float inv = 1.0f / sqrtf(ms / (float)GD + eps);
        const int64_t zo = 2 * nq + (int64_t)Hv * GD + (int64_t)h * GD + t;  // z after q, k, v
        const float val = norm_w[t] * (o * inv) * siluf_(u[zo]);
        out[(int64_t)h * GD + t] = val;
        if (out_sq) {
            // sums of squares of 32-element granules, added as the plain
            // sum-of-squares kernel adds them
            const float sq = half_sum32(val * val);
            if ((t & 31) == 0) out_sq[(int64_t)h * (GD / 32) + (t >> 5)] = sq;
        }
    }
}

constexpr int AD = 256;  // attention head dimension

// Split-KV decode attention, two kernels.
//
// attn_chunk_kernel: the positions 0..pos are cut into chunks of ACH;
// workgroup (g, head group, w) takes chunks w, w + nw, ... of key/value head
// g for a group of the query heads that read it (at most AHG, evened out),
// so every key and value row is read once per head group rather than once
// per query head.
//   set-up: (1 + w) RMSNorm and rotary of the group's queries into LDS (the
//           rotary angle once per thread for all heads: frequency from the
//           host, product and reduction modulo 2 pi in double); the
//           workgroup whose chunks hold pos also forms that position's key
//           and value (the first head group writes them to the caches) and
//           uses its own copy wherever the chunk reads row pos, so no other
//           workgroup depends on that write;
//   scores: wave v takes the chunk's positions 16v .. 16v+15; one load
//           instruction covers 8 whole 1 KB key rows (8 lanes per row, 16 B
//           each) and 16 of them cover the wave's rows; 8-lane DPP sums finish
//           the dot products;
//   softmax: wave v keeps the running max and sum of head v (lane i
//           position i);
//   values: lane l holds dims 4l .. 4l+3, wave v positions 16v .. 16v+15
//           (a value row is one 1 KB load), issued before the scores so
//           they arrive during the scores and the softmax;
//           outputs rescaled whenever the running max moves.
// It writes (output, max, sum) per head, or nothing if it had no chunk.
// attn_combine_kernel: one workgroup per query head merges the chunk
// workgroups in index order and applies the sigmoid gate.  Deterministic:
// fixed chunk assignment and merge order.
constexpr int ACH = 64;  // positions per chunk
constexpr int AHG = 4;   // at most this many query heads per chunk workgroup

// Query heads of a key/value head split into hg groups of hpw (the last may
// be smaller): as few groups of at most AHG heads as possible, evened out
// (6 heads: two groups of 3).
__host__ __device__ inline void attn_head_groups(int rep, int &hpw, int &hg) {
    const int ng = (rep + AHG - 1) / AHG;
    hpw = (rep + ng - 1) / ng;
    hg = (rep + hpw - 1) / hpw;
}
constexpr int APS = AD + 4;  // partial record: 256 outputs, max, sum, 2 pad (16 B rows)

// Rotary frequencies theta^(-2i/R), i < R/2, computed on the host in double.
struct RopeTable {
    double f[AD / 2];
};

__global__ __launch_bounds__(256) void attn_chunk_kernel(
    const float *__restrict__ u, const float *__restrict__ qw, const float *__restrict__ kw,
    float *__restrict__ kc, float *__restrict__ vc, int64_t cap, int64_t pos_val,
    const int64_t *__restrict__ pos_dev, int Hq, int Hkv, int R, const RopeTable rope, float eps,
    int nw, float *__restrict__ part) {
    __shared__ __attribute__((aligned(16))) float qs[AHG][AD];
    __shared__ __attribute__((aligned(16))) float kn[AD];
    __shared__ __attribute__((aligned(16))) float vn[AD];
    __shared__ float sc[AHG][ACH];
    __shared__ float pr[AHG][ACH];
    __shared__ float red[AHG + 1][4];
    __shared__ float ms[AHG], ls[AHG], rs[AHG];
    __shared__ __attribute__((aligned(16))) float oacc[4][AHG][AD];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rep = Hq / Hkv;
    int hpw, hg;
    attn_head_groups(rep, hpw, hg);
    const int wi = blockIdx.x % nw, gg = blockIdx.x / nw;  // gg = g * hg + head group
    const int g = gg / hg, hgi = gg % hg;
    const int h0 = g * rep + hgi * hpw, nh = min(hpw, rep - hgi * hpw);
    const int64_t pos = pos_dev ? *pos_dev : pos_val;
    if (pos < 0 || pos >= cap) return;  // the callers keep pos inside the cache
    const int64_t nchunks = pos / ACH + 1, cpos = pos / ACH;
    if (wi >= nchunks) return;  // no chunk: the merge reads min(nw, nchunks) partials
    const bool own_pos = cpos % nw == wi;

    const float *kg = kc + (int64_t)g * cap * AD, *vg = vc + (int64_t)g * cap * AD;
    const int sub = lane & 7, rsub = lane >> 3;  // 16 B piece, row within 8
    // every key and value load of the wave's 16 rows of chunk c: key row
    // tw + 8 (j & 1) + rsub, dims 32 (j >> 1) + 4 sub .. +3; value row tw + i,
    // dims 4 lane .. +3 (rows past pos read row pos, replaced below)
    float4 k4[16], v4[16];
    auto issue_k = [&](int64_t c) {
        const int64_t tw = c * ACH + 16 * wv;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int64_t t = tw + 8 * (j & 1) + rsub;
            k4[j] = *reinterpret_cast<const float4 *>(kg + min(t, pos) * AD + 32 * (j >> 1) +
                                                      4 * sub);
        }
    };
    auto issue_v = [&](int64_t c) {
        const int64_t tw = c * ACH + 16 * wv;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            v4[i] = *reinterpret_cast<const float4 *>(vg + min(tw + i, pos) * AD + 4 * lane);
    };
    issue_k(wi);  // the first chunk's keys fly during the set-up

    // ---- set-up: normed, rotated queries (and key, value at pos)
    {
        const int d = tid;
        const int64_t ko = (int64_t)Hq * 2 * AD + (int64_t)g * AD;
        const int64_t vo = (int64_t)Hq * 2 * AD + (int64_t)Hkv * AD + (int64_t)g * AD;
        float x[AHG + 1];
#pragma unroll
        for (int hh = 0; hh < AHG; ++hh) x[hh] = hh < nh ? u[(int64_t)(h0 + hh) * 2 * AD + d] : 0.f;
        x[AHG] = own_pos ? u[ko + d] : 0.f;
        // rotary angle pos * theta^(-2i/R) in double (the frequencies come
        // from the host), reduced modulo 2 pi in double, then sine and cosine
        // of the reduced angle in single precision
        float cs = 1.f, sn = 0.f;
        const int half = R / 2;
        if (d < R) {
            const int i = d < half ? d : d - half;
            const double ang = (double)pos * rope.f[i];
            const double nt = rint(ang * 0.15915494309189535);         // turns: ang / (2 pi)
            double red2 = fma(-nt, 6.283185307179586, ang);            // 2 pi, leading part
            red2 = fma(-nt, 2.4492935982947064e-16, red2);             // 2 pi, the rest
            sincosf((float)red2, &sn, &cs);
        }
#pragma unroll
        for (int hh = 0; hh <= AHG; ++hh) {
            const float ssq = wave_sum_dpp(x[hh] * x[hh]);
            if (lane == 0) red[hh][wv] = ssq;
        }
        lds_barrier();
        float n[AHG + 1];
#pragma unroll
        for (int hh = 0; hh <= AHG; ++hh) {
            const float ss = (red[hh][0] + red[hh][1]) + (red[hh][2] + red[hh][3]);
            const float wgt = hh < AHG ? qw[d] : kw[d];
            n[hh] = x[hh] / sqrtf(ss / (float)AD + eps) * (1.0f + wgt);
            if (hh < AHG) qs[hh][d] = n[hh];
            else kn[d] = n[hh];
        }
        lds_barrier();
        float r[AHG + 1];
#pragma unroll
        for (int hh = 0; hh <= AHG; ++hh) {
            const float *row = hh < AHG ? qs[hh] : kn;
            r[hh] = n[hh];
            if (d < R) r[hh] = d < half ? n[hh] * cs - row[d + half] * sn
                                        : n[hh] * cs + row[d - half] * sn;
        }
        lds_barrier();
#pragma unroll
        for (int hh = 0; hh < AHG; ++hh) qs[hh][d] = r[hh];
        if (own_pos) {
            const float v = u[vo + d];
            kn[d] = r[AHG];
            vn[d] = v;
            if (hgi == 0) {
                kc[((int64_t)g * cap + pos) * AD + d] = r[AHG];
                vc[((int64_t)g * cap + pos) * AD + d] = v;
            }
        }
        if (tid < AHG) {
            ms[tid] = -INFINITY;
            ls[tid] = 0.f;
        }
        lds_barrier();
    }

    float o[AHG][4];
#pragma unroll
    for (int hh = 0; hh < AHG; ++hh) o[hh][0] = o[hh][1] = o[hh][2] = o[hh][3] = 0.f;
    const float scale = 1.0f / sqrtf((float)AD);
    for (int64_t c = wi;;) {
        const int64_t tw = c * ACH + 16 * wv;  // this wave's first position
        issue_v(c);  // the values fly during the scores and the softmax
        // rows at or past pos: the key and value formed above (past pos the
        // score is masked and the weight is zero, so they only have to be finite)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int64_t t = tw + 8 * (j & 1) + rsub;
            if (t >= pos) k4[j] = *reinterpret_cast<const float4 *>(&kn[32 * (j >> 1) + 4 * sub]);
        }
        // scores: lane (rsub, sub) sums dims 32 m + 4 sub .. +3 (m = 0..7) of
        // rows tw + rsub and tw + 8 + rsub, then 8-lane sums
#pragma unroll
        for (int hh = 0; hh < AHG; ++hh) {
            float a0 = 0.f, a1 = 0.f;
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const float4 q4 = *reinterpret_cast<const float4 *>(&qs[hh][32 * m + 4 * sub]);
                const float4 ka = k4[2 * m], kb = k4[2 * m + 1];
                a0 = fmaf(q4.x, ka.x, fmaf(q4.y, ka.y, fmaf(q4.z, ka.z, fmaf(q4.w, ka.w, a0))));
                a1 = fmaf(q4.x, kb.x, fmaf(q4.y, kb.y, fmaf(q4.z, kb.z, fmaf(q4.w, kb.w, a1))));
            }
            a0 = sum8_dpp(a0);
            a1 = sum8_dpp(a1);
            if (sub == 0) {
                sc[hh][16 * wv + rsub] = a0;
                sc[hh][16 * wv + 8 + rsub] = a1;
            }
        }
        lds_barrier();
        // online softmax: wave wv takes heads wv and wv + 4, lane = position
        const int64_t t0 = c * ACH;
#pragma unroll
        for (int k2 = 0; k2 < (AHG + 3) / 4; ++k2) {
            const int hh = wv + 4 * k2;
            if (hh >= AHG) break;
            if (hh < nh) {
                const bool ok = t0 + lane <= pos;
                const float s = ok ? sc[hh][lane] * scale : -INFINITY;
                const float mo = ms[hh];
                const float mn = fmaxf(mo, wave_max_dpp(s));
                const float pv = ok ? expf(s - mn) : 0.f;
                const float ssum = wave_sum_dpp(pv);
                pr[hh][lane] = pv;
                if (lane == 0) {
                    const float rr = expf(mo - mn);  // 0 while nothing was seen (mo = -inf)
                    rs[hh] = rr;
                    ms[hh] = mn;
                    ls[hh] = fmaf(ls[hh], rr, ssum);
                }
            } else {
                pr[hh][lane] = 0.f;
                if (lane == 0) rs[hh] = 1.f;
            }
        }
        lds_barrier();
        // values: rescale, then add this wave's 16 rows
        if (tw + 15 >= pos) {
            const float4 vp = *reinterpret_cast<const float4 *>(&vn[4 * lane]);
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (tw + i >= pos) v4[i] = vp;
        }
#pragma unroll
        for (int hh = 0; hh < AHG; ++hh) {
            const float rr = rs[hh];
            o[hh][0] *= rr;
            o[hh][1] *= rr;
            o[hh][2] *= rr;
            o[hh][3] *= rr;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float pv = pr[hh][16 * wv + i];
                o[hh][0] = fmaf(pv, v4[i].x, o[hh][0]);
                o[hh][1] = fmaf(pv, v4[i].y, o[hh][1]);
                o[hh][2] = fmaf(pv, v4[i].z, o[hh][2]);
                o[hh][3] = fmaf(pv, v4[i].w, o[hh][3]);
            }
        }
        lds_barrier();  // sc, pr and rs are rewritten by the next chunk
        c += nw;
        if (c >= nchunks) break;
        issue_k(c);
    }
    // the four waves' outputs, then (output, max, sum) per head
#pragma unroll
    for (int hh = 0; hh < AHG; ++hh)
        *reinterpret_cast<float4 *>(&oacc[wv][hh][4 * lane]) =
            make_float4(o[hh][0], o[hh][1], o[hh][2], o[hh][3]);
    lds_barrier();
    float *pw = part + (int64_t)blockIdx.x * AHG * APS;
#pragma unroll
    for (int hh = 0; hh < AHG; ++hh) {
        if (hh < nh) {
            pw[hh * APS + tid] = (oacc[0][hh][tid] + oacc[1][hh][tid]) +
                                 (oacc[2][hh][tid] + oacc[3][hh][tid]);
            if (tid == 0) {
                pw[hh * APS + AD] = ms[hh];
                pw[hh * APS + AD + 1] = ls[hh];
            }
        }
    }
}

__global__ __launch_bounds__(256) void attn_combine_kernel(
    const float *__restrict__ u, const float *__restrict__ part, int64_t cap, int64_t pos_val,
    const int64_t *__restrict__ pos_dev, int Hq, int Hkv, int nw, float *__restrict__ out,
    float *__restrict__ out_sq) {
    __shared__ float cw[64];
    __shared__ float den_s;
    __shared__ __attribute__((aligned(16))) float acc[4][AD];
    const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t pos = pos_dev ? *pos_dev : pos_val;
    if (pos < 0 || pos >= cap) return;
    const int rep = Hq / Hkv;
    int hpw, hg;
    attn_head_groups(rep, hpw, hg);
    const int g = h / rep, hr = h - g * rep, hgi = hr / hpw, hh = hr - hgi * hpw;
    const int nact = (int)min<int64_t>(nw, pos / ACH + 1);  // nw <= 64
    const float *pb = part + ((int64_t)(g * hg + hgi) * nw * AHG + hh) * APS;
    const int64_t stride = (int64_t)AHG * APS;  // one chunk workgroup
    // outputs first: wave wv loads chunk workgroups wv, wv + 4, ... (lane l
    // dims 4l .. 4l+3), all loads in flight together
    float4 ov[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int w = wv + 4 * i;
        ov[i] = w < nact ? *reinterpret_cast<const float4 *>(pb + w * stride + 4 * lane)
                         : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    // merge weights exp(m_w - M) and the denominator, lane w of wave 0
    if (wv == 0) {
        const bool ok = lane < nact;
        const float m = ok ? pb[lane * stride + AD] : -INFINITY;
        const float l = ok ? pb[lane * stride + AD + 1] : 0.f;
        const float M = wave_max_dpp(m);
        const float c = ok ? expf(m - M) : 0.f;
        cw[lane] = c;
        const float den = wave_sum_dpp(c * l);
        if (lane == 0) den_s = den;
    }
    lds_barrier();
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int w = wv + 4 * i;
        if (w < nact) {
            const float c = cw[w];
            a.x = fmaf(c, ov[i].x, a.x);
            a.y = fmaf(c, ov[i].y, a.y);
            a.z = fmaf(c, ov[i].z, a.z);
            a.w = fmaf(c, ov[i].w, a.w);
        }
    }
    *reinterpret_cast<float4 *>(&acc[wv][4 * lane]) = a;
    lds_barrier();
    const int d = tid;
    const float num = (acc[0][d] + acc[1][d]) + (acc[2][d] + acc[3][d]);
    const float gate = u[(int64_t)h * 2 * AD + AD + d];
    const float val = num / den_s * sigmoidf_(gate);
    out[(int64_t)h * AD + d] = val;
    if (out_sq) {
        // sums of squares of 32-element granules, added as the plain
        // sum-of-squares kernel adds them
        const float sq = half_sum32(val * val);
        if ((d & 31) == 0) out_sq[(int64_t)h * (AD / 32) + (d >> 5)] = sq;
    }
}

}  // namespace

int launch_gdn_step(const GdnShape &s, const float *u, const float *conv_w, const float *a_log,
                    const float *dt_bias, const float *norm_w, float *conv_state, float *S,
                    float *out, float *out_sq, float *scratch, unsigned *cnt,
                    hipStream_t stream) {
    hipLaunchKernelGGL(gdn_step_kernel, dim3((unsigned)(s.Hv * GRS)), dim3(256), 0, stream, u,
                       conv_w, conv_state, s.Hk, s.Hv, a_log, dt_bias, norm_w, s.eps, S, out,
                       out_sq, scratch, cnt, cnt + s.Hv);
    Q4K_HIP(hipGetLastError());
    return Q4K_OK;
}

size_t gdn_scratch_floats(int Hk, int Hv) {
    (void)Hk;
    return (size_t)Hv * GD;
}

size_t attn_chunk_groups(int Hq, int Hkv, int64_t cap) {
    int hpw, hg;
    attn_head_groups(Hq / Hkv, hpw, hg);
    const int64_t nw = std::max<int64_t>(1, std::min<int64_t>(64, (cap + ACH - 1) / ACH));
    return (size_t)Hkv * hg * nw;
}

size_t attn_scratch_floats(int Hq, int Hkv, int64_t cap) {
    return attn_chunk_groups(Hq, Hkv, cap) * AHG * APS;
}

int launch_attn_step(const AttnShape &s, const float *u, const float *q_norm_w,
                     const float *k_norm_w, float *k_cache, float *v_cache, int64_t cap,
                     int64_t pos, const int64_t *pos_dev, float *out, float *out_sq,
                     float *scratch, hipStream_t stream) {
    int hpw, hg;
    attn_head_groups(s.Hq / s.Hkv, hpw, hg);
    const int nw = (int)std::max<int64_t>(1, std::min<int64_t>(64, (cap + ACH - 1) / ACH));
    RopeTable rope = {};
    for (int i = 0; i < s.R / 2; ++i) rope.f[i] = pow((double)s.theta, -2.0 * i / s.R);
    hipLaunchKernelGGL(attn_chunk_kernel, dim3((unsigned)(s.Hkv * hg * nw)), dim3(256), 0, stream,
                       u, q_norm_w, k_norm_w, k_cache, v_cache, cap, pos, pos_dev, s.Hq, s.Hkv,
                       s.R, rope, s.eps, nw, scratch);
    Q4K_HIP(hipGetLastError());
    hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)s.Hq), dim3(256), 0, stream, u, scratch,
                       cap, pos, pos_dev, s.Hq, s.Hkv, nw, out, out_sq);
    Q4K_HIP(hipGetLastError());
    return Q4K_OK;
}

}  // namespace q4k
