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
// Gated DeltaNet step (per token; u = [q | k | v | z | b | a]):
//   gdn_conv_kernel   — one thread per channel of [q|k|v]: silu of the
//                       4-tap causal conv over (state, input), state shifted;
//                       the first threads also form beta = sigmoid(b) and
//                       alpha = exp(-exp(A_log) softplus(a + dt_bias)).
//   gdn_state_kernel  — one workgroup per value head: q and k of its key
//                       head L2-normalised (q also by 1/sqrt(128)), then on
//                       the head's 128 x 128 state (value-dimension major,
//                       S[dv][dk], 64 KB) S <- alpha S,
//                       delta = beta (v - S^T k), S <- S + k delta^T,
//                       o = S^T q, and the gated norm
//                       out = norm_w * o / rms(o) * silu(z).
//                       Thread t holds float4 t + 256 m (m = 0..15) of the
//                       state: rows t/32 + 8m, key dims 4 (t%32) .. +3, so
//                       every load and store instruction moves 4 KB of
//                       contiguous state, and each row's dot products reduce
//                       over the 32 lanes that hold it.
// Gated attention step (position pos; u = [per head: q | gate] x Hq, k, v):
//   attn_step_kernel  — one workgroup per query head: (1 + w) RMSNorm of q
//                       and of its key/value head's k, rotary on the first R
//                       dims (angles in double), k and v written to the cache
//                       at pos by the head's first query head, then an online
//                       softmax over positions 0..pos (four waves, positions
//                       t = w mod 4, 4 dims per lane) and the sigmoid gate.
#include "q4k_device.hpp"
#include "q4k_internal.hpp"

#include <math.h>

namespace q4k {
namespace {

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + expf(-x)); }
__device__ __forceinline__ float siluf_(float x) { return x / (1.0f + expf(-x)); }
__device__ __forceinline__ float softplusf_(float x) { return x > 30.f ? x : log1pf(expf(x)); }

__device__ __forceinline__ float wave_sum64(float v) {
    v += __shfl_xor(v, 32);
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 8);
    v += __shfl_xor(v, 4);
    v += __shfl_xor(v, 2);
    v += __shfl_xor(v, 1);
    return v;
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

// Block (256 threads) sum; every thread gets the total.  red: 4 floats of LDS.
__device__ __forceinline__ float block_sum256(float v, float *red) {
    v = wave_sum64(v);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    return (red[0] + red[1]) + (red[2] + red[3]);
}

constexpr int GD = 128;  // key and value head dimension of the recurrence

__global__ __launch_bounds__(256) void gdn_conv_kernel(const float *__restrict__ u,
                                                       const float *__restrict__ conv_w,
                                                       float *__restrict__ conv_state, int C,
                                                       int Hv, const float *__restrict__ a_log,
                                                       const float *__restrict__ dt_bias,
                                                       float *__restrict__ c_out,
                                                       float *__restrict__ gates) {
    const int ch = blockIdx.x * 256 + threadIdx.x;
    if (ch < C) {
        float *st = conv_state + 3 * (int64_t)ch;
        const float4 w = *reinterpret_cast<const float4 *>(conv_w + 4 * (int64_t)ch);
        const float s0 = st[0], s1 = st[1], s2 = st[2], x = u[ch];
        const float s = fmaf(w.w, x, fmaf(w.z, s2, fmaf(w.y, s1, w.x * s0)));
        c_out[ch] = siluf_(s);
        st[0] = s1;
        st[1] = s2;
        st[2] = x;
    }
    if (blockIdx.x == 0 && threadIdx.x < Hv) {
        const int h = threadIdx.x;
        const int64_t off = (int64_t)C + (int64_t)Hv * GD;  // b after q, k, v and z
        const float b = u[off + h], a = u[off + Hv + h];
        gates[h] = sigmoidf_(b);
        gates[Hv + h] = expf(-expf(a_log[h]) * softplusf_(a + dt_bias[h]));
    }
}

__global__ __launch_bounds__(256) void gdn_state_kernel(const float *__restrict__ c_out,
                                                        const float *__restrict__ gates,
                                                        const float *__restrict__ u, int Hk,
                                                        int Hv, const float *__restrict__ norm_w,
                                                        float eps, float *__restrict__ S,
                                                        float *__restrict__ out) {
    __shared__ float kq[2][GD];
    __shared__ float ov[GD];
    __shared__ float red[4];
    const int h = blockIdx.x, t = threadIdx.x;
    const int j = h / (Hv / Hk);  // key head of this value head
    const int64_t nq = (int64_t)Hk * GD;
    const float *q = c_out + (int64_t)j * GD, *k = c_out + nq + (int64_t)j * GD;
    const float *v = c_out + 2 * nq + (int64_t)h * GD;
    // L2 norms of q and k (threads 0..127: q, 128..255: k)
    const float qk = t < GD ? q[t] : k[t - GD];
    float ssq = t < GD ? qk * qk : 0.f, ssk = t < GD ? 0.f : qk * qk;
    ssq = block_sum256(ssq, red);
    ssk = block_sum256(ssk, red);
    if (t < GD) kq[1][t] = qk / sqrtf(ssq + eps) / sqrtf((float)GD);
    else kq[0][t - GD] = qk / sqrtf(ssk + eps);
    __syncthreads();
    const float alpha = gates[Hv + h], beta = gates[h];
    const int lane32 = t & 31, row0 = t >> 5;
    const float4 kk = *reinterpret_cast<const float4 *>(&kq[0][4 * lane32]);
    const float4 qq = *reinterpret_cast<const float4 *>(&kq[1][4 * lane32]);
    float4 *Sh = reinterpret_cast<float4 *>(S + (int64_t)h * GD * GD);
    float4 s[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) s[m] = Sh[t + 256 * m];
#pragma unroll
    for (int m = 0; m < 16; ++m) {
        const int dv = row0 + 8 * m;
        float4 r = s[m];
        r.x *= alpha;
        r.y *= alpha;
        r.z *= alpha;
        r.w *= alpha;
        float kv = fmaf(r.x, kk.x, fmaf(r.y, kk.y, fmaf(r.z, kk.z, r.w * kk.w)));
        kv = half_sum32(kv);
        const float delta = beta * (v[dv] - kv);
        r.x = fmaf(kk.x, delta, r.x);
        r.y = fmaf(kk.y, delta, r.y);
        r.z = fmaf(kk.z, delta, r.z);
        r.w = fmaf(kk.w, delta, r.w);
        float o = fmaf(r.x, qq.x, fmaf(r.y, qq.y, fmaf(r.z, qq.z, r.w * qq.w)));
        o = half_sum32(o);
        if (lane32 == 0) ov[dv] = o;
        s[m] = r;
    }
#pragma unroll
    for (int m = 0; m < 16; ++m) Sh[t + 256 * m] = s[m];
    __syncthreads();
    // gated RMSNorm of the head's output
    const float o = t < GD ? ov[t] : 0.f;
    const float ms = block_sum256(o * o, red);
    if (t < GD) {
        const float inv = 1.0f / sqrtf(ms / (float)GD + eps);
        const int64_t zo = 2 * nq + (int64_t)Hv * GD + (int64_t)h * GD + t;  // z after q, k, v
        out[(int64_t)h * GD + t] = norm_w[t] * (o * inv) * siluf_(u[zo]);
    }
}

constexpr int AD = 256;  // attention head dimension

// (1 + w) RMSNorm and rotary of one 256-vector, one element per thread;
// returns this thread's element.  buf: 256 floats of LDS, red: 4.
__device__ __forceinline__ float norm_rope(float x, const float *__restrict__ w, float eps, int R,
                                           double theta, int64_t pos, float *buf, float *red) {
    const int d = threadIdx.x;
    const float ss = block_sum256(x * x, red);
    const float n = x / sqrtf(ss / (float)AD + eps) * (1.0f + w[d]);
    buf[d] = n;
    __syncthreads();
    float r = n;
    if (d < R) {
        const int half = R / 2, i = d < half ? d : d - half;
        const double ang = (double)pos * pow(theta, -2.0 * i / R);
        const float cs = (float)cos(ang), sn = (float)sin(ang);
        r = d < half ? n * cs - buf[d + half] * sn : n * cs + buf[d - half] * sn;
    }
    __syncthreads();
    return r;
}

__global__ __launch_bounds__(256) void attn_step_kernel(
    const float *__restrict__ u, const float *__restrict__ qw, const float *__restrict__ kw,
    float *__restrict__ kc, float *__restrict__ vc, int64_t cap, int64_t pos_val,
    const int64_t *__restrict__ pos_dev, int Hq, int Hkv, int R, float theta, float eps,
    float *__restrict__ out) {
    __shared__ float qs[AD], ks[AD], buf[AD];
    __shared__ float red[4];
    __shared__ float wm[4], wl[4];
    __shared__ float wacc[4][AD];
    const int h = blockIdx.x, d = threadIdx.x;
    const int g = h / (Hq / Hkv);
    const int64_t pos = pos_dev ? *pos_dev : pos_val;
    if (pos < 0 || pos >= cap) return;  // the callers keep pos inside the cache
    const float *uq = u + (int64_t)h * 2 * AD;
    const float *uk = u + (int64_t)Hq * 2 * AD + (int64_t)g * AD;
    const float *uv = u + (int64_t)Hq * 2 * AD + (int64_t)Hkv * AD + (int64_t)g * AD;
    const float gate = uq[AD + d];
    qs[d] = norm_rope(uq[d], qw, eps, R, (double)theta, pos, buf, red);
    const float kn = norm_rope(uk[d], kw, eps, R, (double)theta, pos, buf, red);
    const float vn = uv[d];
    ks[d] = kn;
    if (h % (Hq / Hkv) == 0) {  // the key/value head's first query head fills the cache
        kc[((int64_t)g * cap + pos) * AD + d] = kn;
        vc[((int64_t)g * cap + pos) * AD + d] = vn;
    }
    __shared__ float vs[AD];
    vs[d] = vn;
    __syncthreads();
    // online softmax over positions t = w mod 4 (position pos from LDS)
    const int w = d >> 6, lane = d & 63;
    const float4 q4 = *reinterpret_cast<const float4 *>(&qs[4 * lane]);
    const float scale = 1.0f / sqrtf((float)AD);
    float m = -INFINITY, l = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    const float *kg = kc + (int64_t)g * cap * AD, *vg = vc + (int64_t)g * cap * AD;
    for (int64_t t = w; t <= pos; t += 4) {
        const float4 k4 = t == pos ? *reinterpret_cast<const float4 *>(&ks[4 * lane])
                                   : *reinterpret_cast<const float4 *>(kg + t * AD + 4 * lane);
        const float4 v4 = t == pos ? *reinterpret_cast<const float4 *>(&vs[4 * lane])
                                   : *reinterpret_cast<const float4 *>(vg + t * AD + 4 * lane);
        float s = fmaf(q4.x, k4.x, fmaf(q4.y, k4.y, fmaf(q4.z, k4.z, q4.w * k4.w)));
        s = wave_sum64(s) * scale;
        const float mn = fmaxf(m, s);
        const float c = expf(m - mn), e = expf(s - mn);
        l = fmaf(l, c, e);
        acc.x = fmaf(acc.x, c, e * v4.x);
        acc.y = fmaf(acc.y, c, e * v4.y);
        acc.z = fmaf(acc.z, c, e * v4.z);
        acc.w = fmaf(acc.w, c, e * v4.w);
        m = mn;
    }
    if (lane == 0) {
        wm[w] = m;
        wl[w] = l;
    }
    *reinterpret_cast<float4 *>(&wacc[w][4 * lane]) = acc;
    __syncthreads();
    float M = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) M = fmaxf(M, wm[i]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (wm[i] == -INFINITY) continue;  // a wave that saw no position
        const float c = expf(wm[i] - M);
        num = fmaf(wacc[i][d], c, num);
        den = fmaf(wl[i], c, den);
    }
    out[(int64_t)h * AD + d] = num / den * sigmoidf_(gate);
}

}  // namespace

int launch_gdn_step(const GdnShape &s, const float *u, const float *conv_w, const float *a_log,
                    const float *dt_bias, const float *norm_w, float *conv_state, float *S,
                    float *out, float *scratch, hipStream_t stream) {
    const int C = 2 * s.Hk * GD + s.Hv * GD;
    float *c_out = scratch, *gates = scratch + C;
    hipLaunchKernelGGL(gdn_conv_kernel, dim3((unsigned)((C + 255) / 256)), dim3(256), 0, stream, u,
                       conv_w, conv_state, C, s.Hv, a_log, dt_bias, c_out, gates);
    Q4K_HIP(hipGetLastError());
    hipLaunchKernelGGL(gdn_state_kernel, dim3((unsigned)s.Hv), dim3(256), 0, stream, c_out, gates,
                       u, s.Hk, s.Hv, norm_w, s.eps, S, out);
    Q4K_HIP(hipGetLastError());
    return Q4K_OK;
}

int launch_attn_step(const AttnShape &s, const float *u, const float *q_norm_w,
                     const float *k_norm_w, float *k_cache, float *v_cache, int64_t cap,
                     int64_t pos, const int64_t *pos_dev, float *out, hipStream_t stream) {
    hipLaunchKernelGGL(attn_step_kernel, dim3((unsigned)s.Hq), dim3(256), 0, stream, u, q_norm_w,
                       k_norm_w, k_cache, v_cache, cap, pos, pos_dev, s.Hq, s.Hkv, s.R, s.theta,
                       s.eps, out);
    Q4K_HIP(hipGetLastError());
    return Q4K_OK;
}

}  // namespace q4k
