// q4k_gemv.hip — Q4_K GEMV kernels for gfx950 (batch-1, N-vector, and the
// fused-epilogue variants used by the decode stack).
//
// The decode matmul is bandwidth-bound ("Mac Qwen3.6-27B Metal Q4_K perf
// diagnosis", §2-§4): every weight byte is read once and the job is to stream
// them at HBM speed.  Mapping on the CDNA4 execution model:
//
//  * A wave owns 64 consecutive rows, one row per lane, and walks a range of
//    super-block columns.  All lanes of a wave therefore need the same 256
//    activations at the same time: those are fetched with scalar loads (the
//    activation pointer is in the constant address space) and enter every
//    FMA as an SGPR operand — no vector-memory traffic and no LDS for x.
//  * Each lane streams its row's 144-byte block as nine 16-byte loads; the
//    next block's loads are issued before the current block is computed.
//  * Per weight the VALU work is one byte-to-float conversion and one FMA
//    (plus one AND per four weights); the scale/min algebra is applied once
//    per 32-weight sub-block:  y += d*sc * sum(q*x) - dmin*m * sum(x).
//    High nibbles are converted in place (16*q) and their scale carries the
//    exact factor 1/16.  The per-sub-block sums of x are formed once per
//    block by the wave (one 16-byte load per lane, a 3-step butterfly).
//  * K is split across the waves of a workgroup (reduced through LDS in a
//    fixed order) and, for short M, across workgroups: partials go to a
//    workspace and the last-arriving workgroup of a row tile (per-tile
//    atomic counter) adds them in split order, so results are deterministic.
//    The counter is returned to zero by that workgroup.
#include "q4k_device.hpp"
#include "q4k_internal.hpp"

#include <algorithm>
#include <atomic>

namespace q4k {

namespace {

__device__ __forceinline__ float wave_sum(float v) {
    // xor butterfly: partners add the same two values, so every lane ends
    // with the same bits.
    v += __shfl_xor(v, 32);
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 8);
    v += __shfl_xor(v, 4);
    v += __shfl_xor(v, 2);
    v += __shfl_xor(v, 1);
    return v;
}

template <int NV>
__device__ __forceinline__ void sub_block_sums(const float *x, int64_t xs, int j, int lane,
                                               float (&xsum)[NV][8]) {
#pragma unroll
    for (int n = 0; n < NV; ++n) {
        const float4 v = *reinterpret_cast<const float4 *>(x + n * xs + 256 * j + 4 * lane);
        float s = (v.x + v.y) + (v.z + v.w);
        s += __shfl_xor(s, 1);
        s += __shfl_xor(s, 2);
        s += __shfl_xor(s, 4);
#pragma unroll
        for (int sb = 0; sb < 8; ++sb)
            xsum[n][sb] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s), 8 * sb));
    }
}

template <int NMAT>
__device__ __forceinline__ void load_blocks(const uint8_t *const (&rp)[NMAT], int j,
                                            uint4 (&b)[NMAT][9]) {
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
        const uint8_t *p = rp[m] + (int64_t)j * kBlockBytes;
#pragma unroll
        for (int i = 0; i < 9; ++i) b[m][i] = ldg16(p + 16 * i);
    }
}

// acc[n] += sum over the block of w * x_n (factored per sub-block).
template <int NV>
__device__ __forceinline__ void block_dot(const uint4 (&b)[9], const float *xblk, int64_t xs,
                                          const float (&xsum)[NV][8], float (&acc)[NV]) {
    constexpr int C = NV >= 4 ? 1 : (NV == 2 ? 2 : 4);  // independent FMA chains per sum
    const float d = half_lo(b[0].x);
    const float dmin = half_hi(b[0].x);
    const Scales sc = unpack_scales(b[0].y, b[0].z, b[0].w);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        float tl[NV][C], th[NV][C];
#pragma unroll
        for (int n = 0; n < NV; ++n)
#pragma unroll
            for (int c = 0; c < C; ++c) tl[n][c] = th[n][c] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t v = word_of(b[1 + 2 * g + (i >> 2)], i & 3);
            const uint32_t lo = and_mask(v, 0x0F0F0F0Fu);  // q
            const uint32_t hi = and_mask(v, 0xF0F0F0F0u);  // 16*q
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) {
                const float ql = ubyte(lo, bb);
                const float qh = ubyte(hi, bb);
#pragma unroll
                for (int n = 0; n < NV; ++n) {
                    cfloat *xp = as_const(xblk + n * xs + 64 * g);
                    tl[n][bb % C] = fmaf(ql, xp[4 * i + bb], tl[n][bb % C]);
                    th[n][bb % C] = fmaf(qh, xp[32 + 4 * i + bb], th[n][bb % C]);
                }
            }
        }
        const float dl = d * scale_of(sc, 2 * g);
        const float dh = d * scale_of(sc, 2 * g + 1) * 0.0625f;  // exact: undoes the 16*q
        const float ml = dmin * min_of(sc, 2 * g);
        const float mh = dmin * min_of(sc, 2 * g + 1);
#pragma unroll
        for (int n = 0; n < NV; ++n) {
            float tls = tl[n][0], ths = th[n][0];
#pragma unroll
            for (int c = 1; c < C; ++c) {
                tls += tl[n][c];
                ths += th[n][c];
            }
            float a = acc[n];
            a = fmaf(dl, tls, a);
            a = fmaf(-ml, xsum[n][2 * g], a);
            a = fmaf(dh, ths, a);
            a = fmaf(-mh, xsum[n][2 * g + 1], a);
            acc[n] = a;
        }
    }
}

template <int NV, int NMAT, int EPI, int WK>
__global__ __launch_bounds__(64 * WK) void gemv_kernel(const GemvParams p) {
    constexpr int NA = NMAT * NV;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int tile = blockIdx.x;
    const int split = blockIdx.y;
    const int row = tile * 64 + lane;
    const int rowc = row < p.M ? row : p.M - 1;
    const int nchunks = p.ks * WK;
    const int chunk = split * WK + wave;
    const int jb = (int)(((int64_t)chunk * p.nb) / nchunks);
    const int je = (int)(((int64_t)(chunk + 1) * p.nb) / nchunks);

    const uint8_t *rp[NMAT];
    rp[0] = p.w0 + (int64_t)rowc * p.row_bytes;
    if constexpr (NMAT == 2) rp[1] = p.w1 + (int64_t)rowc * p.row_bytes;

    float acc[NMAT][NV];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int n = 0; n < NV; ++n) acc[m][n] = 0.f;

    uint4 cur[NMAT][9];
    if (jb < je) load_blocks<NMAT>(rp, jb, cur);
    for (int j = jb; j < je; ++j) {
        uint4 nxt[NMAT][9];
        const bool more = j + 1 < je;
        if (more) load_blocks<NMAT>(rp, j + 1, nxt);
        float xsum[NV][8];
        sub_block_sums<NV>(p.x, p.x_stride, j, lane, xsum);
        const float *xblk = p.x + 256 * (int64_t)j;
#pragma unroll
        for (int m = 0; m < NMAT; ++m) block_dot<NV>(cur[m], xblk, p.x_stride, xsum, acc[m]);
        if (more) {
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
                for (int i = 0; i < 9; ++i) cur[m][i] = nxt[m][i];
        }
    }

    // ---- reduce the WK waves of the group (fixed order) ----
    float tot[NA];
    if constexpr (WK > 1) {
        __shared__ float red[WK][NA][64];
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int n = 0; n < NV; ++n) red[wave][m * NV + n][lane] = acc[m][n];
        __syncthreads();
        if (wave != 0) return;
#pragma unroll
        for (int a = 0; a < NA; ++a) {
            float s = red[0][a][lane];
#pragma unroll
            for (int w = 1; w < WK; ++w) s += red[w][a][lane];
            tot[a] = s;
        }
    } else {
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int n = 0; n < NV; ++n) tot[m * NV + n] = acc[m][n];
    }

    // ---- reduce the K splits across workgroups: last arriver, split order ----
    if (p.ks > 1) {
        if (row < p.M) {
#pragma unroll
            for (int a = 0; a < NA; ++a) p.ws[((int64_t)split * NA + a) * p.M + row] = tot[a];
        }
        __threadfence();
        unsigned prev = 0;
        if (lane == 0) prev = atomicAdd(&p.cnt[tile], 1u);
        prev = __shfl(prev, 0);
        if (prev != (unsigned)(p.ks - 1)) return;
        __threadfence();
#pragma unroll
        for (int a = 0; a < NA; ++a) {
            float s = 0.f;
            if (row < p.M)
                for (int sp = 0; sp < p.ks; ++sp) s += p.ws[((int64_t)sp * NA + a) * p.M + row];
            tot[a] = s;
        }
        if (lane == 0) p.cnt[tile] = 0u;
    }

    // ---- epilogue (one lane per row) ----
    if constexpr (EPI == EPI_PLAIN) {
        if (row < p.M) {
#pragma unroll
            for (int n = 0; n < NV; ++n) p.y[(int64_t)n * p.y_stride + row] = tot[n];
        }
    } else {
        float ss = 0.f;
        for (int i = lane; i < p.in_sq_n; i += 64) ss += p.in_sq[i];
        ss = wave_sum(ss);
        const float inv = 1.0f / sqrtf(ss / (float)p.in_len + p.eps);
        float val;
        if constexpr (EPI == EPI_SCALE) {
            val = tot[0] * inv;
        } else if constexpr (EPI == EPI_RESID) {
            val = fmaf(tot[0], inv, p.resid[rowc]);
        } else {
            const float g = tot[0] * inv;
            const float v = tot[NV] * inv;
            if (row < p.M) {
                p.y_g[row] = g;
                p.y_v[row] = v;
            }
            val = g / (1.0f + expf(-g)) * v;
        }
        if (row < p.M) p.y[row] = val;
        const float sq = wave_sum(row < p.M ? val * val : 0.f);
        if (lane == 0) p.out_sq[tile] = sq;
    }
}

__global__ __launch_bounds__(64) void sumsq_kernel(const float *__restrict__ v, int64_t n,
                                                   float *__restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * 64 + threadIdx.x;
    const float a = i < n ? v[i] : 0.f;
    const float s = wave_sum(a * a);
    if (threadIdx.x == 0) out[blockIdx.x] = s;
}

std::atomic<int> g_override_wk{0};
std::atomic<int> g_override_ks{0};

template <int NV, int NMAT, int EPI>
int launch_wk(const GemvParams &p, const GemvLaunch &L, hipStream_t stream) {
    const dim3 grid((unsigned)((p.M + 63) / 64), (unsigned)L.ks);
    switch (L.wk) {
        case 2: hipLaunchKernelGGL((gemv_kernel<NV, NMAT, EPI, 2>), grid, dim3(128), 0, stream, p); break;
        case 4: hipLaunchKernelGGL((gemv_kernel<NV, NMAT, EPI, 4>), grid, dim3(256), 0, stream, p); break;
        case 8: hipLaunchKernelGGL((gemv_kernel<NV, NMAT, EPI, 8>), grid, dim3(512), 0, stream, p); break;
        default: return fail(Q4K_EINVAL, "unsupported waves-per-group %d", L.wk);
    }
    Q4K_HIP(hipGetLastError());
    return Q4K_OK;
}

}  // namespace

void set_gemv_override(int wk, int ks) {
    g_override_wk = wk;
    g_override_ks = ks;
}

GemvLaunch choose_gemv_launch(int64_t M, int64_t K, int nv, int nmat) {
    (void)nv;
    (void)nmat;
    const int64_t tiles = (M + 63) / 64;
    const int64_t nb = K / 256;
    GemvLaunch L;
    L.wk = 4;
    // Aim for ~8 waves per CU across 256 CUs so that enough 16-byte loads are
    // in flight to cover HBM latency; keep at least one block per wave.
    const double target_waves = 2048.0;
    int64_t ks = (int64_t)(target_waves / (double)(tiles * L.wk) + 0.5);
    ks = std::max<int64_t>(1, std::min<int64_t>(ks, std::max<int64_t>(1, nb / L.wk)));
    L.ks = (int)std::min<int64_t>(ks, 64);
    const int owk = g_override_wk.load(), oks = g_override_ks.load();
    if (owk > 0) L.wk = owk;
    if (oks > 0) L.ks = (int)std::min<int64_t>(oks, std::max<int64_t>(1, nb));
    if ((int64_t)L.ks * L.wk > nb) L.ks = (int)std::max<int64_t>(1, nb / L.wk);
    return L;
}

size_t gemv_partial_floats(const GemvLaunch &L, int64_t M, int nv, int nmat) {
    return L.ks > 1 ? (size_t)L.ks * (size_t)nmat * (size_t)nv * (size_t)M : 0;
}

size_t gemv_counters(int64_t M) { return (size_t)((M + 63) / 64); }

int launch_gemv(const GemvParams &p, int nv, int nmat, int epi, const GemvLaunch &L,
                hipStream_t stream) {
    if (nmat == 1 && epi == EPI_PLAIN) {
        switch (nv) {
            case 1: return launch_wk<1, 1, EPI_PLAIN>(p, L, stream);
            case 2: return launch_wk<2, 1, EPI_PLAIN>(p, L, stream);
            case 4: return launch_wk<4, 1, EPI_PLAIN>(p, L, stream);
            case 8: return launch_wk<8, 1, EPI_PLAIN>(p, L, stream);
            case 16: return launch_wk<16, 1, EPI_PLAIN>(p, L, stream);
            default: return fail(Q4K_EINVAL, "unsupported vector count %d", nv);
        }
    }
    if (nv != 1) return fail(Q4K_EINVAL, "fused epilogues take one vector");
    if (nmat == 1 && epi == EPI_SCALE) return launch_wk<1, 1, EPI_SCALE>(p, L, stream);
    if (nmat == 1 && epi == EPI_RESID) return launch_wk<1, 1, EPI_RESID>(p, L, stream);
    if (nmat == 2 && epi == EPI_SWIGLU) return launch_wk<1, 2, EPI_SWIGLU>(p, L, stream);
    return fail(Q4K_EINVAL, "unsupported GEMV variant");
}

int launch_sumsq(const float *v, int64_t n, float *out, hipStream_t stream) {
    const unsigned blocks = (unsigned)((n + 63) / 64);
    if (!blocks) return Q4K_OK;
    hipLaunchKernelGGL(sumsq_kernel, dim3(blocks), dim3(64), 0, stream, v, n, out);
    Q4K_HIP(hipGetLastError());
    return Q4K_OK;
}

}  // namespace q4k
