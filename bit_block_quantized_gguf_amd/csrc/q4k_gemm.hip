// q4k_gemm.hip — prefill GEMM Y[P][M] = X[P][K] * W^T on gfx950 bf16 MFMA.
//
// Prefill is the compute-bound phase ("Qwen3.6-27B on Apple M3 Pro — the
// llama.cpp parity bar", the prefill-loves-the-GPU argument; "Mac Qwen3.6-27B
// Metal Q4_K perf diagnosis", §2 prefill phases), so this is the one matmul
// that runs on the matrix cores: v_mfma_f32_32x32x16_bf16 with f32
// accumulation.
//
// Tiling.  A workgroup of four waves computes a 128-token x 128-row tile of
// Y, walking K one super-block (256 columns) at a time:
//   * X (tokens) is the MFMA A operand.  Each step the workgroup loads the
//     128 x 256 f32 slice (each wave reads whole 1 KiB token rows), rounds it
//     to bf16 (RNE, v_cvt_pk_bf16_f32) and stores it in LDS with a 16-byte
//     row pad, so the fragment reads (32 tokens, same column) hit 16
//     distinct 4-bank groups.
//   * W is the B operand and never goes through LDS: each wave owns 32 rows
//     of the tile, lane l handles row l%32 and half h = l/32 of every 32-byte
//     quant group.  Its 16 quant bytes hold 16 low-nibble weights
//     (sub-block 2g) and 16 high-nibble weights (sub-block 2g+1); each run of
//     8 converts (w = fma(q, d*sc, -dmin*m), exact f32, then bf16 RNE) into
//     one B fragment.  Because a fragment may pair any 8 columns per lane as
//     long as X is read at the same columns, the lane's column offset is
//     64g + 32*hi + 16h + 8t, and the A fragment is read from LDS at that
//     same offset.  Every weight is dequantised once per tile.
//   * Output layout of the 32x32 MFMA: lane l holds column l%32 (a W row)
//     and rows 8(v/4) + 4(l/32) + v%4 (tokens) of accumulator v, so each
//     store instruction writes 32 consecutive floats of a token row.
//   * For short M the K range is split across workgroups: each split writes
//     its partial tile to a workspace and a second kernel adds the splits in
//     order (deterministic; no cross-workgroup synchronisation inside a
//     kernel).
#include "q4k_device.hpp"
#include "q4k_internal.hpp"

#include <algorithm>
#include <atomic>

namespace q4k {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128;  // W rows per tile
constexpr int BN = 128;  // tokens per tile
constexpr int XS = 256 + 8;  // LDS row stride of the staged X slice, in bf16

struct GemmParams {
    const uint8_t *w;
    const float *X;
    float *Y;
    int32_t M, K, P, nb;
    int64_t row_bytes;
    int32_t ks;
    int32_t row_tiles;
    float *ws;
};

__device__ __forceinline__ bf16x8 dequant8(uint32_t q0, uint32_t q1, float ds, float dm) {
    bf16x8 r;
    r[0] = (__bf16)fmaf(ubyte(q0, 0), ds, -dm);
    r[1] = (__bf16)fmaf(ubyte(q0, 1), ds, -dm);
    r[2] = (__bf16)fmaf(ubyte(q0, 2), ds, -dm);
    r[3] = (__bf16)fmaf(ubyte(q0, 3), ds, -dm);
    r[4] = (__bf16)fmaf(ubyte(q1, 0), ds, -dm);
    r[5] = (__bf16)fmaf(ubyte(q1, 1), ds, -dm);
    r[6] = (__bf16)fmaf(ubyte(q1, 2), ds, -dm);
    r[7] = (__bf16)fmaf(ubyte(q1, 3), ds, -dm);
    return r;
}

__global__ __launch_bounds__(256, 2) void gemm_kernel(const GemmParams p) {
    __shared__ __attribute__((aligned(16))) __bf16 xs[BN * XS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int rt = blockIdx.x, tt = blockIdx.y, split = blockIdx.z;
    const int row0 = rt * BM, tok0 = tt * BN;
    const int jb = (int)(((int64_t)split * p.nb) / p.ks);
    const int je = (int)(((int64_t)(split + 1) * p.nb) / p.ks);

    // this lane's W row and half-group
    const int wrow = row0 + 32 * wave + (lane & 31);
    const int wrowc = wrow < p.M ? wrow : p.M - 1;
    const int h = lane >> 5;
    const uint8_t *wr = p.w + (int64_t)wrowc * p.row_bytes;

    f32x16 acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][v] = 0.f;

    for (int j = jb; j < je; ++j) {
        // ---- W: this lane's header and four 16-byte quant words (issued early) ----
        const uint8_t *bp = wr + (int64_t)j * kBlockBytes;
        const uint4 hdr = ldg16(bp);
        uint4 qw[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) qw[g] = ldg16(bp + 16 + 32 * g + 16 * h);

        // ---- X: stage the 128 x 256 slice as bf16 ----
        __syncthreads();
#pragma unroll 8
        for (int it = 0; it < 32; ++it) {
            const int idx = it * 256 + tid;
            const int t = idx >> 6;         // token within tile
            const int kq = idx & 63;        // float4 index within the 256 columns
            int tok = tok0 + t;
            tok = tok < p.P ? tok : p.P - 1;
            const float4 v = *reinterpret_cast<const float4 *>(p.X + (int64_t)tok * p.K +
                                                               256 * (int64_t)j + 4 * kq);
            bf16x4 b;
            b[0] = (__bf16)v.x;
            b[1] = (__bf16)v.y;
            b[2] = (__bf16)v.z;
            b[3] = (__bf16)v.w;
            *reinterpret_cast<bf16x4 *>(&xs[t * XS + 4 * kq]) = b;
        }
        __syncthreads();

        // ---- dequantise into B fragments and multiply ----
        const float d = half_lo(hdr.x), dmin = half_hi(hdr.x);
        const Scales sc = unpack_scales(hdr.y, hdr.z, hdr.w);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const float dsl = d * scale_of(sc, 2 * g), dml = dmin * min_of(sc, 2 * g);
            const float dsh = d * scale_of(sc, 2 * g + 1), dmh = dmin * min_of(sc, 2 * g + 1);
            const uint4 q = qw[g];
            const uint32_t l0 = and_mask(q.x, 0x0F0F0F0Fu), l1 = and_mask(q.y, 0x0F0F0F0Fu);
            const uint32_t l2 = and_mask(q.z, 0x0F0F0F0Fu), l3 = and_mask(q.w, 0x0F0F0F0Fu);
            const uint32_t h0 = and_mask(q.x >> 4, 0x0F0F0F0Fu), h1 = and_mask(q.y >> 4, 0x0F0F0F0Fu);
            const uint32_t h2 = and_mask(q.z >> 4, 0x0F0F0F0Fu), h3 = and_mask(q.w >> 4, 0x0F0F0F0Fu);
            bf16x8 bfr[4];
            bfr[0] = dequant8(l0, l1, dsl, dml);
            bfr[1] = dequant8(l2, l3, dsl, dml);
            bfr[2] = dequant8(h0, h1, dsh, dmh);
            bfr[3] = dequant8(h2, h3, dsh, dmh);
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                // column offset of this lane's 8 weights inside the block
                const int kofs = 64 * g + 32 * (f >> 1) + 16 * h + 8 * (f & 1);
#pragma unroll
                for (int ti = 0; ti < 4; ++ti) {
                    const bf16x8 a =
                        *reinterpret_cast<const bf16x8 *>(&xs[(32 * ti + (lane & 31)) * XS + kofs]);
                    acc[ti] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bfr[f], acc[ti], 0, 0, 0);
                }
            }
        }
    }

    // ---- epilogue ----
    const int col = row0 + 32 * wave + (lane & 31);   // W row = Y column
    const bool col_ok = col < p.M;
    // K split across workgroups: this split's partial tile goes to the
    // workspace; a second kernel adds the splits in order.
    float *out = p.ks > 1 ? p.ws + (int64_t)split * p.P * p.M : p.Y;
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int tok = tok0 + 32 * ti + 8 * (v >> 2) + 4 * h + (v & 3);
            if (col_ok && tok < p.P) out[(int64_t)tok * p.M + col] = acc[ti][v];
        }
}

// Y[i] = sum over splits of ws[s][i], in split order (one element per thread).
__global__ __launch_bounds__(256) void gemm_reduce_kernel(const float *__restrict__ ws,
                                                          float *__restrict__ Y, int64_t n,
                                                          int ks) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    float t = ws[i];
    for (int s = 1; s < ks; ++s) t += ws[(int64_t)s * n + i];
    Y[i] = t;
}

std::atomic<int> g_override_ks{0};

}  // namespace

void set_gemm_override(int ks) { g_override_ks = ks; }

GemmLaunch choose_gemm_launch(int64_t M, int64_t K, int64_t P) {
    const int64_t tiles = ((M + BM - 1) / BM) * ((P + BN - 1) / BN);
    const int64_t nb = K / 256;
    GemmLaunch L;
    // Two workgroups fit per CU; split K while fewer than ~one workgroup per
    // CU would run, keeping at least 8 super-blocks per split.
    int64_t ks = 1;
    while (tiles * ks < 256 && nb / (ks * 2) >= 8) ks *= 2;
    L.ks = (int)ks;
    const int o = g_override_ks.load();
    if (o > 0) L.ks = (int)std::min<int64_t>(o, nb);
    return L;
}

size_t gemm_partial_floats(const GemmLaunch &L, int64_t M, int64_t P) {
    return L.ks > 1 ? (size_t)L.ks * (size_t)P * (size_t)M : 0;
}

size_t gemm_counters(int64_t M, int64_t P) {
    (void)M;
    (void)P;
    return 0;
}

int launch_gemm(const uint8_t *w, const float *X, float *Y, int64_t M, int64_t K, int64_t P,
                const GemmLaunch &L, const Workspace &ws, hipStream_t stream) {
    GemmParams p;
    p.w = w;
    p.X = X;
    p.Y = Y;
    p.M = (int32_t)M;
    p.K = (int32_t)K;
    p.P = (int32_t)P;
    p.nb = (int32_t)(K / 256);
    p.row_bytes = (K / 256) * kBlockBytes;
    p.ks = L.ks;
    p.row_tiles = (int32_t)((M + BM - 1) / BM);
    p.ws = ws.partials;
    const dim3 grid((unsigned)p.row_tiles, (unsigned)((P + BN - 1) / BN), (unsigned)L.ks);
    if (grid.y > 65535 || grid.z > 65535)
        return fail(Q4K_EUNSUPPORTED, "gemm: P or split count too large");
    hipLaunchKernelGGL(gemm_kernel, grid, dim3(256), 0, stream, p);
    Q4K_HIP(hipGetLastError());
    if (L.ks > 1) {
        const int64_t n = P * M;
        const int64_t groups = (n + 255) / 256;
        if (groups > 0x7FFFFFFF) return fail(Q4K_EUNSUPPORTED, "gemm: output too large");
        hipLaunchKernelGGL(gemm_reduce_kernel, dim3((unsigned)groups), dim3(256), 0, stream,
                           (const float *)ws.partials, Y, n, L.ks);
        Q4K_HIP(hipGetLastError());
    }
    return Q4K_OK;
}

}  // namespace q4k
