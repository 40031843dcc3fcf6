// q4k_gemm.hip — prefill GEMM Y[P][M] = X[P][K] * W^T on gfx950 bf16 MFMA.
//
// Prefill is the compute-bound phase ("Qwen3.6-27B on Apple M3 Pro — the
// llama.cpp parity bar", the prefill-loves-the-GPU argument; "Mac Qwen3.6-27B
// Metal Q4_K perf diagnosis", §2 prefill phases), so this is the one matmul
// that runs on the matrix cores: v_mfma_f32_32x32x16_bf16 with f32
// accumulation.
//
//  * X is rounded to bf16 once (round to nearest even) by a prologue kernel
//    into a workspace whose token count is padded to the tile with zeros, so
//    the main loop moves half the bytes, spends no VALU on conversion and
//    needs no token clamping.
//  * Workgroup tile: 256 W rows x (32 * T) tokens, four waves, one workgroup
//    per CU.  Wave w owns W rows 64w .. 64w+63 (two 32-row groups) for all
//    tokens of the tile, so every W weight is dequantised exactly once per
//    tile and every X fragment read from LDS feeds two MFMAs.  The 32 * T
//    accumulator registers per 32x32 output block live in the AGPR file.
//  * K advances half a super-block (128 columns, quant groups g0, g0+1) per
//    step.  The step's X slice (32T tokens x 128 columns of bf16) is copied
//    from global memory straight into LDS with global_load_lds_dwordx4, so
//    it never occupies registers; it is double-buffered.  Each token row is
//    256 bytes = 16 chunks of 16 bytes and chunk c of token t is stored at
//    slot c ^ (t & 15), so the 32 lanes of a fragment read (32 consecutive
//    tokens, one chunk) cover all banks.
//  * W never goes through LDS: lane l handles row l%32 of each of its row
//    groups and half h = l/32 of every 32-byte quant group.  Its 16 quant
//    bytes hold 16 low-nibble weights (sub-block 2g) and 16 high-nibble
//    weights (sub-block 2g+1); each run of 8 converts (w = fma(q, d*sc,
//    -dmin*m), exact in f32, then bf16 RNE) into one B fragment.  A fragment
//    may pair any 8 columns per lane as long as X is read at the same
//    columns, so the lane's column offset is 64g + 32*hi + 16h + 8t and the
//    A fragment (X) is read from LDS at that offset.  The next step's W bytes
//    are loaded into registers while the current step computes.
//  * Output layout of the 32x32 MFMA: lane l holds column l%32 (a W row) and
//    rows 8(v/4) + 4(l/32) + v%4 (tokens) of accumulator v, so each store
//    instruction writes 32 consecutive floats of a token row.
//  * When there are too few tiles to fill the chip the K range is split
//    across workgroups: each split writes its partial tile to a workspace and
//    a second kernel adds the splits in order (deterministic; no
//    cross-workgroup synchronisation inside a kernel).
#include "q4k_device.hpp"
#include "q4k_internal.hpp"

#include <algorithm>
#include <atomic>

namespace q4k {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) void gvoid;
typedef __attribute__((address_space(3))) void lvoid;

constexpr int BM = 256;        // W rows per tile
constexpr int KS = 128;        // columns per step (half a super-block)
constexpr int TOK_PAD = 256;   // token padding of the bf16 X copy (the wider tile)

// (lo, hi) -> two bf16 (RNE) in one dword, lo in the low half: v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

struct GemmParams {
    const uint8_t *w;
    const __bf16 *Xb;   // X rounded to bf16, [P padded to TOK_PAD][K], padding rows zero
    float *Y;
    int32_t M, K, P, nb;
    int64_t row_bytes;
    int32_t ks;
    float *ws;
};

// Eight weights q[0..7] (bytes of q0, q1) -> bf16 fragment of fma(q, ds, -dm).
// The f32 value is exact; each pair is rounded to bf16 (RNE) by one packed convert.
__device__ __forceinline__ bf16x8 dequant8(uint32_t q0, uint32_t q1, float ds, float dm) {
    uint4 r;
    r.x = pack_bf16(fmaf(ubyte(q0, 0), ds, -dm), fmaf(ubyte(q0, 1), ds, -dm));
    r.y = pack_bf16(fmaf(ubyte(q0, 2), ds, -dm), fmaf(ubyte(q0, 3), ds, -dm));
    r.z = pack_bf16(fmaf(ubyte(q1, 0), ds, -dm), fmaf(ubyte(q1, 1), ds, -dm));
    r.w = pack_bf16(fmaf(ubyte(q1, 2), ds, -dm), fmaf(ubyte(q1, 3), ds, -dm));
    return __builtin_bit_cast(bf16x8, r);
}

// Xb[t][k] = bf16(X[t][k]) for t < P, 0 for P <= t < Pp.  Four elements per thread.
__global__ __launch_bounds__(256) void to_bf16_kernel(const float *__restrict__ X,
                                                      __bf16 *__restrict__ Xb, int64_t n,
                                                      int64_t n_pad) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= n_pad) return;
    bf16x4 b;
    if (i + 3 < n) {
        const float4 v = *reinterpret_cast<const float4 *>(X + i);
        b[0] = (__bf16)v.x;
        b[1] = (__bf16)v.y;
        b[2] = (__bf16)v.z;
        b[3] = (__bf16)v.w;
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) b[e] = (__bf16)(i + e < n ? X[i + e] : 0.f);
    }
    *reinterpret_cast<bf16x4 *>(Xb + i) = b;
}

// W bytes of one super-block for one 32-row group: the block header and the
// lane's 16-byte halves of the four 32-byte quant groups.
struct WBlock {
    uint4 hdr, q[4];
};

// One workgroup: 256 W rows x 32T tokens.  See the file comment for the
// fragment layout.  Pipeline: while half-block step s is computed from one LDS
// buffer, the X slice of step s+1 is copied into the other buffer, and the W
// bytes of the next super-block are loaded into the other register set; the
// copies are spread over the step's MFMA blocks.
template <int T>
__global__ __launch_bounds__(256, 1) void gemm_kernel(const GemmParams p) {
    constexpr int BN = 32 * T;
    // buffer `half` holds X columns [256j + 128 half, +128) of the tile's tokens
    __shared__ __attribute__((aligned(1024))) __bf16 xs[2][BN * KS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rt = blockIdx.x, tt = blockIdx.y, split = blockIdx.z;
    const int row0 = rt * BM, tok0 = tt * BN;
    // K range of this split in whole super-blocks [jb, je)
    const int jb = (int)(((int64_t)split * p.nb) / p.ks);
    const int je = (int)(((int64_t)(split + 1) * p.nb) / p.ks);
    const int h = lane >> 5;

    // W row pointers of the lane's two row groups (rows past M clamp to M-1)
    const uint8_t *wr[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        int row = row0 + 64 * wave + 32 * r + (lane & 31);
        row = row < p.M ? row : p.M - 1;
        wr[r] = p.w + (int64_t)row * p.row_bytes;
    }

    // X copy: wave instruction i moves token rows 4b .. 4b+3 (b = 4i + wave),
    // 1 KB of LDS; lane L brings chunk (L & 15) ^ (t & 15) of token t = 4b + L/16.
    // (4b + L/16) & 15 = (4 * wave + L/16) & 15 because 4b - 4*wave = 16i.  The
    // per-lane part of the source address is a 32-bit byte offset; the rest is
    // wave-uniform.
    constexpr int XI = BN / 16;  // copy instructions per wave per half-block step
    const int t_in = lane >> 4;
    const uint32_t xoff =
        (uint32_t)(((4 * wave + t_in) * p.K + 8 * ((lane & 15) ^ ((4 * wave + t_in) & 15))) * 2);
    const char *xbase = reinterpret_cast<const char *>(p.Xb) + (int64_t)tok0 * p.K * 2;

    // X copy instruction i of step (j, half) into LDS buffer `half`, and W word
    // k (0: header, 1..4: quant group k-1) of super-block j, row group r, into
    // w.  Issued a few per MFMA block (see compute): a burst of them at once
    // stalls the wave on the memory pipeline's queue.
    auto copy_x = [&](int j, int half, int i) {
        const int64_t kbyte = ((int64_t)j * 256 + 128 * half) * 2;
        const int b = 4 * i + wave;
        const char *src = xbase + (int64_t)16 * i * p.K * 2 + kbyte;
        __builtin_amdgcn_global_load_lds((gvoid *)(src + xoff), (lvoid *)&xs[half][b * 4 * KS], 16,
                                         0, 0);
    };
    auto load_w = [&](int j, int r, int k, WBlock (&w)[2]) {
        const uint8_t *bp = wr[r] + (int64_t)j * kBlockBytes;
        if (k == 0) w[r].hdr = ldg16(bp);
        else w[r].q[k - 1] = ldg16(bp + 16 + 32 * (k - 1) + 16 * h);
    };

    // LDS offset of chunk kc of this lane's fragment row: slot kc ^ (lane & 15);
    // kc = 8gg + 4(f>>1) + 2h + (f&1) and bit 1 of the constant part is clear,
    // so kc ^ (lane & 15) = cst ^ m with m = 2h ^ (lane & 15).
    const int m = (2 * h) ^ (lane & 15);
    const int arow = (lane & 31) * KS;

    f32x16 acc[2][T];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int i = 0; i < T; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[r][i][v] = 0.f;

    // Half-block step (quant groups 2 half, 2 half + 1) from LDS buffer buf, in
    // eight blocks b = (gg, f): block b reads T A fragments (X at column offset
    // cst(b)) and dequantises two B fragments (one per row group), then issues
    // 2T MFMAs.  Block b+1's LDS reads and dequantisation are issued in the
    // shadow of block b's MFMAs (software pipeline).
    // While computing, block b also issues X copy instructions of step
    // (xj, 1 - half) into the other buffer and (b < 5) W word b of row group
    // `half` of super-block wj into wn.
    auto compute = [&](int half, const WBlock (&wc)[2], int xj, int wj, WBlock (&wn)[2]) {
        const __bf16 *xb = &xs[half][arow];
        float ds[2][2][2], dm[2][2][2];  // [gg][r][lo/hi sub-block]
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const float d = half_lo(wc[r].hdr.x), dmin = half_hi(wc[r].hdr.x);
            const Scales sc = unpack_scales(wc[r].hdr.y, wc[r].hdr.z, wc[r].hdr.w);
#pragma unroll
            for (int gg = 0; gg < 2; ++gg) {
                const int g = 2 * half + gg;
                ds[gg][r][0] = d * scale_of(sc, 2 * g);
                dm[gg][r][0] = dmin * min_of(sc, 2 * g);
                ds[gg][r][1] = d * scale_of(sc, 2 * g + 1);
                dm[gg][r][1] = dmin * min_of(sc, 2 * g + 1);
            }
        }
        auto load_a = [&](int b, bf16x8 (&A)[T]) {
            const int gg = b >> 2, f = b & 3;
            const int cst = 8 * gg + 4 * (f >> 1) + (f & 1);
            const __bf16 *xa = xb + 8 * (cst ^ m);
#pragma unroll
            for (int ti = 0; ti < T; ++ti)
                A[ti] = *reinterpret_cast<const bf16x8 *>(xa + ti * 32 * KS);
        };
        auto make_b = [&](int b, bf16x8 (&B)[2]) {
            const int gg = b >> 2, f = b & 3, hi = f >> 1;
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const uint4 q = wc[r].q[2 * half + gg];
                const uint32_t a0 = (f & 1) ? q.z : q.x, a1 = (f & 1) ? q.w : q.y;
                B[r] = dequant8(and_mask(hi ? a0 >> 4 : a0, 0x0F0F0F0Fu),
                                and_mask(hi ? a1 >> 4 : a1, 0x0F0F0F0Fu), ds[gg][r][hi],
                                dm[gg][r][hi]);
            }
        };
        bf16x8 A[2][T], B[2][2];
        load_a(0, A[0]);
        make_b(0, B[0]);
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const int c = b & 1;
#pragma unroll
            for (int i = b * XI / 8; i < (b + 1) * XI / 8; ++i) copy_x(xj, 1 - half, i);
            if (b < 5) load_w(wj, half, b, wn);
            if (b < 7) {
                load_a(b + 1, A[c ^ 1]);
                make_b(b + 1, B[c ^ 1]);
            }
#pragma unroll
            for (int ti = 0; ti < T; ++ti) {
                acc[0][ti] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[c][ti], B[c][0], acc[0][ti], 0, 0, 0);
                acc[1][ti] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[c][ti], B[c][1], acc[1][ti], 0, 0, 0);
            }
            if (b < 7) {
                // interleave: each MFMA pair carries one LDS read and a share of the VALU
#pragma unroll
                for (int ti = 0; ti < T; ++ti) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
                    __builtin_amdgcn_sched_group_barrier(0x002, 24 / T + 1, 0);  // VALU
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x002, 24 / T + 1, 0);  // VALU
                }
            }
            __builtin_amdgcn_sched_barrier(0);  // keep blocks in order
        }
    };

    // Super-blocks alternate between register sets wa and wb.  Copies past
    // the split's end re-read an in-range block (clamped) and are never used,
    // so the loop body has no branches.
    auto step_end = [&]() {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies have landed
        __syncthreads();
    };
    WBlock wa[2], wb[2];
    if (jb < je) {
#pragma unroll
        for (int i = 0; i < XI; ++i) copy_x(jb, 0, i);
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int k = 0; k < 5; ++k) load_w(jb, r, k, wa);
    }
    step_end();
    const int last = p.nb - 1;
    int j = jb;
    for (; j + 1 < je; j += 2) {
        const int j2 = j + 2 < p.nb ? j + 2 : last;
        compute(0, wa, j, j + 1, wb);
        step_end();
        compute(1, wa, j + 1, j + 1, wb);
        step_end();
        compute(0, wb, j + 1, j2, wa);
        step_end();
        compute(1, wb, j2, j2, wa);
        step_end();
    }
    if (j < je) {  // odd count: super-block je-1; its X half 0 and W (set wa) are in place
        compute(0, wa, j, j, wb);
        step_end();
        compute(1, wa, j, j, wb);
        step_end();
    }

    // ---- epilogue ----
    float *out = p.ks > 1 ? p.ws + (int64_t)split * p.P * p.M : p.Y;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int col = row0 + 64 * wave + 32 * r + (lane & 31);  // W row = Y column
        const bool col_ok = col < p.M;
#pragma unroll
        for (int ti = 0; ti < T; ++ti)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int tok = tok0 + 32 * ti + 8 * (v >> 2) + 4 * h + (v & 3);
                if (col_ok && tok < p.P) out[(int64_t)tok * p.M + col] = acc[r][ti][v];
            }
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
std::atomic<int> g_override_t{0};

int64_t padded_tokens(int64_t P) { return (P + TOK_PAD - 1) / TOK_PAD * TOK_PAD; }

}  // namespace

void set_gemm_override(int token_groups, int ks) {
    g_override_t = token_groups;
    g_override_ks = ks;
}

// Tile and split choice.  Every workgroup holds a CU to itself (LDS and
// register file), so the chip runs 256 workgroups at a time; the cost model
// counts rounds of 256 times the per-workgroup work (super-blocks per split
// times the measured time of one super-block for the tile width) plus the
// traffic of the split partials (written once, read once by the reduction),
// and picks the cheapest (tile width, split count).
GemmLaunch choose_gemm_launch(int64_t M, int64_t K, int64_t P) {
    const int64_t nb = K / 256;
    const int ot = g_override_t.load(), oks = g_override_ks.load();
    GemmLaunch best{1, 4};
    double best_cost = 1e300;
    for (int t : {4, 8}) {
        if (ot != 0 && t != ot) continue;
        const int64_t tiles = ((M + BM - 1) / BM) * ((P + 32 * t - 1) / (32 * t));
        const double sb_us = t == 8 ? 6.0 : 3.6;  // one super-block of one tile (measured)
        for (int64_t ks = 1; ks <= 16 && nb / ks >= 2; ++ks) {
            if (oks != 0 && ks != std::min<int64_t>(oks, nb)) continue;
            const int64_t rounds = (tiles * ks + 255) / 256;
            double cost = rounds * (double)((nb + ks - 1) / ks) * sb_us;
            if (ks > 1) cost += (double)(2 * ks + 1) * P * M * 4 / 5.0e6;  // bytes / (5 TB/s), in us
            if (cost < best_cost - 1e-9) {
                best_cost = cost;
                best.ks = (int)ks;
                best.r = t;
            }
        }
    }
    if (oks > 16 || (oks != 0 && nb / oks < 2)) best.ks = (int)std::min<int64_t>(oks, nb);
    return best;
}

size_t gemm_partial_floats(const GemmLaunch &L, int64_t M, int64_t P) {
    const size_t n = L.ks > 1 ? (size_t)L.ks * (size_t)P * (size_t)M : 0;
    return (n + 63) / 64 * 64;  // keeps the bf16 X section 256-byte aligned
}

size_t gemm_xb_floats(int64_t K, int64_t P) {
    // bf16 copy of X with the token count padded to the tile
    return (size_t)(padded_tokens(P) * K * 2 / 4);
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
    p.Y = Y;
    p.M = (int32_t)M;
    p.K = (int32_t)K;
    p.P = (int32_t)P;
    p.nb = (int32_t)(K / 256);
    p.row_bytes = (K / 256) * kBlockBytes;
    p.ks = L.ks;
    p.ws = ws.partials;
    // workspace: [split partials][bf16 X, tokens padded]
    __bf16 *xb = reinterpret_cast<__bf16 *>(ws.partials + gemm_partial_floats(L, M, P));
    p.Xb = xb;
    const int64_t n = P * K, n_pad = padded_tokens(P) * K;
    const int64_t cgroups = (n_pad / 4 + 255) / 256;
    if (cgroups > 0x7FFFFFFF) return fail(Q4K_EUNSUPPORTED, "gemm: X too large");
    hipLaunchKernelGGL(to_bf16_kernel, dim3((unsigned)cgroups), dim3(256), 0, stream, X, xb, n,
                       n_pad);
    Q4K_HIP(hipGetLastError());
    const int BN = 32 * L.r;
    const dim3 grid((unsigned)((M + BM - 1) / BM), (unsigned)((P + BN - 1) / BN), (unsigned)L.ks);
    if (grid.y > 65535 || grid.z > 65535)
        return fail(Q4K_EUNSUPPORTED, "gemm: P or split count too large");
    if (L.r == 8) hipLaunchKernelGGL(gemm_kernel<8>, grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL(gemm_kernel<4>, grid, dim3(256), 0, stream, p);
    Q4K_HIP(hipGetLastError());
    if (L.ks > 1) {
        const int64_t m = P * M;
        const int64_t groups = (m + 255) / 256;
        if (groups > 0x7FFFFFFF) return fail(Q4K_EUNSUPPORTED, "gemm: output too large");
        hipLaunchKernelGGL(gemm_reduce_kernel, dim3((unsigned)groups), dim3(256), 0, stream,
                           (const float *)ws.partials, Y, m, L.ks);
        Q4K_HIP(hipGetLastError());
    }
    return Q4K_OK;
}

}  // namespace q4k
