// q4k_gemm.hip — prefill GEMM Y[P][M] = X[P][K] * W^T on gfx950 bf16 MFMA.
//
// Prefill is the compute-bound phase ("Qwen3.6-27B on Apple M3 Pro — the
// llama.cpp parity bar", the prefill-loves-the-GPU argument; "Mac Qwen3.6-27B
// Metal Q4_K perf diagnosis", §2 prefill phases), so this is the one matmul
// that runs on the matrix cores: v_mfma_f32_32x32x16_bf16 with f32
// accumulation.
//
//  * For tiles of 64 or more tokens, X is rounded to bf16 once (round to
//    nearest even) by a prologue kernel into a workspace whose token count
//    is padded to the tile with zeros, so the main loop moves half the
//    bytes, spends no VALU on conversion and needs no token clamping.
//    32-token tiles (short prompts) read X in f32 and round it on its way
//    into LDS instead, which saves the prologue launch; the LDS contents
//    are the same bits either way.
//  * Workgroup tile: 256 W rows x (32 * T) tokens, T = 1, 2, 4 or 8 (the
//    narrow tiles serve short prompts: the dequantisation of a super-block
//    costs the same at every width, the MFMA work shrinks with it), four
//    waves, one workgroup
//    per CU.  Wave w owns W rows 64w .. 64w+63 (two 32-row groups) for all
//    tokens of the tile, so every W weight is dequantised exactly once per
//    tile and every X fragment read from LDS feeds two MFMAs.  The 32 * T
//    accumulator registers per 32x32 output block live in the AGPR file.
//  * K advances half a super-block (128 columns, quant groups g0, g0+1) per
//    step.  The step's X slice (32T tokens x 128 columns of bf16) is copied
//    from global memory straight into LDS with global_load_lds_dwordx4, so
//    it never occupies registers (32-token tiles: through registers, see
//    copy_x); it is double-buffered (256-token tiles) or
//    held in four buffers, both halves of the next super-block copied while
//    this one computes (narrower tiles: one wait per super-block).  Each token row is
//    256 bytes = 16 chunks of 16 bytes and chunk c of token t is stored at
//    slot c ^ (t & 15), so the 32 lanes of a fragment read (32 consecutive
//    tokens, one chunk) cover all banks.
//  * W never goes through LDS: lane l handles row l%32 of each of its row
//    groups and half h = l/32 of every 32-byte quant group.  Its 16 quant
//    bytes hold 16 low-nibble weights (sub-block 2g) and 16 high-nibble
//    weights (sub-block 2g+1); each run of 8 converts (w = d*sc*q - dmin*m,
//    exact in f32 by one v_fma_mix_f32 per weight, then bf16 RNE) into one B
//    fragment.  A fragment may pair any 8 columns per lane as long as X is
//    read at the same columns, so the lane's column offset is
//    64g + 32*hi + 16h + 8t and the A fragment (X) is read from LDS at that
//    offset.  The next step's W bytes
//    are loaded into registers while the current step computes.
//  * Output layout of the 32x32 MFMA: lane l holds column l%32 (a W row) and
//    rows 8(v/4) + 4(l/32) + v%4 (tokens) of accumulator v, so each store
//    instruction writes 32 consecutive floats of a token row.
//  * Stream-K scheduling: the (tile, super-block) work items, tile-major,
//    are cut into one equal contiguous range per workgroup (by default one
//    workgroup per CU), so every CU gets the same number of super-blocks
//    whatever the tile count.  A tile wholly inside a range is written to Y;
//    a range's first and last tile, when the range starts or ends inside
//    them, go to two partial slots of the workgroup, and a fix-up kernel adds
//    each cut tile's pieces in workgroup order (ascending K).  Deterministic;
//    no cross-workgroup synchronisation inside a kernel.
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
constexpr int TOK_PAD = 256;   // tokens the workspace's bf16 X copy is sized for (the widest tile)
#ifndef GEMM_T1_US
#define GEMM_T1_US 2.45
#endif
#ifndef GEMM_T2_US
#define GEMM_T2_US 3.45
#endif

// (lo, hi) -> two bf16 (RNE) in one dword, lo in the low half: v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Partition of the (tile, super-block) work items, tile-major.  Tile t covers
// W rows 256 (t mod rtiles) .. +255 and tokens BN (t div rtiles) .. +BN-1.
// With at least G tiles and a remainder, the first dp * G tiles are handed out
// whole (round r gives workgroup g tile r * G + g: written straight to Y), and
// only the rest, items [U0, U), is split into G equal contiguous stream-K
// ranges.  Otherwise dp = 0, U0 = 0 and all items are split.  Either way every
// workgroup gets the same number of super-blocks, and at most two partial
// tiles (its stream-K range's first and last).
struct SKUnits {
    int nb;       // super-blocks per row (work items per tile)
    int rtiles;   // 256-row tiles
    int64_t U;    // total work items = tiles * nb
    int G;        // workgroups
    int dp;       // whole-tile rounds before the stream-K part
    int64_t U0;   // first stream-K item = dp * G * nb
    __host__ __device__ __forceinline__ int64_t begin(int g) const {
        return U0 + (int64_t)g * (U - U0) / G;
    }
    // workgroup whose stream-K range contains item u (U0 <= u < U)
    __host__ __device__ __forceinline__ int owner(int64_t u) const {
        const int64_t n = U - U0;
        return (int)(((u - U0 + 1) * (int64_t)G + n - 1) / n - 1);
    }
};

struct GemmParams {
    const uint8_t *w;
    const __bf16 *Xb;   // X rounded to bf16, [P rounded up to the tile][K], padding rows zero
    const float *X;     // X itself, [P][K] (read directly by 32-token tiles)
    float *Y;
    int32_t M, K, P, nb;
    int64_t row_bytes;
    int32_t ks;
    float *ws;
};

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// Eight weights of one fragment from quant words a0, a1 (bytes 0..3 of each,
// in K order): the nibbles of bytes 0 and 2, then of bytes 1 and 3, are put
// in the two 16-bit halves of a dword by one AND each (mask 0x000F000F for the
// low nibbles, 0x00F000F0 for the high ones, kept in place as 16 q).  Read as
// binary16, a half holding c is the subnormal c * 2^-24, so with
// a = d*sc*2^24 (low) or d*sc*2^20 (high) and b = -dmin*m one v_fma_mix_f32
// gives d*sc*q - dmin*m rounded once: the product is exact, so the value is
// bit for bit fmaf(q, d*sc, -dmin*m).  That is 2.25 VALU instructions per
// weight with the pack below, against 2.9 for a byte-to-float convert and an
// FMA per weight.
__device__ __forceinline__ void weights8(uint32_t a0, uint32_t a1, uint32_t mask, float a,
                                         float b, float (&w)[8]) {
    const half2v e0 = __builtin_bit_cast(half2v, and_mask(a0, mask));
    const half2v o0 = __builtin_bit_cast(half2v, and_mask(a0 >> 8, mask));
    const half2v e1 = __builtin_bit_cast(half2v, and_mask(a1, mask));
    const half2v o1 = __builtin_bit_cast(half2v, and_mask(a1 >> 8, mask));
    w[0] = fmaf((float)e0.x, a, b);
    w[1] = fmaf((float)o0.x, a, b);
    w[2] = fmaf((float)e0.y, a, b);
    w[3] = fmaf((float)o0.y, a, b);
    w[4] = fmaf((float)e1.x, a, b);
    w[5] = fmaf((float)o1.x, a, b);
    w[6] = fmaf((float)e1.y, a, b);
    w[7] = fmaf((float)o1.y, a, b);
}

// Eight exact weights -> one bf16 B fragment (RNE, one packed convert per
// pair).  make_b forms both row groups' weights before packing either, so no
// convert directly follows the v_fma_mix_f32 it reads (a wait state each on
// gfx950).
__device__ __forceinline__ bf16x8 pack8(const float (&w)[8]) {
    uint4 r;
    r.x = pack_bf16(w[0], w[1]);
    r.y = pack_bf16(w[2], w[3]);
    r.z = pack_bf16(w[4], w[5]);
    r.w = pack_bf16(w[6], w[7]);
    return __builtin_bit_cast(bf16x8, r);
}

// Xb[t][k] = bf16(X[t][k]) for t < P, 0 for P <= t < Pp.  Eight elements per
// thread (two 16-byte loads, one 16-byte store); n_pad is a multiple of 8.
__global__ __launch_bounds__(256) void to_bf16_kernel(const float *__restrict__ X,
                                                      __bf16 *__restrict__ Xb, int64_t n,
                                                      int64_t n_pad) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (i >= n_pad) return;
    bf16x8 b;
    if (i + 7 < n) {
        const float4 v0 = *reinterpret_cast<const float4 *>(X + i);
        const float4 v1 = *reinterpret_cast<const float4 *>(X + i + 4);
        b[0] = (__bf16)v0.x;
        b[1] = (__bf16)v0.y;
        b[2] = (__bf16)v0.z;
        b[3] = (__bf16)v0.w;
        b[4] = (__bf16)v1.x;
        b[5] = (__bf16)v1.y;
        b[6] = (__bf16)v1.z;
        b[7] = (__bf16)v1.w;
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) b[e] = (__bf16)(i + e < n ? X[i + e] : 0.f);
    }
    *reinterpret_cast<bf16x8 *>(Xb + i) = b;
}

// W bytes of one super-block for one 32-row group: the block header and the
// lane's 16-byte halves of the four 32-byte quant groups.
struct WBlock {
    uint4 hdr, q[4];
};

// One workgroup: 256 W rows x 32T tokens.  See the file comment for the
// fragment layout.  Pipeline: while a half-block step is computed from one LDS
// buffer, the X slice of a later step is copied into another buffer, and the W
// bytes of the next super-block are loaded into the other register set; the
// copies are spread over the step's MFMA blocks.
// One segment: super-blocks [jb, je) of tile `tile`.  A whole tile is written
// to Y; a part of a tile goes to the workgroup's partial slot (0: the first
// tile of its range, 1: the last) for the fix-up kernel.  xs: the LDS X
// buffers (BN tokens x 128 columns each; two or four, see NBUF).
template <int T>
__device__ __forceinline__ void gemm_segment(const GemmParams &p, const SKUnits &su, int g,
                                             int tile, int jb, int je, int slot,
                                             __bf16 (*xs)[32 * T * KS]) {
    // X buffers: two (half-blocks alternate) for 256-token tiles; four for
    // narrower tiles (buffer 2 (j mod 2) + half: both halves of the next
    // super-block are copied while this one computes, one wait per super-block)
    constexpr int NBUF = T <= 4 ? 4 : 2;
    constexpr int BN = 32 * T;
    // opaque per segment: nothing derived from the thread index is hoisted out
    // of the caller's segment loop and kept live across the main loop
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rt = tile % su.rtiles, tt = tile / su.rtiles;
    const int row0 = rt * BM, tok0 = tt * BN;
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
    // 32-token tiles read X in f32 and round it to bf16 on its way into LDS,
    // so no separate rounding launch precedes them: each copy instruction
    // becomes two 16-byte loads into registers (token rows past P load row
    // P-1 and are zeroed), and step_end converts them and writes the 16
    // bytes the DMA would have written, once the step's loads have landed.
    constexpr bool XF = T == 1;
    constexpr int XS = XF ? 2 * XI : 1;  // copies staged per super-block
    const int cx = (lane & 15) ^ ((4 * wave + t_in) & 15);
    float4 xst[XS][2];
    auto copy_x = [&](int j, int half, int buf, int i) {
        if constexpr (XF) {
            const int t = tok0 + 16 * i + 4 * wave + t_in;
            const float *src = p.X + (int64_t)(t < p.P ? t : p.P - 1) * p.K + j * 256 +
                               128 * half + 8 * cx;
            xst[half * XI + i][0] = *reinterpret_cast<const float4 *>(src);
            xst[half * XI + i][1] = *reinterpret_cast<const float4 *>(src + 4);
        } else {
            const int64_t kbyte = ((int64_t)j * 256 + 128 * half) * 2;
            const int b = 4 * i + wave;
            const char *src = xbase + (int64_t)16 * i * p.K * 2 + kbyte;
            __builtin_amdgcn_global_load_lds((gvoid *)(src + xoff), (lvoid *)&xs[buf][b * 4 * KS],
                                             16, 0, 0);
        }
    };
    // staged copies of the two halves -> LDS buffers cb and cb + 1
    auto flush_x = [&](int cb) {
        if constexpr (XF) {
#pragma unroll
            for (int half = 0; half < 2; ++half)
#pragma unroll
                for (int i = 0; i < XI; ++i) {
                    const int b = 4 * i + wave;
                    const bool in = tok0 + 4 * b + t_in < p.P;
                    const float4 u = xst[half * XI + i][0], v = xst[half * XI + i][1];
                    uint4 r;
                    r.x = in ? pack_bf16(u.x, u.y) : 0u;
                    r.y = in ? pack_bf16(u.z, u.w) : 0u;
                    r.z = in ? pack_bf16(v.x, v.y) : 0u;
                    r.w = in ? pack_bf16(v.z, v.w) : 0u;
                    *reinterpret_cast<uint4 *>(&xs[cb + half][b * 4 * KS + 8 * lane]) = r;
                }
        }
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

    // Half-block step `half` (quant groups 2 half, 2 half + 1) from LDS buffer
    // rbuf, in eight blocks b = (gg, f): block b reads T A fragments (X at
    // column offset cst(b)) and dequantises two B fragments (one per row
    // group), then issues 2T MFMAs.  Block b+1's LDS reads and dequantisation
    // are issued in the shadow of block b's MFMAs (software pipeline).
    // While computing, block b also issues X copy instructions of step
    // (cj, chalf) into buffer cbuf and (b < 5) W word b of row group `half` of
    // super-block wj into wn.
    auto compute = [&](int half, const WBlock (&wc)[2], int rbuf, int cj, int chalf, int cbuf,
                       int wj, WBlock (&wn)[2]) {
        const __bf16 *xb = &xs[rbuf][arow];
        // per sub-block: a = d*sc*2^24 (low nibbles) or d*sc*2^20 (high), b = -dmin*m
        float ds[2][2][2], dm[2][2][2];  // [gg][r][lo/hi sub-block]
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const float d = half_lo(wc[r].hdr.x), ndmin = -half_hi(wc[r].hdr.x);
            const float d24 = d * 16777216.f, d20 = d * 1048576.f;
            const Scales sc = unpack_scales(wc[r].hdr.y, wc[r].hdr.z, wc[r].hdr.w);
#pragma unroll
            for (int gg = 0; gg < 2; ++gg) {
                const int g = 2 * half + gg;
                ds[gg][r][0] = d24 * scale_of(sc, 2 * g);
                dm[gg][r][0] = ndmin * min_of(sc, 2 * g);
                ds[gg][r][1] = d20 * scale_of(sc, 2 * g + 1);
                dm[gg][r][1] = ndmin * min_of(sc, 2 * g + 1);
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
            float wf[2][8];
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const uint4 q = wc[r].q[2 * half + gg];
                const uint32_t a0 = (f & 1) ? q.z : q.x, a1 = (f & 1) ? q.w : q.y;
                weights8(a0, a1, hi ? 0x00F000F0u : 0x000F000Fu, ds[gg][r][hi], dm[gg][r][hi],
                         wf[r]);
            }
            B[0] = pack8(wf[0]);
            B[1] = pack8(wf[1]);
        };
        bf16x8 A[2][T], B[2][2];
        load_a(0, A[0]);
        make_b(0, B[0]);
        // Block 0's LDS reads issue together: left to itself the scheduler
        // sinks each next to its MFMA and waits for them one at a time.
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const int c = b & 1;
#pragma unroll
            for (int i = b * XI / 8; i < (b + 1) * XI / 8; ++i) copy_x(cj, chalf, cbuf, i);
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
                // interleave: the next block's T LDS reads ride on the first T
                // MFMAs (so they land before the block ends) and every MFMA
                // carries a share of the VALU
#pragma unroll
                for (int i = 0; i < 2 * T; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                    if (i < T) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
                    __builtin_amdgcn_sched_group_barrier(0x002, 24 / T + 1, 0);  // VALU
                }
            }
            __builtin_amdgcn_sched_barrier(0);  // keep blocks in order
        }
    };

    // Super-blocks alternate between register sets wa and wb.  Copies past
    // the split's end re-read an in-range block (clamped) and are never used,
    // so the loop body has no branches.
    auto step_end = [&](int cb) {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies have landed
        flush_x(cb);
        __syncthreads();
    };
    WBlock wa[2], wb[2];
    if (jb < je) {
#pragma unroll
        for (int i = 0; i < XI; ++i) copy_x(jb, 0, NBUF == 4 ? 2 * (jb & 1) : 0, i);
        if constexpr (NBUF == 4) {
#pragma unroll
            for (int i = 0; i < XI; ++i) copy_x(jb, 1, 2 * (jb & 1) + 1, i);
        }
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int k = 0; k < 5; ++k) load_w(jb, r, k, wa);
    }
    step_end(NBUF == 4 ? 2 * (jb & 1) : 0);
    const int last = p.nb - 1;
    int j = jb;
    if constexpr (NBUF == 4) {
        // super-block j reads buffers 2 (j & 1) + h and fills those of j + 1
        // (copies past the segment's end re-read an in-range block, unused)
        for (; j + 1 < je; j += 2) {
            const int j1 = j + 1, j2 = j + 2 < p.nb ? j + 2 : last;
            const int bj = 2 * (j & 1), bn = 2 - bj;
            compute(0, wa, bj, j1, 0, bn, j1, wb);
            compute(1, wa, bj + 1, j1, 1, bn + 1, j1, wb);
            step_end(bn);
            compute(0, wb, bn, j2, 0, bj, j2, wa);
            compute(1, wb, bn + 1, j2, 1, bj + 1, j2, wa);
            step_end(bj);
        }
        if (j < je) {  // odd count: super-block je-1 (X and W set wa in place)
            const int bj = 2 * (j & 1), bn = 2 - bj;
            compute(0, wa, bj, j, 0, bn, j, wb);
            compute(1, wa, bj + 1, j, 1, bn + 1, j, wb);
            step_end(bn);
        }
    } else {
        for (; j + 1 < je; j += 2) {
            const int j2 = j + 2 < p.nb ? j + 2 : last;
            compute(0, wa, 0, j, 1, 1, j + 1, wb);
            step_end(0);
            compute(1, wa, 1, j + 1, 0, 0, j + 1, wb);
            step_end(0);
            compute(0, wb, 0, j + 1, 1, 1, j2, wa);
            step_end(0);
            compute(1, wb, 1, j2, 0, 0, j2, wa);
            step_end(0);
        }
        if (j < je) {  // odd count: super-block je-1; its X half 0 and W (set wa) are in place
            compute(0, wa, 0, j, 1, 1, j, wb);
            step_end(0);
            compute(1, wa, 1, j, 0, 0, j, wb);
            step_end(0);
        }
    }

    // ---- epilogue ----
    // A whole tile goes to Y; a part of one to the partial slot, laid out
    // [token][column] like Y's tile with a row stride of BM.
    const bool whole = jb == 0 && je == p.nb;
    float *out = whole ? p.Y + (int64_t)tok0 * p.M + row0
                       : p.ws + ((int64_t)g * 2 + slot) * (BM * BN);
    const int ld = whole ? p.M : BM;
    const int cmax = whole ? p.M - row0 : BM, tmax = whole ? p.P - tok0 : BN;
    if (cmax >= BM && tmax >= BN) {
        // Every element of the tile is in range (partial slots always are):
        // no per-element conditions.  Each store takes a wave-uniform token row
        // base (scalar adds) plus the lane's fixed 32-bit byte offset (its
        // column, and 4 token rows further for the upper half-wave); the
        // condition-guarded form below spends a branch, a 64-bit multiply and
        // an exec-mask spill on every store.
        const uint32_t lofs = (uint32_t)((4 * h * ld + 64 * wave + (lane & 31)) * 4);
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int ti = 0; ti < T; ++ti)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int tu = 32 * ti + 8 * (v >> 2) + (v & 3);  // uniform token row
                    char *rowp = reinterpret_cast<char *>(out + (int64_t)tu * ld + 32 * r);
                    *reinterpret_cast<float *>(rowp + lofs) = acc[r][ti][v];
                }
        return;
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int cl = 64 * wave + 32 * r + (lane & 31);  // W row = Y column
        const bool col_ok = cl < cmax;
#pragma unroll
        for (int ti = 0; ti < T; ++ti)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int tl = 32 * ti + 8 * (v >> 2) + 4 * h + (v & 3);
                if (col_ok && tl < tmax) out[(int64_t)tl * ld + cl] = acc[r][ti][v];
            }
    }
}

template <int T>
__global__ __launch_bounds__(256, 1) void gemm_kernel(const GemmParams p, const SKUnits su) {
    // X buffers of the tile's tokens, 128 columns (half a super-block) each
    __shared__ __attribute__((aligned(1024))) __bf16 xs[T <= 4 ? 4 : 2][32 * T * KS];
    const int g = blockIdx.x;
    // the whole tiles of the data-parallel rounds and the stream-K range's
    // segments: even workgroups take the whole tiles first, odd ones the
    // stream-K range first, so that the tile stores of the two halves of the
    // grid do not all fall at the same moment.  One call site, so the segment
    // body is inlined once.
    const int64_t ua = su.begin(g), ub = su.begin(g + 1);
    const int first_tile = (int)(ua / su.nb);
    const bool sk_first = (g & 1) != 0;
    int r = 0;
    int64_t u = ua;
    while (true) {
        int tile, jb, je;
        if (r < su.dp && !(sk_first && u < ub)) {
            tile = r * su.G + g;
            jb = 0;
            je = su.nb;
            ++r;
        } else if (u < ub) {
            tile = (int)(u / su.nb);
            const int64_t tb = (int64_t)tile * su.nb;
            jb = (int)(u - tb);
            je = (int)((ub < tb + su.nb ? ub : tb + su.nb) - tb);
            u = tb + je;
        } else if (r < su.dp) {
            tile = r * su.G + g;
            jb = 0;
            je = su.nb;
            ++r;
        } else {
            break;
        }
        gemm_segment<T>(p, su, g, tile, jb, je, tile == first_tile ? 0 : 1, xs);
    }
}

// Cut tiles: Y = sum of the contributors' partial tiles, in workgroup order
// (ascending K).  by_tile: blockIdx.x is a tile of the stream-K part (fewer
// such tiles than range boundaries), and a tile inside one range exits.
// Otherwise blockIdx.x + 1 = range boundary b; the tile it falls in is fixed
// up by the first boundary that cuts it.  Either way whole tiles do nothing
// and no tile is done twice.  blockIdx.y: FT tokens of the tile; thread: one
// column, FT independent loads per contributor.
constexpr int FT = 8;
template <int T>
__global__ __launch_bounds__(256) void gemm_fixup_kernel(const GemmParams p, const SKUnits su,
                                                         int by_tile) {
    constexpr int BN = 32 * T;
    int tile;
    int64_t tb;
    if (by_tile) {
        tile = (int)(su.U0 / su.nb) + (int)blockIdx.x;
        tb = (int64_t)tile * su.nb;
    } else {
        const int bnd = blockIdx.x + 1;
        const int64_t ub = su.begin(bnd);
        tile = (int)(ub / su.nb);
        tb = (int64_t)tile * su.nb;
        if (ub == tb || su.begin(bnd - 1) > tb) return;  // not a cut, or cut by an earlier boundary
    }
    const int gf = su.owner(tb), gl = su.owner(tb + su.nb - 1);
    if (gf == gl) return;  // inside one range: written to Y by its workgroup
    const int rt = tile % su.rtiles, tt = tile / su.rtiles;
    const int cl = threadIdx.x;  // column of the tile
    const int col = rt * BM + cl;
    const int tl0 = blockIdx.y * FT;
    const int tok0 = tt * BN + tl0;
    if (col >= p.M || tok0 >= p.P) return;
    float s[FT];
#pragma unroll
    for (int i = 0; i < FT; ++i) s[i] = 0.f;
    // FC contributors per round with all their loads in flight together: a
    // tile cut among many workgroups (a long K on few tiles) would otherwise
    // pay one memory round trip per contributor.  Additions stay in
    // contributor order.
    constexpr int FC = 4;
    for (int w0 = gf; w0 <= gl; w0 += FC) {
        float v[FC][FT];
#pragma unroll
        for (int c = 0; c < FC; ++c) {
            const int w = w0 + c <= gl ? w0 + c : gl;  // past gl: loaded, not added
            const int slot = su.begin(w) / su.nb == tile ? 0 : 1;
            const float *src = p.ws + ((int64_t)w * 2 + slot) * (BM * BN) + (int64_t)tl0 * BM + cl;
#pragma unroll
            for (int i = 0; i < FT; ++i) v[c][i] = src[i * BM];
        }
#pragma unroll
        for (int c = 0; c < FC; ++c)
            if (w0 + c <= gl) {
#pragma unroll
                for (int i = 0; i < FT; ++i) s[i] += v[c][i];
            }
    }
#pragma unroll
    for (int i = 0; i < FT; ++i)
        if (tok0 + i < p.P) p.Y[(int64_t)(tok0 + i) * p.M + col] = s[i];
}

std::atomic<int> g_override_ks{0};
std::atomic<int> g_override_t{0};

int64_t padded_tokens(int64_t P) { return (P + TOK_PAD - 1) / TOK_PAD * TOK_PAD; }

// tokens the bf16 X copy holds for tiles of 32 r tokens: P rounded up to the
// tile (at most padded_tokens(P), what the workspace is sized for)
int64_t filled_tokens(int64_t P, int r) { return (P + 32 * r - 1) / (32 * r) * (32 * r); }

}  // namespace

void set_gemm_override(int token_groups, int workgroups) {
    g_override_t = token_groups;
    g_override_ks = workgroups;
}

// Tile choice and grid.  Every workgroup holds a CU to itself (LDS and
// register file), so the grid is one workgroup per CU and the stream-K
// partition gives each the same number of super-block items.  The cost model
// per tile width: items per workgroup times the measured time of one item,
// plus the traffic of the partial tiles (each workgroup writes at most two,
// the fix-up kernel reads them back) and the fix-up launch.
namespace {
int device_cus() {
    static std::atomic<int> cached{0};
    int c = cached.load();
    if (c > 0) return c;
    int dev = 0;
    c = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            v > 0)
            c = v;
    }
    cached = c;
    return c;
}

SKUnits sk_units(int64_t M, int64_t K, int64_t P, int t, int G) {
    SKUnits su;
    su.nb = (int)(K / 256);
    su.rtiles = (int)((M + BM - 1) / BM);
    const int64_t tiles = (int64_t)su.rtiles * ((P + 32 * t - 1) / (32 * t));
    su.U = tiles * su.nb;
    su.G = (int)std::max<int64_t>(1, std::min<int64_t>(G, su.U));
    su.dp = 0;
    su.U0 = 0;
    // whole-tile rounds when there are at least G tiles, a remainder, and
    // enough remaining items to give every workgroup one (no empty ranges)
    const int64_t rem = tiles % su.G;
    if (tiles > su.G && rem != 0 && rem * su.nb >= su.G && tiles / su.G <= 0x7FFFFFFF) {
        su.dp = (int)(tiles / su.G);
        su.U0 = (int64_t)su.dp * su.G * su.nb;
    }
    return su;
}

// A range boundary falls inside a tile unless every range is whole tiles.
bool has_split_tiles(const SKUnits &su) {
    const int64_t tiles = (su.U - su.U0) / su.nb;
    return !(tiles % su.G == 0);
}
}  // namespace

// Partial tiles the workgroups write (a range's first and last tile when the
// range starts or ends inside it), and how many tiles need the fix-up.
static void split_pieces(const SKUnits &su, int64_t &pieces, int64_t &split_tiles) {
    pieces = 0;
    split_tiles = 0;
    int64_t last_split = -1;
    for (int g = 0; g < su.G; ++g) {
        const int64_t ua = su.begin(g), ub = su.begin(g + 1);
        if (ua >= ub) continue;
        const int64_t t0 = ua / su.nb, t1 = (ub - 1) / su.nb;
        const bool cut0 = ua % su.nb != 0 || (t0 == t1 && ub % su.nb != 0);
        const bool cut1 = t1 != t0 && ub % su.nb != 0;
        if (cut0) {
            ++pieces;
            if (t0 != last_split) ++split_tiles, last_split = t0;
        }
        if (cut1) {
            ++pieces;
            if (t1 != last_split) ++split_tiles, last_split = t1;
        }
    }
}

// Tile width and workgroup count.  Every workgroup holds a CU to itself (LDS
// and register file).  The cost model takes the longest range (work items,
// whole-tile rounds included, times the time of one super-block of one tile
// at that width), plus, when some tile is cut, the partial tiles a workgroup
// writes (about 48 GB/s per CU with every CU writing) and the fix-up launch
// with its traffic (partials read, Y written; about 12 TB/s, the partials
// being still in cache).  The constants are a least-squares fit to measured
// calls at 128 and 256 tokens on both MLP shapes at P = 256, 512 and 1024,
// constrained to rank the two widths as the measurements do.
GemmLaunch choose_gemm_launch(int64_t M, int64_t K, int64_t P) {
    const int ot = g_override_t.load(), og = g_override_ks.load();
    const int G = og > 0 ? og : device_cus();
    GemmLaunch best{G, 4};
    double best_cost = 1e300;
    for (int t : {1, 2, 4, 8}) {
        if (ot != 0 && t != ot) continue;
        const SKUnits su = sk_units(M, K, P, t, G);
        // one super-block of one tile (measured): the dequantisation costs the
        // same at every width, the MFMA work grows with it
        const double item_us = t == 8 ? 6.9 : t == 4 ? 4.2 : t == 2 ? GEMM_T2_US : GEMM_T1_US;
        const int64_t per = (int64_t)su.dp * su.nb + (su.U - su.U0 + su.G - 1) / su.G;
        double cost = per * item_us;
        if (has_split_tiles(su)) {
            int64_t pieces, split_tiles;
            split_pieces(su, pieces, split_tiles);
            const double tile_bytes = (double)BM * 32 * t * 4;
            cost += (double)(pieces + su.G - 1) / su.G * tile_bytes / 48.0e3 + 3.0 +
                    (double)(pieces + split_tiles) * tile_bytes / 12.0e6;
        }
        if (cost < best_cost - 1e-9) {
            best_cost = cost;
            best.ks = su.G;
            best.r = t;
        }
    }
    return best;
}

size_t gemm_partial_floats(const GemmLaunch &L, int64_t M, int64_t P) {
    (void)M;
    (void)P;
    // two partial tiles per workgroup, rounded to 64 floats (keeps the bf16 X
    // section after it 256-byte aligned)
    const size_t n = (size_t)L.ks * 2 * BM * 32 * L.r;
    return (n + 63) / 64 * 64;
}

size_t gemm_xb_floats(int64_t K, int64_t P) {
    // bf16 copy of X with the token count padded to the widest tile
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
    // workspace: [partial tiles][bf16 X, tokens rounded up to the tile]
    __bf16 *xb = reinterpret_cast<__bf16 *>(ws.partials + gemm_partial_floats(L, M, P));
    p.Xb = xb;
    p.X = X;
    if (L.r != 1) {  // 32-token tiles round X themselves
        const int64_t n = P * K, n_pad = filled_tokens(P, L.r) * K;
        const int64_t cgroups = (n_pad / 8 + 255) / 256;
        if (cgroups > 0x7FFFFFFF) return fail(Q4K_EUNSUPPORTED, "gemm: X too large");
        hipLaunchKernelGGL(to_bf16_kernel, dim3((unsigned)cgroups), dim3(256), 0, stream, X, xb,
                           n, n_pad);
        Q4K_HIP(hipGetLastError());
    }
    const SKUnits su = sk_units(M, K, P, L.r, L.ks);
    const int64_t tiles = su.U / su.nb;
    if (tiles > 0x7FFFFFFF) return fail(Q4K_EUNSUPPORTED, "gemm: too many tiles");
    const dim3 gg((unsigned)su.G);
    switch (L.r) {
        case 8: hipLaunchKernelGGL(gemm_kernel<8>, gg, dim3(256), 0, stream, p, su); break;
        case 4: hipLaunchKernelGGL(gemm_kernel<4>, gg, dim3(256), 0, stream, p, su); break;
        case 2: hipLaunchKernelGGL(gemm_kernel<2>, gg, dim3(256), 0, stream, p, su); break;
        case 1: hipLaunchKernelGGL(gemm_kernel<1>, gg, dim3(256), 0, stream, p, su); break;
        default: return fail(Q4K_EINVAL, "gemm: tile of %d token groups", L.r);
    }
    Q4K_HIP(hipGetLastError());
    if (has_split_tiles(su)) {  // implies G >= 2: there are G - 1 range boundaries
        // one x-group per stream-K tile when they are fewer than the boundaries
        const int64_t sk_tiles = (su.U - su.U0) / su.nb;
        const int by_tile = sk_tiles < su.G - 1 ? 1 : 0;
        const dim3 fg((unsigned)(by_tile ? sk_tiles : su.G - 1), (unsigned)(32 * L.r / FT));
        switch (L.r) {
            case 8: hipLaunchKernelGGL(gemm_fixup_kernel<8>, fg, dim3(256), 0, stream, p, su, by_tile); break;
            case 4: hipLaunchKernelGGL(gemm_fixup_kernel<4>, fg, dim3(256), 0, stream, p, su, by_tile); break;
            case 2: hipLaunchKernelGGL(gemm_fixup_kernel<2>, fg, dim3(256), 0, stream, p, su, by_tile); break;
            default: hipLaunchKernelGGL(gemm_fixup_kernel<1>, fg, dim3(256), 0, stream, p, su, by_tile); break;
        }
        Q4K_HIP(hipGetLastError());
    }
    return Q4K_OK;
}

// Host-side check of a GEMM launch's stream-K partition, with the kernels'
// own range and owner arithmetic (SKUnits): contiguous non-empty ranges
// covering every work item once; the segments a workgroup walks (as
// gemm_kernel does) write at most one partial tile per slot, inside the
// partial area the launch reserves, and read only token rows inside the
// padded bf16 X copy; every tile the fix-up sums has consecutive
// contributors that all wrote a partial of it, in the slot the fix-up reads.
int check_gemm_partition(int64_t M, int64_t K, int64_t P, int tile_tokens, int groups) {
    if (M <= 0 || K <= 0 || K % 256 != 0 || P <= 0)
        return fail(Q4K_EINVAL, "check: bad arguments");
    GemmLaunch L = choose_gemm_launch(M, K, P);
    if (tile_tokens > 0) L.r = tile_tokens / 32;
    if (groups > 0) L.ks = groups;
    if (L.r != 1 && L.r != 2 && L.r != 4 && L.r != 8)
        return fail(Q4K_EINVAL, "check: tile of %d tokens", 32 * L.r);
    const SKUnits su = sk_units(M, K, P, L.r, L.ks);
    const int64_t BN = 32 * L.r, tile_floats = (int64_t)BM * BN;
    const int64_t partials = (int64_t)gemm_partial_floats(L, M, P);
    const int64_t ptok = filled_tokens(P, L.r);
    if (ptok > padded_tokens(P) || (int64_t)gemm_xb_floats(K, P) * 2 < ptok * K)
        return fail(Q4K_EINVAL, "check: bf16 X copy smaller than its padded tokens");
    if (su.U0 != (int64_t)su.dp * su.G * su.nb || su.U0 > su.U || su.U0 % su.nb != 0)
        return fail(Q4K_EINVAL, "check: %d whole-tile rounds do not end at item %lld",
                    su.dp, (long long)su.U0);
    // whole tiles r * G + g of the data-parallel rounds: in range, tokens
    // inside the padded copy, written straight to Y (no partial slot)
    for (int r = 0; r < su.dp; ++r)
        for (int g = 0; g < su.G; ++g) {
            const int64_t tile = (int64_t)r * su.G + g;
            if ((tile + 1) * su.nb > su.U0)
                return fail(Q4K_EINVAL, "check: round %d tile %lld past the rounds", r,
                            (long long)tile);
            if ((tile / su.rtiles + 1) * BN > ptok)
                return fail(Q4K_EINVAL, "check: tile %lld reads tokens past the padded copy",
                            (long long)tile);
        }
    int64_t prev = su.U0;
    for (int g = 0; g < su.G; ++g) {
        const int64_t ua = su.begin(g), ub = su.begin(g + 1);
        if (ua != prev || ub <= ua)
            return fail(Q4K_EINVAL, "check: range of workgroup %d is [%lld, %lld)", g,
                        (long long)ua, (long long)ub);
        prev = ub;
        if (su.owner(ua) != g || su.owner(ub - 1) != g)
            return fail(Q4K_EINVAL, "check: owner() disagrees with begin() at workgroup %d", g);
        const int64_t first_tile = ua / su.nb;
        int used[2] = {0, 0};
        for (int64_t u = ua; u < ub;) {
            const int64_t tile = u / su.nb, tb = tile * su.nb;
            const int64_t je = std::min<int64_t>(ub, tb + su.nb) - tb, jb = u - tb;
            const int64_t tt = tile / su.rtiles;
            if ((tt + 1) * BN > ptok)
                return fail(Q4K_EINVAL, "check: tile %lld reads tokens past the padded copy",
                            (long long)tile);
            if (!(jb == 0 && je == su.nb)) {
                const int slot = tile == first_tile ? 0 : 1;
                if (++used[slot] > 1)
                    return fail(Q4K_EINVAL, "check: workgroup %d writes slot %d twice", g, slot);
                if (((int64_t)g * 2 + slot + 1) * tile_floats > partials)
                    return fail(Q4K_EINVAL, "check: partial slot of workgroup %d outside", g);
            }
            u = tb + je;
        }
    }
    if (prev != su.U) return fail(Q4K_EINVAL, "check: ranges end at %lld of %lld items",
                                  (long long)prev, (long long)su.U);
    // the fix-up's two views (per range boundary, per stream-K tile) must
    // find the same cut tiles, each read from contributors that wrote it
    auto check_cut = [&](int64_t tile) -> int {
        const int64_t tb = tile * su.nb;
        const int gf = su.owner(tb), gl = su.owner(tb + su.nb - 1);
        if (gf >= gl) return fail(Q4K_EINVAL, "check: cut tile %lld has one contributor",
                                  (long long)tile);
        for (int w = gf; w <= gl; ++w) {
            const int64_t a = su.begin(w), b = su.begin(w + 1);
            const int slot = a / su.nb == tile ? 0 : 1;
            const bool wrote = a < tb + su.nb && b > tb && !(a <= tb && b >= tb + su.nb);
            const bool slot_ok = slot == 0 ? a >= tb : (a < tb && (b - 1) / su.nb == tile);
            if (!wrote || !slot_ok)
                return fail(Q4K_EINVAL, "check: fix-up of tile %lld reads workgroup %d slot %d "
                            "that it did not write", (long long)tile, w, slot);
        }
        return Q4K_OK;
    };
    int64_t cut_by_boundary = 0, cut_by_tile = 0;
    for (int bnd = 1; bnd < su.G; ++bnd) {
        const int64_t ub = su.begin(bnd), tile = ub / su.nb, tb = tile * su.nb;
        if (ub == tb || su.begin(bnd - 1) > tb) continue;
        if (int rc = check_cut(tile)) return rc;
        ++cut_by_boundary;
    }
    for (int64_t tile = su.U0 / su.nb; tile < su.U / su.nb; ++tile) {
        const int64_t tb = tile * su.nb;
        if (su.owner(tb) == su.owner(tb + su.nb - 1)) continue;
        if (int rc = check_cut(tile)) return rc;
        ++cut_by_tile;
    }
    if (cut_by_boundary != cut_by_tile)
        return fail(Q4K_EINVAL, "check: %lld tiles cut by range boundaries, %lld by owners",
                    (long long)cut_by_boundary, (long long)cut_by_tile);
    return Q4K_OK;
}

}  // namespace q4k
