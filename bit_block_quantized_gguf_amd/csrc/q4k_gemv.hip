// q4k_gemv.hip — Q4_K GEMV kernels for gfx950 (batch-1, N-vector, and the
// fused-epilogue variants used by the decode stack).
//
// The decode matmul is bandwidth-bound ("Mac Qwen3.6-27B Metal Q4_K perf
// diagnosis", §2-§4): every weight byte is read once and the job is to stream
// the bytes at HBM speed while spending as few vector instructions per weight
// as possible.  Mapping on the CDNA4 execution model:
//
//  * Work unit = 64 "lane rows" x 4 consecutive super-blocks (64 rows of one
//    matrix, or 32 rows of gate plus the same 32 rows of up for the fused
//    SwiGLU).  A workgroup of 4 waves copies the unit's 64 row segments of
//    576 bytes into LDS with 16-byte loads in address order, so each wave
//    instruction reads contiguous bytes and every row contributes one 576-byte
//    run (144-byte runs measured ~30% slower on HBM).  LDS rows are padded to
//    592 bytes, which makes the row-strided reads below conflict-free.
//  * Wave w then computes block w of the unit for all 64 lane rows, one row
//    per lane.  All lanes need the same 256 activations at the same time:
//    they arrive by scalar loads (constant address space) and enter every FMA
//    as an SGPR operand.  The wave index goes through readfirstlane so the
//    compiler can prove those addresses wave-uniform.  For one and two
//    vectors the scalar loads are software-pipelined one stage (two or one
//    quant words) ahead of the FMAs that use them.
//  * Per weight the VALU work is one FMA taking the nibble as a binary16
//    operand (v_fma_mix_f32), plus four ANDs and a shift per eight weights:
//    one AND places two nibbles (of bytes 0 and 2, or of bytes 1 and 3 after
//    the shift) straight into the two 16-bit halves of a dword.  Per block
//    the scale/min algebra is
//       y += d * sum_j sc_j * T_j  -  dmin * sum_j m_j * X_j
//    with T_j = sum(q*x) and X_j = sum(x) over sub-block j; high nibbles are
//    converted in place (16*q) and their partial sum carries the exact factor
//    1/16.  X_j comes from one 16-byte load per lane and a 3-step butterfly.
//  * The loads of unit u+1 are issued into registers before unit u is
//    computed (the activation-sum load goes first, so the in-order vmcnt wait
//    for it does not drain the prefetch), then copied to LDS between two
//    workgroup barriers.
//  * Launch: as many workgroups as fit on the device at once; each takes a
//    contiguous range of units in (row tile, K) order,
//    accumulating a row tile's blocks in registers.  A tile whose units all
//    fall in one workgroup is finished there (four waves added in LDS in wave
//    order, then the epilogue).  A tile split between workgroups is finished
//    by its last-arriving contributor, which adds the partials in workgroup
//    order (see finish_split_tile): deterministic, no second kernel, and no
//    cache-wide fence.
#include "q4k_device.hpp"
#include "q4k_internal.hpp"

#include <string.h>

#include <algorithm>
#include <atomic>
#include <map>
#include <vector>
#include <mutex>
#include <utility>

namespace q4k {

namespace {

constexpr int WK = 4;                    // waves per workgroup = blocks per unit
constexpr int SEG = WK * kBlockBytes;    // 576 bytes of a row per unit
constexpr int SEGP = SEG + 16;           // padded LDS row stride
constexpr int CH_ROW = SEG / 16;         // 36 16-byte chunks per row segment
constexpr int CH_THREAD = 9;             // 64 * 36 / 256 chunks per thread per unit

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

typedef _Float16 half2v __attribute__((ext_vector_type(2)));


// Activations of one pipeline stage of block_dot_mix: for each vector, the
// 4*SW values of the low-nibble sub-block and the 4*SW matching values of the
// high-nibble sub-block that SW quant words multiply.
template <int NV, int SW>
struct XStage {
    float l[NV][4 * SW], h[NV][4 * SW];
};

// Stage st of a block covers the SW quant words i = SW*(st mod 8/SW) ..
// +SW-1 of 32-byte group g = st / (8/SW) (word i of group g is dword i mod 4
// of the block's 16-byte chunk 1 + 2g + i/4); its activations are
// x[64g + 4i + e] (low nibbles) and x[64g + 32 + 4i + e] (high nibbles),
// e = 0..3.
template <int NV, int SW>
__device__ __forceinline__ void load_stage(XStage<NV, SW> &s, cfloat *xb, int64_t xs, int st) {
    constexpr int SPG = 8 / SW;  // stages per group
    // An offset the optimiser cannot see through (always 0) pins the loads
    // after this point: without it they are hoisted to the block start and
    // their values spilled.
    int z;
    asm volatile("s_mov_b32 %0, 0" : "=s"(z));
    const int o = 64 * (st / SPG) + 4 * SW * (st % SPG) + z;
#pragma unroll
    for (int n = 0; n < NV; ++n)
#pragma unroll
        for (int e = 0; e < 4 * SW; ++e) {
            s.l[n][e] = xb[n * xs + o + e];
            s.h[n][e] = xb[n * xs + o + 32 + e];
        }
}

// One quant word (8 weights) of a stage: four ANDs and a shift place the
// nibbles into binary16 halves (l02 / l13: the low nibbles of bytes 0, 2 and
// 1, 3; h02 / h13: the high nibbles, kept in place as 16 q); byte_fma then
// spends one v_fma_mix_f32 per weight, into two chains per sub-block (even
// and odd bytes).
struct WordQ {
    half2v l02, l13, h02, h13;
};

__device__ __forceinline__ WordQ word_unpack(uint32_t v) {
    const uint32_t v8 = v >> 8;
    WordQ q;
    q.l02 = __builtin_bit_cast(half2v, and_mask(v, 0x000F000Fu));   // q0, q2
    q.l13 = __builtin_bit_cast(half2v, and_mask(v8, 0x000F000Fu));  // q1, q3
    q.h02 = __builtin_bit_cast(half2v, and_mask(v, 0x00F000F0u));   // 16 q
    q.h13 = __builtin_bit_cast(half2v, and_mask(v8, 0x00F000F0u));
    return q;
}

// Weight factors of one 32-byte quant group g (sub-blocks 2g and 2g+1): a
// nibble c in a binary16 half is the subnormal c * 2^-24 (high nibbles sit
// in place as 16 q), so with al = d*sc*2^24, ah = d*sc*2^20 and b = -dmin*m
// one v_fma_mix_f32 fma(half, a, b) yields d*sc*q - dmin*m rounded once:
// every product is exact (d has 11 significant bits, sc 6, q 4) and the
// scaling by a power of two is exact, so the value is the dequantised weight,
// bit for bit.
struct GroupF {
    float al, bl, ah, bh;
};

__device__ __forceinline__ GroupF group_factors(const Scales &sc, int g, float d24, float d20,
                                                float ndm) {
    GroupF f;
    f.al = d24 * scale_of(sc, 2 * g);
    f.bl = ndm * min_of(sc, 2 * g);
    f.ah = d20 * scale_of(sc, 2 * g + 1);
    f.bh = ndm * min_of(sc, 2 * g + 1);
    return f;
}

// byte e of word w of the stage: the two weights it carries, each formed
// exactly (one v_fma_mix_f32), then one FMA per vector and weight
template <int NV, int SW>
__device__ __forceinline__ void byte_fma(const WordQ &q, const GroupF &f, const XStage<NV, SW> &s,
                                         int w, int e, float (&cl)[NV][2], float (&ch)[NV][2]) {
    const int c = e & 1;
    const half2v ql = c ? q.l13 : q.l02, qh = c ? q.h13 : q.h02;
    const float wl = fmaf((e & 2) ? (float)ql.y : (float)ql.x, f.al, f.bl);
    const float wh = fmaf((e & 2) ? (float)qh.y : (float)qh.x, f.ah, f.bh);
#pragma unroll
    for (int n = 0; n < NV; ++n) {
        cl[n][c] = fmaf(wl, s.l[n][4 * w + e], cl[n][c]);
        ch[n][c] = fmaf(wh, s.h[n][4 * w + e], ch[n][c]);
    }
}

// block_dot for one or two vectors: acc[n] += sum over the block of w * x_n.
// Each weight is formed exactly (group_factors) and enters one FMA per
// vector, into four chains per vector (low/high nibbles, even/odd bytes) so
// that neighbouring FMAs are independent.  Summing w*x rather than applying
// the scales to separate sums of q*x and of x keeps the rounding error a
// multiple of sum |w*x|, also on rows whose weights cancel (d*sc*q = dmin*m).
// The activations are software-pipelined through SGPRs: the scalar loads of stage st+1 are issued
// right after the first word of stage st has consumed its (already waited)
// operands, so each wait for scalar data covers loads issued one stage
// earlier.  Scalar loads complete out of order, so every wait is a full
// lgkmcnt(0); the order wait -> issue next -> compute keeps exactly one stage
// in flight.
template <int NV>
__device__ __forceinline__ void block_dot_mix(const uint4 (&b)[9], const float *xblk, int64_t xs,
                                              float (&acc)[NV]) {
    constexpr int SW = NV == 1 ? 2 : 1;  // quant words per stage
    constexpr int SPG = 8 / SW;          // stages per group
    constexpr int NST = 4 * SPG;         // stages per block
    const float d = half_lo(b[0].x);
    const float ndm = -half_hi(b[0].x);
    const float d24 = d * 16777216.0f, d20 = d * 1048576.0f;
    const Scales sc = unpack_scales(b[0].y, b[0].z, b[0].w);
    cfloat *xc = as_const(xblk);
    float cl[NV][2], ch[NV][2];
#pragma unroll
    for (int n = 0; n < NV; ++n) cl[n][0] = cl[n][1] = ch[n][0] = ch[n][1] = 0.f;
    XStage<NV, SW> xs_a, xs_b;
    load_stage<NV, SW>(xs_a, xc, xs, 0);
    GroupF f = group_factors(sc, 0, d24, d20, ndm);
    auto stage = [&](int st, const XStage<NV, SW> &cur, XStage<NV, SW> &nxt) {
        const int g = st / SPG;
        if (st % SPG == 0 && g > 0) f = group_factors(sc, g, d24, d20, ndm);
#pragma unroll
        for (int w = 0; w < SW; ++w) {
            const int i = SW * (st % SPG) + w;  // word of the group
            const WordQ q = word_unpack(word_of(b[1 + 2 * g + (i >> 2)], i & 3));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                byte_fma<NV, SW>(q, f, cur, w, e, cl, ch);
                if (w == 0 && e == 3) {
                    // The stage's first word has waited for its activations.
                    // The chains pass through an empty volatile asm, so the
                    // next stage's loads are issued only now and the rest of
                    // the stage covers their latency.  (Issuing them after the
                    // first FMA instead measured 2-3% slower.)
#pragma unroll
                    for (int n = 0; n < NV; ++n)
                        asm volatile("" : "+v"(cl[n][0]), "+v"(cl[n][1]), "+v"(ch[n][0]),
                                     "+v"(ch[n][1]));
                    if (st + 1 < NST) load_stage<NV, SW>(nxt, xc, xs, st + 1);
                }
            }
        }
    };
#pragma unroll
    for (int st = 0; st < NST; st += 2) {
        stage(st, xs_a, xs_b);
        stage(st + 1, xs_b, xs_a);
    }
#pragma unroll
    for (int n = 0; n < NV; ++n) acc[n] += (cl[n][0] + cl[n][1]) + (ch[n][0] + ch[n][1]);
}

// acc[n] += sum over the block of w * x_n.  For three or more vectors each
// weight is formed exactly once (one v_fma_mix_f32, as in block_dot_mix) and
// shared by NV FMAs; one and two vectors go to block_dot_mix.
template <int NV>
__device__ __forceinline__ void block_dot(const uint4 (&b)[9], const float *xblk, int64_t xs,
                                          float (&acc)[NV]) {
    if constexpr (NV <= 2) {
        block_dot_mix<NV>(b, xblk, xs, acc);
        return;
    }
    const float d = half_lo(b[0].x);
    const float ndm = -half_hi(b[0].x);
    const float d24 = d * 16777216.0f, d20 = d * 1048576.0f;
    const Scales sc = unpack_scales(b[0].y, b[0].z, b[0].w);
    float tl[NV], th[NV];
#pragma unroll
    for (int n = 0; n < NV; ++n) tl[n] = th[n] = 0.f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const GroupF f = group_factors(sc, g, d24, d20, ndm);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const WordQ q = word_unpack(word_of(b[1 + 2 * g + (i >> 2)], i & 3));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const half2v ql = (e & 1) ? q.l13 : q.l02, qh = (e & 1) ? q.h13 : q.h02;
                const float wl = fmaf((e & 2) ? (float)ql.y : (float)ql.x, f.al, f.bl);
                const float wh = fmaf((e & 2) ? (float)qh.y : (float)qh.x, f.ah, f.bh);
#pragma unroll
                for (int n = 0; n < NV; ++n) {
                    tl[n] = fmaf(wl, as_const(xblk + n * xs + 64 * g)[4 * i + e], tl[n]);
                    th[n] = fmaf(wh, as_const(xblk + n * xs + 64 * g + 32)[4 * i + e], th[n]);
                }
            }
        }
    }
#pragma unroll
    for (int n = 0; n < NV; ++n) acc[n] += tl[n] + th[n];
}

// Inverse RMS of an input vector from its per-32-element sums of squares.
// Up to 1024 granules (K <= 32768) every lane issues its loads before adding
// them (in the same order as the plain loop), so the latency is paid once.
__device__ __forceinline__ float inv_rms(const GemvParams &p, int lane) {
    if (p.in_sq == nullptr && p.in_len > 0) {
        // no per-32 sums of squares: add x's squares directly (lane-strided
        // float4s, then the butterfly)
        float ss = 0.f;
        for (int i = 4 * lane; i < p.in_len; i += 256) {
            const float4 v = *reinterpret_cast<const float4 *>(p.x + i);
            ss = fmaf(v.x, v.x, fmaf(v.y, v.y, fmaf(v.z, v.z, fmaf(v.w, v.w, ss))));
        }
        ss = wave_sum(ss);
        return 1.0f / sqrtf(ss / (float)p.in_len + p.eps);
    }
    if (p.in_sq == nullptr) return 1.f;  // input taken as it is (no normalisation)
    float ss = 0.f;
    if (p.in_sq_n <= 16 * 64) {
        float v[16];
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            const int i = lane + 64 * c;
            v[c] = i < p.in_sq_n ? p.in_sq[i] : 0.f;
        }
#pragma unroll
        for (int c = 0; c < 16; ++c) ss += v[c];
    } else {
        for (int i = lane; i < p.in_sq_n; i += 64) ss += p.in_sq[i];
    }
    ss = wave_sum(ss);
    return 1.0f / sqrtf(ss / (float)p.in_len + p.eps);
}

// Output store: plain, or device-coherent (sc1: written through past the
// per-XCD L2) for outputs that other workgroups of the same kernel read.
template <bool COH>
__device__ __forceinline__ void st_out(float *ptr, float v) {
    if constexpr (COH) __hip_atomic_store(ptr, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else *ptr = v;
}

// Epilogue for one wave holding the final sums of a tile's 64 lane rows.
// NMAT == 1: lane = output row (row0 + lane).  NMAT == 2: lanes 0..31 hold the
// gate rows row0 + lane, lanes 32..63 the up rows of the same indices.
template <int NV, int NMAT, int EPI, bool COH = false>
__device__ __forceinline__ void epilogue(const GemvParams &p, int row0, int lane,
                                         const float (&tot)[NV], float inv) {
    if constexpr (EPI == EPI_PLAIN) {
        const int row = row0 + lane;
        if (row < p.M) {
#pragma unroll
            for (int n = 0; n < NV; ++n) st_out<COH>(&p.y[(int64_t)n * p.y_stride + row], tot[n]);
        }
    } else {
        float val;
        int row;
        bool ok;
        if constexpr (EPI == EPI_SWIGLU) {
            const float mine = tot[0] * inv;
            const float other = __shfl(mine, (lane + 32) & 63);
            row = row0 + (lane & 31);
            ok = lane < 32 && row < p.M;
            const float g = mine, v = other;
            val = g / (1.0f + expf(-g)) * v;
            if (ok && p.y_g) {
                st_out<COH>(&p.y_g[row], g);
                st_out<COH>(&p.y_v[row], v);
            }
        } else {
            row = row0 + lane;
            ok = row < p.M;
            const int rowc = ok ? row : p.M - 1;
            if constexpr (EPI == EPI_SCALE) val = tot[0] * inv;
            else val = fmaf(tot[0], inv, p.resid[rowc]);
        }
        if (ok) st_out<COH>(&p.y[row], val);
        if (!p.out_sq) return;
        // sums of squares per 32 output rows (lanes 0..31 and 32..63)
        float sq = ok ? val * val : 0.f;
        sq += __shfl_xor(sq, 16);
        sq += __shfl_xor(sq, 8);
        sq += __shfl_xor(sq, 4);
        sq += __shfl_xor(sq, 2);
        sq += __shfl_xor(sq, 1);
        if ((lane & 31) == 0) {
            const int granule = row0 / 32 + (lane >> 5);
            if ((NMAT == 1 || lane == 0) && granule * 32 < p.M) st_out<COH>(&p.out_sq[granule], sq);
        }
    }
}

// 64-bit forms of the range arithmetic below.  They are only reached when
// (U + 1) * G does not fit in 32 bits, which at two workgroups per CU takes
// more weight bytes than the device holds, so they use a one-bit-per-step
// restoring division: a few scalar instructions of code instead of the long
// inlined sequence a 64-bit '/' expands to (which grew every kernel to
// 40 KB, most of it copies of that sequence).
__host__ __device__ __forceinline__ uint64_t udiv64_compact(uint64_t n, uint64_t d) {
    uint64_t q = 0, r = 0;
#pragma unroll 1
    for (int i = 63; i >= 0; --i) {
        r = (r << 1) | ((n >> i) & 1u);
        if (r >= d) {
            r -= d;
            q |= (uint64_t)1 << i;
        }
    }
    return q;
}
__host__ __device__ __forceinline__ int64_t range_begin64(int g, int64_t U, int G) {
    return (int64_t)udiv64_compact((uint64_t)g * (uint64_t)U, (uint64_t)G);
}
__host__ __device__ __forceinline__ int range_owner64(int64_t u, int64_t U, int G) {
    return (int)udiv64_compact((uint64_t)(u + 1) * (uint64_t)G + (uint64_t)U - 1, (uint64_t)U) - 1;
}

// Unit bookkeeping shared by the GEMV kernels.  The divisions run in 32 bits
// when the products fit.
struct Units {
    int upt;      // units per row tile = ceil(nb / 4)
    int64_t U;    // total units = tiles * upt
    int G;        // workgroups in the main grid
    bool small;   // (U + 1) * G < 2^32
    __host__ __device__ __forceinline__ int64_t begin(int g) const {
        if (small) return (int64_t)((uint32_t)g * (uint32_t)U / (uint32_t)G);
        return range_begin64(g, U, G);
    }
    // workgroup whose range contains unit u
    __host__ __device__ __forceinline__ int owner(int64_t u) const {
        if (small)
            return (int)(((uint32_t)(u + 1) * (uint32_t)G + (uint32_t)U - 1) / (uint32_t)U) - 1;
        return range_owner64(u, U, G);
    }
};

// A tile whose units are split between workgroups: each contributor stores
// its partial sums with device-coherent stores (sc1: they bypass the per-XCD
// L2 copies, so no cache write-back or invalidation is needed), waits until
// they have completed, and counts itself in on the tile's arrival counter.
// The last contributor reads the partials with device-coherent loads, adds
// them in workgroup order — the same sum whichever workgroup arrives last —
// applies the epilogue and resets the counter to zero for the next launch.
// Counters start at zero in a fresh (zero-filled) workspace.  The partials
// are loaded in chunks of 16 / NV contributors, all loads of a chunk in
// flight together.
//
// Memory ordering rests on that hardware behaviour of gfx950 (completed sc1
// stores are visible to sc1 loads from any XCD), not on release/acquire
// atomics: those add an L2 write-back before the counter update and an L2
// invalidate after it, which measured about twice the kernel time on the
// 50 MB matrices (17408x5120: 18.3 -> 35.6 us).
template <int NV, int NMAT, int EPI, bool COH = false>
__device__ __forceinline__ void finish_split_tile(const GemvParams &p, const Units &un, int g,
                                                  int t, int slot, int lane,
                                                  const float (&tot)[NV], float inv) {
    constexpr int ROWS = 64 / NMAT;
    constexpr int CH = NV >= 16 ? 1 : 16 / NV;
#pragma unroll
    for (int n = 0; n < NV; ++n)
        __hip_atomic_store(&p.ws[(((int64_t)g * 2 + slot) * NV + n) * 64 + lane], tot[n],
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the partial stores have completed
    const int gf = un.owner((int64_t)t * un.upt);
    const int gl = un.owner((int64_t)(t + 1) * un.upt - 1);
    // The counter of tile t is that of its first contributor gf: a workgroup
    // owns the first unit of at most one cut tile (any later tile starting in
    // its range would make this one whole).
    unsigned old = 0;
    if (lane == 0)
        old = __hip_atomic_fetch_add(&p.cnt[gf], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    old = __builtin_amdgcn_readfirstlane(old);
    if (old != (unsigned)(gl - gf)) return;  // not the last contributor
    if (lane == 0) __hip_atomic_store(&p.cnt[gf], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // Contributor g2 stored its partial in slot 0 when tile t is its first
    // tile.  Every contributor after gf starts inside tile t; gf does when its
    // range starts exactly at the tile's first unit.
    const int slot_gf = un.begin(gf) < (int64_t)t * un.upt ? 1 : 0;
    float sum[NV];
#pragma unroll
    for (int n = 0; n < NV; ++n) sum[n] = 0.f;
    for (int c0 = gf; c0 <= gl; c0 += CH) {
        float part[CH][NV];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int g2 = c0 + c;
            if (g2 <= gl) {
                const int sl = g2 == gf ? slot_gf : 0;
#pragma unroll
                for (int n = 0; n < NV; ++n)
                    part[c][n] = __hip_atomic_load(&p.ws[(((int64_t)g2 * 2 + sl) * NV + n) * 64 + lane],
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
#pragma unroll
        for (int c = 0; c < CH; ++c)
            if (c0 + c <= gl) {
#pragma unroll
                for (int n = 0; n < NV; ++n) sum[n] += part[c][n];
            }
    }
    epilogue<NV, NMAT, EPI, COH>(p, t * ROWS, lane, sum, inv);
}

template <int NV, int NMAT, int EPI>
__global__ __launch_bounds__(64 * WK) void gemv_kernel(const GemvParams p, const Units un) {
    __shared__ __attribute__((aligned(16))) uint8_t stage[64 * SEGP];
    __shared__ float red[WK][NV][64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    constexpr int ROWS = 64 / NMAT;  // output rows per tile
    const int g = blockIdx.x;
    const int64_t ua = un.begin(g), ub = un.begin(g + 1);
    if (ua >= ub) return;
    const int first_tile = un.small ? (int)((uint32_t)ua / (uint32_t)un.upt) : (int)(ua / un.upt);

    // this thread's copy chunks of a full unit: lane row r = q / 36, chunk c = q % 36
    int coff[CH_THREAD];  // byte offset inside the row's 576-byte segment
    int crow[CH_THREAD];  // lane row
#pragma unroll
    for (int i = 0; i < CH_THREAD; ++i) {
        const int q = i * 64 * WK + tid;
        crow[i] = q / CH_ROW;
        coff[i] = 16 * (q - crow[i] * CH_ROW);
    }
    uint4 reg[CH_THREAD];
#pragma unroll
    for (int i = 0; i < CH_THREAD; ++i) reg[i] = make_uint4(0u, 0u, 0u, 0u);
    // An interior unit (all rows of its tile below M, all WK blocks inside the
    // row) loads every chunk at an offset that does not depend on the unit:
    // computed once here, so its loads cost no vector instructions.  Only in
    // the plain-output kernels up to eight vectors: at sixteen the nine extra
    // registers spill to scratch, and the decode stack's fused-epilogue
    // variants measured 0.8% slower with them (same-process A/B).
    constexpr bool kFast = NV <= 8 && EPI == EPI_PLAIN;
    uint32_t ofull[kFast ? CH_THREAD : 1];
    if constexpr (kFast) {
#pragma unroll
        for (int i = 0; i < CH_THREAD; ++i) {
            const int r = NMAT == 2 ? (crow[i] & 31) : crow[i];
            ofull[i] = (uint32_t)r * (uint32_t)p.row_bytes + (uint32_t)coff[i];
        }
    }
    // Loads of unit u: a uniform tile base (SGPRs) plus a 32-bit lane offset;
    // rows past M are clamped to the last row (their results are not stored).
    // Unit u = t * upt + k is passed as (t, k): no 64-bit division in the loop.
    auto fetch = [&](int t, int k) {
        const int j0 = k * WK;
        const int64_t base = (int64_t)t * ROWS * p.row_bytes + (int64_t)j0 * kBlockBytes;
        const uint8_t *b0 = p.w0 + base;
        const uint8_t *b1 = NMAT == 2 ? p.w1 + base : b0;
        if constexpr (kFast) {
            if ((t + 1) * ROWS <= p.M && j0 + WK <= p.nb) {  // wave-uniform
#pragma unroll
                for (int i = 0; i < CH_THREAD; ++i) {
                    const uint8_t *src = (NMAT == 2 && crow[i] >= 32) ? b1 : b0;
                    reg[i] = ldg16(src + ofull[i]);
                }
                return;
            }
        }
        const int valid = min(WK, p.nb - j0) * kBlockBytes;  // bytes per row segment
        const int rmax = min(ROWS - 1, p.M - 1 - t * ROWS);
#pragma unroll
        for (int i = 0; i < CH_THREAD; ++i) {
            // chunks past the row's last block re-read the unit's first chunk
            // (in range; blocks past the row end are never computed), so the
            // loads need no branches
            const int cr = crow[i], co = coff[i] < valid ? coff[i] : 0;
            const int r = NMAT == 2 ? (cr & 31) : cr;
            const uint32_t off = (uint32_t)min(r, rmax) * (uint32_t)p.row_bytes + (uint32_t)co;
            const uint8_t *src = (NMAT == 2 && cr >= 32) ? b1 : b0;
            reg[i] = ldg16(src + off);
        }
    };
    auto commit = [&]() {
#pragma unroll
        for (int i = 0; i < CH_THREAD; ++i)
            *reinterpret_cast<uint4 *>(&stage[crow[i] * SEGP + coff[i]]) = reg[i];
    };

    float acc[NV];
#pragma unroll
    for (int n = 0; n < NV; ++n) acc[n] = 0.f;

    int t = first_tile, k = (int)(ua - (int64_t)first_tile * un.upt);  // unit u = t*upt + k
    fetch(t, k);
    // the epilogue's 1/rms(x), read while the first unit is in flight
    const float inv = EPI == EPI_PLAIN ? 1.f : inv_rms(p, lane);
    commit();
    __syncthreads();
    bool seg_first = k == 0;  // the current tile's range started at its first unit
    for (int64_t u = ua; u < ub; ++u) {
        const int j = k * WK + wave;  // this wave's block
        const bool active = j < p.nb;
        const bool last_of_tile = k + 1 == un.upt;
        const int tn = last_of_tile ? t + 1 : t, kn = last_of_tile ? 0 : k + 1;
        const bool more = u + 1 < ub;
        if (more) fetch(tn, kn);
        if (active) {
            const uint8_t *lp = &stage[lane * SEGP + wave * kBlockBytes];
            uint4 b[9];
#pragma unroll
            for (int i = 0; i < 9; ++i) b[i] = *reinterpret_cast<const uint4 *>(lp + 16 * i);
            block_dot<NV>(b, p.x + 256 * (int64_t)j, p.x_stride, acc);
        }
        const bool seg_end = !more || last_of_tile;
        if (seg_end) {
#pragma unroll
            for (int n = 0; n < NV; ++n) {
                red[wave][n][lane] = acc[n];
                acc[n] = 0.f;
            }
        }
        __syncthreads();
        if (seg_end && wave == 0) {
            float tot[NV];
#pragma unroll
            for (int n = 0; n < NV; ++n) {
                float s = red[0][n][lane];
#pragma unroll
                for (int w = 1; w < WK; ++w) s += red[w][n][lane];
                tot[n] = s;
            }
            const bool whole = seg_first && last_of_tile;
            if (whole)
                epilogue<NV, NMAT, EPI>(p, t * ROWS, lane, tot, inv);
            else
                finish_split_tile<NV, NMAT, EPI>(p, un, g, t, t == first_tile ? 0 : 1, lane, tot,
                                                 inv);
        }
        if (seg_end) seg_first = true;
        t = tn;
        k = kn;
        if (more) commit();
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Batched GEMV on the matrix cores (four or eight vectors; sixteen compile
// too but run on gemv_split_kernel below).  Same
// units, ranges, LDS staging and cut-tile finishing as gemv_kernel: lane l
// reads row l of the wave's block from LDS and forms each of its 256 weights
// exactly (one v_fma_mix_f32: d*sc*q - dmin*m).  The products go to
// v_mfma_f32_4x4x1_16b_f32, sixteen independent 4x4 outer products per
// instruction: product block b = l / 4 takes the weights of rows 4b .. 4b+3
// (lane 4b + i supplies row i) and the activations of four vectors at the
// same column (lane 4b + j supplies vector j), so one instruction applies one
// column of the 64 rows to four vectors and accumulates W[row][k] * X[vec][k]
// in f32 (an exact weight times an f32 activation).  Lane 4b + j ends with
// rows 4b + i (register i) of vector j: no cross-lane reduction is needed.
// The unit's activations (NV vectors x 1024 columns) are staged in LDS next
// to its weights, loaded and committed with them; a lane reads them as
// float4 runs of four columns (four distinct addresses per instruction).
// Four accumulator chains per 4-vector group (low/high nibbles, even/odd
// byte) keep consecutive MFMAs independent.
typedef float f4v __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// (lo, hi) -> two bf16 (RNE) in one dword, lo in the low half: v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
// the f32 values of the two bf16 halves of a dword (exact)
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// Eight f32 values -> high parts w1 = bf16(w) and low parts bf16(w - w1)
// (RNE both; w - w1 is exact in f32).
__device__ __forceinline__ void split8(const float (&w)[8], bf16x8 &hi, bf16x8 &lo) {
    uint4 h, l;
    h.x = pack_bf16(w[0], w[1]);
    h.y = pack_bf16(w[2], w[3]);
    h.z = pack_bf16(w[4], w[5]);
    h.w = pack_bf16(w[6], w[7]);
    l.x = pack_bf16(w[0] - bf16_lo(h.x), w[1] - bf16_hi(h.x));
    l.y = pack_bf16(w[2] - bf16_lo(h.y), w[3] - bf16_hi(h.y));
    l.z = pack_bf16(w[4] - bf16_lo(h.z), w[5] - bf16_hi(h.z));
    l.w = pack_bf16(w[6] - bf16_lo(h.w), w[7] - bf16_hi(h.w));
    hi = __builtin_bit_cast(bf16x8, h);
    lo = __builtin_bit_cast(bf16x8, l);
}

template <int NV>
__global__ __launch_bounds__(64 * WK) void gemv_mfma_kernel(const GemvParams p, const Units un) {
    static_assert(NV == 4 || NV == 8 || NV == 16, "four, eight or sixteen vectors");
    constexpr int VG = NV / 4;  // 4-vector groups
    constexpr int XQ = NV;      // float4s of activations per thread per unit
    __shared__ __attribute__((aligned(16))) uint8_t stage[64 * SEGP];
    __shared__ __attribute__((aligned(16))) float xs[NV][256 * WK];
    __shared__ float red[WK][NV][64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = blockIdx.x;
    const int64_t ua = un.begin(g), ub = un.begin(g + 1);
    if (ua >= ub) return;
    const int first_tile = un.small ? (int)((uint32_t)ua / (uint32_t)un.upt) : (int)(ua / un.upt);

    int coff[CH_THREAD], crow[CH_THREAD];
#pragma unroll
    for (int i = 0; i < CH_THREAD; ++i) {
        const int q = i * 64 * WK + tid;
        crow[i] = q / CH_ROW;
        coff[i] = 16 * (q - crow[i] * CH_ROW);
    }
    uint4 reg[CH_THREAD];
#pragma unroll
    for (int i = 0; i < CH_THREAD; ++i) reg[i] = make_uint4(0u, 0u, 0u, 0u);
    float4 xreg[XQ];
    auto fetch = [&](int t, int k) {
        const int j0 = k * WK;
        const uint8_t *b0 = p.w0 + (int64_t)t * 64 * p.row_bytes + (int64_t)j0 * kBlockBytes;
        const int valid = min(WK, p.nb - j0) * kBlockBytes;
        const int rmax = min(63, p.M - 1 - t * 64);
#pragma unroll
        for (int i = 0; i < CH_THREAD; ++i) {
            const int co = coff[i] < valid ? coff[i] : 0;
            reg[i] = ldg16(b0 + (uint32_t)min(crow[i], rmax) * (uint32_t)p.row_bytes + (uint32_t)co);
        }
        // activations of the unit's columns: float4 q = tid + 256 m is vector
        // q / 256, columns 4 (q % 256) .. +3 of the unit (zero past K)
#pragma unroll
        for (int m = 0; m < XQ; ++m) {
            const int q = tid + 256 * m;
            const int col = 256 * j0 + 4 * (q & 255);
            xreg[m] = col < p.K ? *reinterpret_cast<const float4 *>(
                                      p.x + (int64_t)(q >> 8) * p.x_stride + col)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    auto commit = [&]() {
#pragma unroll
        for (int i = 0; i < CH_THREAD; ++i)
            *reinterpret_cast<uint4 *>(&stage[crow[i] * SEGP + coff[i]]) = reg[i];
#pragma unroll
        for (int m = 0; m < XQ; ++m) {
            const int q = tid + 256 * m;
            *reinterpret_cast<float4 *>(&xs[q >> 8][4 * (q & 255)]) = xreg[m];
        }
    };

    // acc[v][c]: vector group v, chain c (bit 0: high nibbles, bit 1: odd byte)
    f4v acc[VG][4];
#pragma unroll
    for (int v = 0; v < VG; ++v)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[v][c] = f4v{0.f, 0.f, 0.f, 0.f};

    int t = first_tile, k = (int)(ua - (int64_t)first_tile * un.upt);
    fetch(t, k);
    commit();
    __syncthreads();
    bool seg_first = k == 0;
    for (int64_t u = ua; u < ub; ++u) {
        const int j = k * WK + wave;
        const bool last_of_tile = k + 1 == un.upt;
        const int tn = last_of_tile ? t + 1 : t, kn = last_of_tile ? 0 : k + 1;
        const bool more = u + 1 < ub;
        if (more) fetch(tn, kn);
        if (j < p.nb) {
            const uint8_t *lp = &stage[lane * SEGP + wave * kBlockBytes];
            uint4 b[9];
#pragma unroll
            for (int i = 0; i < 9; ++i) b[i] = *reinterpret_cast<const uint4 *>(lp + 16 * i);
            const float d = half_lo(b[0].x), ndm = -half_hi(b[0].x);
            const float d24 = d * 16777216.0f, d20 = d * 1048576.0f;
            const Scales sc = unpack_scales(b[0].y, b[0].z, b[0].w);
            const float *xr[VG];
#pragma unroll
            for (int v = 0; v < VG; ++v) xr[v] = &xs[4 * v + (lane & 3)][256 * wave];
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const GroupF f = group_factors(sc, gq, d24, d20, ndm);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const WordQ q = word_unpack(word_of(b[1 + 2 * gq + (i >> 2)], i & 3));
                    float4 xl[VG], xh[VG];
#pragma unroll
                    for (int v = 0; v < VG; ++v) {
                        xl[v] = *reinterpret_cast<const float4 *>(xr[v] + 64 * gq + 4 * i);
                        xh[v] = *reinterpret_cast<const float4 *>(xr[v] + 64 * gq + 32 + 4 * i);
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const half2v ql = (e & 1) ? q.l13 : q.l02, qh = (e & 1) ? q.h13 : q.h02;
                        const float wl = fmaf((e & 2) ? (float)ql.y : (float)ql.x, f.al, f.bl);
                        const float wh = fmaf((e & 2) ? (float)qh.y : (float)qh.x, f.ah, f.bh);
#pragma unroll
                        for (int v = 0; v < VG; ++v) {
                            const float xle = e == 0 ? xl[v].x : e == 1 ? xl[v].y : e == 2 ? xl[v].z : xl[v].w;
                            const float xhe = e == 0 ? xh[v].x : e == 1 ? xh[v].y : e == 2 ? xh[v].z : xh[v].w;
                            acc[v][2 * (e & 1)] = __builtin_amdgcn_mfma_f32_4x4x1f32(
                                wl, xle, acc[v][2 * (e & 1)], 0, 0, 0);
                            acc[v][2 * (e & 1) + 1] = __builtin_amdgcn_mfma_f32_4x4x1f32(
                                wh, xhe, acc[v][2 * (e & 1) + 1], 0, 0, 0);
                        }
                    }
                }
            }
        }
        const bool seg_end = !more || last_of_tile;
        if (seg_end) {
            // lane 4b + j holds rows 4b + i (register i) of vector 4v + j
#pragma unroll
            for (int v = 0; v < VG; ++v) {
                const f4v s = (acc[v][0] + acc[v][1]) + (acc[v][2] + acc[v][3]);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    red[wave][4 * v + (lane & 3)][(lane & ~3) + i] = s[i];
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[v][c] = f4v{0.f, 0.f, 0.f, 0.f};
            }
        }
        __syncthreads();
        if (seg_end && wave == 0) {
            float tot[NV];
#pragma unroll
            for (int n = 0; n < NV; ++n) {
                float s = red[0][n][lane];
#pragma unroll
                for (int w = 1; w < WK; ++w) s += red[w][n][lane];
                tot[n] = s;
            }
            if (seg_first && last_of_tile)
                epilogue<NV, 1, EPI_PLAIN>(p, t * 64, lane, tot, 1.f);
            else
                finish_split_tile<NV, 1, EPI_PLAIN>(p, un, g, t, t == first_tile ? 0 : 1, lane, tot,
                                                    1.f);
        }
        if (seg_end) seg_first = true;
        t = tn;
        k = kn;
        if (more) commit();
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Batched GEMV for sixteen vectors (eight also compile) on
// v_mfma_f32_16x16x32_bf16, with each exact f32 weight and activation split into two bf16 parts:
// w = w1 + w2 + e_w and x = x1 + x2 + e_x (w1 = bf16(w), w2 = bf16(w - w1),
// both RNE; w - w1 is exact in f32), so |e_w| <= 2^-18 |w| and likewise for
// x.  Three products w1 x1 + w1 x2 + w2 x1 leave out w2 x2 and the e terms,
// at most about 3 * 2^-18 |w x| per product: well inside an f32 bound of
// 1e-4 sum |w x|.  A weight that is exactly zero (a row whose scale and min
// cancel) stays exactly zero in both parts.  One instruction takes 16 rows x
// 32 columns of W against 32 columns x 16 vectors, so the three of them
// replace eight 16x16x4 f32 instructions.
// Same units, staging, ranges and cut-tile finishing as gemv_mfma_kernel.
// Lane l = 16 kk + r supplies row r of a 16-row group (A) and vector r (B,
// vector r mod NV when NV < 16: those output columns are never read) for
// columns 8 kk .. 8 kk + 7 of a 32-column sub-block: its 8 quant bytes
// 8 kk .. 8 kk + 7 of the 32-byte group hold the low-nibble weights of
// sub-block 2 gq and the high-nibble ones of sub-block 2 gq + 1 at exactly
// those columns.  The activations are split once per unit when they are
// staged, into two bf16 copies whose vector rows are padded by 16 bytes (the
// sixteen vectors of one fragment read then start on different banks).
// Lane 16 kk + j ends with rows 4 kk + r (register r) of each group for
// vector j (the 16x16 output layout); two accumulator chains per group (low
// and high nibbles), and consecutive instructions use different ones.
template <int NV>
__global__ __launch_bounds__(64 * WK) void gemv_split_kernel(const GemvParams p, const Units un) {
    static_assert(NV == 8 || NV == 16, "eight or sixteen vectors");
    constexpr int XQ = NV;              // float4s of activations per thread per unit
    constexpr int XR = 256 * WK + 8;    // bf16 per staged vector row (16-byte pad)
    __shared__ __attribute__((aligned(16))) uint8_t stage[64 * SEGP];
    __shared__ __attribute__((aligned(16))) __bf16 x1s[NV][XR];
    __shared__ __attribute__((aligned(16))) __bf16 x2s[NV][XR];
    __shared__ float red[WK][NV][64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = blockIdx.x;
    const int64_t ua = un.begin(g), ub = un.begin(g + 1);
    if (ua >= ub) return;
    const int first_tile = un.small ? (int)((uint32_t)ua / (uint32_t)un.upt) : (int)(ua / un.upt);

    int coff[CH_THREAD], crow[CH_THREAD];
#pragma unroll
    for (int i = 0; i < CH_THREAD; ++i) {
        const int q = i * 64 * WK + tid;
        crow[i] = q / CH_ROW;
        coff[i] = 16 * (q - crow[i] * CH_ROW);
    }
    uint4 reg[CH_THREAD];
#pragma unroll
    for (int i = 0; i < CH_THREAD; ++i) reg[i] = make_uint4(0u, 0u, 0u, 0u);
    float4 xreg[XQ];
    auto fetch = [&](int t, int k) {
        const int j0 = k * WK;
        const uint8_t *b0 = p.w0 + (int64_t)t * 64 * p.row_bytes + (int64_t)j0 * kBlockBytes;
        const int valid = min(WK, p.nb - j0) * kBlockBytes;
        const int rmax = min(63, p.M - 1 - t * 64);
#pragma unroll
        for (int i = 0; i < CH_THREAD; ++i) {
            const int co = coff[i] < valid ? coff[i] : 0;
            reg[i] = ldg16(b0 + (uint32_t)min(crow[i], rmax) * (uint32_t)p.row_bytes + (uint32_t)co);
        }
        // float4 q = tid + 256 m is vector q / 256, columns 4 (q % 256) .. +3
        // of the unit (zero past K)
#pragma unroll
        for (int m = 0; m < XQ; ++m) {
            const int q = tid + 256 * m;
            const int col = 256 * j0 + 4 * (q & 255);
            xreg[m] = col < p.K ? *reinterpret_cast<const float4 *>(
                                      p.x + (int64_t)(q >> 8) * p.x_stride + col)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    auto commit = [&]() {
#pragma unroll
        for (int i = 0; i < CH_THREAD; ++i)
            *reinterpret_cast<uint4 *>(&stage[crow[i] * SEGP + coff[i]]) = reg[i];
#pragma unroll
        for (int m = 0; m < XQ; ++m) {
            const int q = tid + 256 * m;
            const float4 v = xreg[m];
            const uint32_t h01 = pack_bf16(v.x, v.y), h23 = pack_bf16(v.z, v.w);
            const uint32_t l01 = pack_bf16(v.x - bf16_lo(h01), v.y - bf16_hi(h01));
            const uint32_t l23 = pack_bf16(v.z - bf16_lo(h23), v.w - bf16_hi(h23));
            *reinterpret_cast<uint2 *>(&x1s[q >> 8][4 * (q & 255)]) = make_uint2(h01, h23);
            *reinterpret_cast<uint2 *>(&x2s[q >> 8][4 * (q & 255)]) = make_uint2(l01, l23);
        }
    };

    const int r16 = lane & 15, kk = lane >> 4;
    f4v acc[4][2];  // row group, low / high nibbles
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) acc[rg][0] = acc[rg][1] = f4v{0.f, 0.f, 0.f, 0.f};

    int t = first_tile, k = (int)(ua - (int64_t)first_tile * un.upt);
    fetch(t, k);
    commit();
    __syncthreads();
    bool seg_first = k == 0;
    for (int64_t u = ua; u < ub; ++u) {
        const int j = k * WK + wave;
        const bool last_of_tile = k + 1 == un.upt;
        const int tn = last_of_tile ? t + 1 : t, kn = last_of_tile ? 0 : k + 1;
        const bool more = u + 1 < ub;
        if (more) fetch(tn, kn);
        if (j < p.nb) {
            // the scale and min of this lane's row in each row group
            const uint8_t *blk = &stage[r16 * SEGP + wave * kBlockBytes];
            Scales sc[4];
            float d24[4], d20[4], ndm[4];
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const uint4 h = *reinterpret_cast<const uint4 *>(blk + 16 * rg * SEGP);
                const float d = half_lo(h.x);
                ndm[rg] = -half_hi(h.x);
                d24[rg] = d * 16777216.0f;
                d20[rg] = d * 1048576.0f;
                sc[rg] = unpack_scales(h.y, h.z, h.w);
            }
            const int xo = 256 * wave + 8 * kk;
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                bf16x8 b1[2], b2[2];  // [low / high nibble sub-block]
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    b1[hf] = *reinterpret_cast<const bf16x8 *>(&x1s[r16 % NV][xo + 64 * gq + 32 * hf]);
                    b2[hf] = *reinterpret_cast<const bf16x8 *>(&x2s[r16 % NV][xo + 64 * gq + 32 * hf]);
                }
                bf16x8 a1[4][2], a2[4][2];  // [row group][low / high]
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) {
                    const GroupF f = group_factors(sc[rg], gq, d24[rg], d20[rg], ndm[rg]);
                    const uint2 qd =
                        *reinterpret_cast<const uint2 *>(blk + 16 * rg * SEGP + 16 + 32 * gq + 8 * kk);
                    const WordQ q0 = word_unpack(qd.x), q1 = word_unpack(qd.y);
                    float wl[8], wh[8];  // columns 8 kk + e, e = 4 i + byte
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        const WordQ &q = i ? q1 : q0;
                        wl[4 * i + 0] = fmaf((float)q.l02.x, f.al, f.bl);
                        wl[4 * i + 1] = fmaf((float)q.l13.x, f.al, f.bl);
                        wl[4 * i + 2] = fmaf((float)q.l02.y, f.al, f.bl);
                        wl[4 * i + 3] = fmaf((float)q.l13.y, f.al, f.bl);
                        wh[4 * i + 0] = fmaf((float)q.h02.x, f.ah, f.bh);
                        wh[4 * i + 1] = fmaf((float)q.h13.x, f.ah, f.bh);
                        wh[4 * i + 2] = fmaf((float)q.h02.y, f.ah, f.bh);
                        wh[4 * i + 3] = fmaf((float)q.h13.y, f.ah, f.bh);
                    }
                    split8(wl, a1[rg][0], a2[rg][0]);
                    split8(wh, a1[rg][1], a2[rg][1]);
                }
                // three products per fragment; consecutive instructions go to
                // different accumulators
#pragma unroll
                for (int term = 0; term < 3; ++term)
#pragma unroll
                    for (int rg = 0; rg < 4; ++rg)
#pragma unroll
                        for (int hf = 0; hf < 2; ++hf) {
                            const bf16x8 &A = term == 2 ? a2[rg][hf] : a1[rg][hf];
                            const bf16x8 &B = term == 1 ? b2[hf] : b1[hf];
                            acc[rg][hf] =
                                __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, acc[rg][hf], 0, 0, 0);
                        }
            }
        }
        const bool seg_end = !more || last_of_tile;
        if (seg_end) {
            // lane 16 kk + j holds rows 16 rg + 4 kk + r (register r) of vector j
            if (r16 < NV) {
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) {
                    const f4v s = acc[rg][0] + acc[rg][1];
#pragma unroll
                    for (int r = 0; r < 4; ++r) red[wave][r16][16 * rg + 4 * kk + r] = s[r];
                }
            }
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) acc[rg][0] = acc[rg][1] = f4v{0.f, 0.f, 0.f, 0.f};
        }
        __syncthreads();
        if (seg_end && wave == 0) {
            float tot[NV];
#pragma unroll
            for (int n = 0; n < NV; ++n) {
                float s = red[0][n][lane];
#pragma unroll
                for (int w = 1; w < WK; ++w) s += red[w][n][lane];
                tot[n] = s;
            }
            if (seg_first && last_of_tile)
                epilogue<NV, 1, EPI_PLAIN>(p, t * 64, lane, tot, 1.f);
            else
                finish_split_tile<NV, 1, EPI_PLAIN>(p, un, g, t, t == first_tile ? 0 : 1, lane, tot,
                                                    1.f);
        }
        if (seg_end) seg_first = true;
        t = tn;
        k = kn;
        if (more) commit();
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Persistent decode kernel: the whole per-token chain of GEMV nodes in one
// launch ("Mac Qwen3.6-27B Metal Q4_K perf diagnosis", §4: one submission per
// token with the activation resident).  Every workgroup walks the node list;
// within a node it takes its unit range exactly as gemv_kernel does (same
// unit loop, same in-kernel finishing of cut tiles).  Between nodes:
//   * the workgroup loads its first unit of the next node into LDS and issues
//     the loads of its second unit, then waits until every workgroup has
//     finished the current node (16 counters per node, workgroup g counting
//     into counter g mod 16 so arrivals do not queue on one address; weights do not depend on
//     activations, so the memory pipe keeps streaming across the boundary);
//   * outputs are written with device-coherent (sc1) stores and each
//     workgroup counts itself in only after its stores have completed, so
//     the next node's workgroups, on any XCD, read them after the wait.
//     Every activation buffer is written once per token before any workgroup
//     reads it, and caches are invalidated at each kernel start, so no stale
//     copy can be read.
// The counters grow by the grid size every token (epoch): token e waits for
// (e + 1) * G arrivals, compared as a signed difference.  Each wait is
// bounded: past spin_limit polls the workgroup records an error flag and
// goes on, so every workgroup always reaches the end of the kernel.  The
// grid must be co-resident (cooperative launch).
struct StackNode {
    GemvParams p;
    Units un;
    int32_t nmat, epi;
};

// The node parameters are read from memory, so the compiler cannot tell that
// their pointers address global memory and would access through them with
// flat instructions, which also count against the LDS wait counter (a wait
// for the staged weights would then wait for the next unit's loads too).
// A round trip through the global address space lets it use global ones.
template <class T>
__device__ __forceinline__ T *as_global(T *p) {
    return (T *)(__attribute__((address_space(1))) T *)(uintptr_t)p;
}

// Wave 0 waits until every workgroup has counted itself in on the node's
// kStackSyncLanes counters (lane l reads counter l, which workgroups
// g = l mod kStackSyncLanes increment once per token); bounded by spin_limit
// polls, after which the error word is set and the wait gives up.
__device__ __forceinline__ void wait_arrivals(unsigned *c, unsigned epoch, int G, int lane,
                                              int spin_limit, unsigned *err) {
    constexpr int NS = kStackSyncLanes;
    const bool mine = lane < NS;
    const unsigned target = mine ? (epoch + 1u) * (unsigned)((G - lane + NS - 1) / NS) : 0u;
    int i = 0;
    while (true) {
        bool ok = true;
        if (mine)
            ok = (int)(__hip_atomic_load(c + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) -
                       target) >= 0;
        if (__all(ok)) return;
        if (++i > spin_limit) {
            if (lane == 0) __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
        __builtin_amdgcn_s_sleep(1);
    }
}

template <int NMAT, int EPI>
__device__ __forceinline__ void node_finish(const GemvParams &p, const Units &un, int g, int t,
                                            int first_tile, bool whole, int lane,
                                            const float (&tot)[1], float inv) {
    constexpr int ROWS = 64 / NMAT;
    if (whole)
        epilogue<1, NMAT, EPI, true>(p, t * ROWS, lane, tot, inv);
    else
        finish_split_tile<1, NMAT, EPI, true>(p, un, g, t, t == first_tile ? 0 : 1, lane, tot, inv);
}

__global__ __launch_bounds__(64 * WK) void stack_kernel(const StackNode *__restrict__ nodes,
                                                        int n_nodes, unsigned *done,
                                                        unsigned epoch, unsigned *err,
                                                        int spin_limit) {
    __shared__ __attribute__((aligned(16))) uint8_t stage[64 * SEGP];
    __shared__ float red[WK][1][64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = blockIdx.x;
    const unsigned G = gridDim.x;
    int coff[CH_THREAD], crow[CH_THREAD];
#pragma unroll
    for (int i = 0; i < CH_THREAD; ++i) {
        const int q = i * 64 * WK + tid;
        crow[i] = q / CH_ROW;
        coff[i] = 16 * (q - crow[i] * CH_ROW);
    }
    uint4 reg[CH_THREAD];
#pragma unroll
    for (int i = 0; i < CH_THREAD; ++i) reg[i] = make_uint4(0u, 0u, 0u, 0u);

    for (int n = 0; n < n_nodes; ++n) {
        GemvParams p = nodes[n].p;
        p.w0 = as_global(p.w0);
        p.w1 = as_global(p.w1);
        p.x = as_global(p.x);
        p.y = as_global(p.y);
        p.y_g = as_global(p.y_g);
        p.y_v = as_global(p.y_v);
        p.ws = as_global(p.ws);
        p.cnt = as_global(p.cnt);
        p.in_sq = as_global(p.in_sq);
        p.resid = as_global(p.resid);
        p.out_sq = as_global(p.out_sq);
        const Units un = nodes[n].un;
        const int nmat = nodes[n].nmat, epi = nodes[n].epi;
        const int rows = 64 / nmat;
        // a node with fewer units than workgroups runs on its first U
        // workgroups (un.G = min(G, U)), one unit or more each: every
        // workgroup between a cut tile's first and last contributor then
        // contributes to it
        const bool have = g < un.G;
        const int64_t ua = have ? un.begin(g) : 0, ub = have ? un.begin(g + 1) : 0;
        const int first_tile =
            !have ? 0 : un.small ? (int)((uint32_t)ua / (uint32_t)un.upt) : (int)(ua / un.upt);
        auto fetch = [&](int t, int k) {
            const int j0 = k * WK;
            const int64_t base = (int64_t)t * rows * p.row_bytes + (int64_t)j0 * kBlockBytes;
            const uint8_t *b0 = p.w0 + base;
            const uint8_t *b1 = nmat == 2 ? p.w1 + base : b0;
            const int valid = min(WK, p.nb - j0) * kBlockBytes;
            const int rmax = min(rows - 1, p.M - 1 - t * rows);
#pragma unroll
            for (int i = 0; i < CH_THREAD; ++i) {
                const int cr = crow[i], co = coff[i] < valid ? coff[i] : 0;
                const int r = nmat == 2 ? (cr & 31) : cr;
                const uint32_t off = (uint32_t)min(r, rmax) * (uint32_t)p.row_bytes + (uint32_t)co;
                const uint8_t *src = (nmat == 2 && cr >= 32) ? b1 : b0;
                reg[i] = ldg16(src + off);
            }
        };
        auto commit = [&]() {
#pragma unroll
            for (int i = 0; i < CH_THREAD; ++i)
                *reinterpret_cast<uint4 *>(&stage[crow[i] * SEGP + coff[i]]) = reg[i];
        };
        int t = first_tile, k = have ? (int)(ua - (int64_t)first_tile * un.upt) : 0;
        // this node's first unit into LDS and its second in flight, then the
        // wait for the previous node (the LDS is free: the previous node's
        // loop ended with a barrier)
        if (have) {
            fetch(t, k);
            commit();
            if (ua + 1 < ub) {
                const bool lt = k + 1 == un.upt;
                fetch(lt ? t + 1 : t, lt ? 0 : k + 1);
            }
        }
        if (n > 0 && wave == 0)
            wait_arrivals(&done[(n - 1) * kStackSyncLanes], epoch, (int)G, lane, spin_limit, err);
        __syncthreads();
        if (have) {
            const float inv = epi == EPI_PLAIN ? 1.f : inv_rms(p, lane);
            float acc[1] = {0.f};
            bool seg_first = k == 0;
            for (int64_t u = ua; u < ub; ++u) {
                const int j = k * WK + wave;
                const bool active = j < p.nb;
                const bool last_of_tile = k + 1 == un.upt;
                const int tn = last_of_tile ? t + 1 : t, kn = last_of_tile ? 0 : k + 1;
                const bool more = u + 1 < ub;
                if (more && u > ua) fetch(tn, kn);  // unit ua + 1 was fetched before the wait
                if (active) {
                    const uint8_t *lp = &stage[lane * SEGP + wave * kBlockBytes];
                    uint4 b[9];
#pragma unroll
                    for (int i = 0; i < 9; ++i) b[i] = *reinterpret_cast<const uint4 *>(lp + 16 * i);
                    block_dot<1>(b, p.x + 256 * (int64_t)j, p.x_stride, acc);
                }
                const bool seg_end = !more || last_of_tile;
                if (seg_end) {
                    red[wave][0][lane] = acc[0];
                    acc[0] = 0.f;
                }
                __syncthreads();
                if (seg_end && wave == 0) {
                    float tot[1] = {red[0][0][lane]};
#pragma unroll
                    for (int w = 1; w < WK; ++w) tot[0] += red[w][0][lane];
                    const bool whole = seg_first && last_of_tile;
                    if (epi == EPI_SWIGLU)
                        node_finish<2, EPI_SWIGLU>(p, un, g, t, first_tile, whole, lane, tot, inv);
                    else if (epi == EPI_RESID)
                        node_finish<1, EPI_RESID>(p, un, g, t, first_tile, whole, lane, tot, inv);
                    else if (epi == EPI_SCALE)
                        node_finish<1, EPI_SCALE>(p, un, g, t, first_tile, whole, lane, tot, inv);
                    else
                        node_finish<1, EPI_PLAIN>(p, un, g, t, first_tile, whole, lane, tot, inv);
                }
                if (seg_end) seg_first = true;
                t = tn;
                k = kn;
                if (more) commit();
                __syncthreads();
            }
        }
        // count this workgroup in once its stores have completed (only wave 0
        // stores node outputs)
        if (wave == 0) {
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
            if (lane == 0)
                __hip_atomic_fetch_add(&done[n * kStackSyncLanes + (g % kStackSyncLanes)], 1u,
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

__global__ __launch_bounds__(64) void sumsq_kernel(const float *__restrict__ v, int64_t n,
                                                   float *__restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * 64 + threadIdx.x;
    const float a = i < n ? v[i] : 0.f;
    float s = a * a;
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 8);
    s += __shfl_xor(s, 4);
    s += __shfl_xor(s, 2);
    s += __shfl_xor(s, 1);
    const int64_t granule = (int64_t)blockIdx.x * 2 + (threadIdx.x >> 5);
    if ((threadIdx.x & 31) == 0 && granule * 32 < n) out[granule] = s;
}

// ---------------------------------------------------------------------------
// Q8_0 GEMV (one vector).  Q8_0 stores 32 weights in 34 bytes: a binary16
// scale d, then 32 two's-complement int8 quants; w = d * q (public GGUF
// convention; the pages run the lm_head matmul in Q8, "Mac Qwen3.6-27B Metal
// Q4_K perf diagnosis", §2 decode profile).  Same skeleton as the Q4_K
// kernel: a unit is 64 rows x 16 blocks (one 544-byte run per row), copied to
// LDS in address order (rows padded to 560 bytes) with the next unit's loads
// in flight; wave w then takes blocks 4w .. 4w+3 of every row, one row per
// lane.  Per dword of quants, an XOR with 0x80 per byte makes u = q + 128
// (0..255), and one AND (of the dword, or of it shifted by 8) places two
// bytes into the 16-bit halves, where binary16 reads u as the subnormal
// u * 2^-24: one v_fma_mix_f32 per weight.  Per block, sum(q x) =
// 2^24 * sum(u x) - 128 * sum(x); the block sums of x come from one 16-byte
// load per lane and a 3-step butterfly.
constexpr int Q8_BB = 34;                      // bytes per block
constexpr int Q8_UNIT_BLOCKS = 16;             // blocks per row per unit
constexpr int Q8_SEG = Q8_UNIT_BLOCKS * Q8_BB;  // 544-byte row run
constexpr int Q8_SEGP = Q8_SEG + 16;           // LDS row stride
constexpr int Q8_CH_ROW = Q8_SEG / 16;         // 34 chunks per row
constexpr int Q8_CH_UNIT = 64 * Q8_CH_ROW;     // 2176 chunks per unit
constexpr int Q8_CH_THREAD = (Q8_CH_UNIT + 64 * WK - 1) / (64 * WK);  // 9 (the last for half the threads)
static_assert(Q8_SEG % 16 == 0 && Q8_SEGP % 16 == 0, "16-byte chunks");

// sum over a block's 32 quants of q * x; q8 holds the 8 quant dwords, x the
// block's 32 activations.  Two bytes at a time go into the 16-bit halves of
// a dword as 0x6400 | (q + 128), the binary16 value 1024 + (q + 128), and one
// v_pk_add_f16 of -1152 leaves q itself, exactly (small integers are exact in
// binary16); each weight then costs one v_fma_mix_f32.
__device__ __forceinline__ float q8_block_dot(const uint32_t (&q8)[8], cfloat *x) {
    const half2v bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    float c0 = 0.f, c1 = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t u = q8[i] ^ 0x80808080u;  // q + 128 per byte
        const half2v q02 = __builtin_bit_cast(half2v, and_or(u, 0x00FF00FFu, 0x64006400u)) + bias;
        const half2v q13 =
            __builtin_bit_cast(half2v, and_or(u >> 8, 0x00FF00FFu, 0x64006400u)) + bias;
        c0 = fmaf((float)q02.x, x[4 * i + 0], c0);
        c1 = fmaf((float)q13.x, x[4 * i + 1], c1);
        c0 = fmaf((float)q02.y, x[4 * i + 2], c0);
        c1 = fmaf((float)q13.y, x[4 * i + 3], c1);
    }
    return c0 + c1;
}

__global__ __launch_bounds__(64 * WK) void gemv_q8_kernel(const GemvParams p, const Units un) {
    __shared__ __attribute__((aligned(16))) uint8_t stage[64 * Q8_SEGP];
    __shared__ float red[WK][1][64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = blockIdx.x;
    const int64_t ua = un.begin(g), ub = un.begin(g + 1);
    if (ua >= ub) return;
    const int first_tile = un.small ? (int)((uint32_t)ua / (uint32_t)un.upt) : (int)(ua / un.upt);

    int crow[Q8_CH_THREAD], coff[Q8_CH_THREAD];
#pragma unroll
    for (int i = 0; i < Q8_CH_THREAD; ++i) {
        const int q = i * 64 * WK + tid;  // past Q8_CH_UNIT only in the last slot (waves 2, 3)
        crow[i] = q / Q8_CH_ROW;
        coff[i] = 16 * (q - crow[i] * Q8_CH_ROW);
    }
    uint4 reg[Q8_CH_THREAD];
#pragma unroll
    for (int i = 0; i < Q8_CH_THREAD; ++i) reg[i] = make_uint4(0u, 0u, 0u, 0u);
    auto fetch = [&](int t, int k) {
        const int j0 = k * Q8_UNIT_BLOCKS;
        const int valid = min(Q8_UNIT_BLOCKS, p.nb - j0) * Q8_BB;  // bytes of this row run
        const int rmax = min(63, p.M - 1 - t * 64);
        const uint8_t *b0 = p.w0 + (int64_t)t * 64 * p.row_bytes + (int64_t)j0 * Q8_BB;
#pragma unroll
        for (int i = 0; i < Q8_CH_THREAD; ++i) {
            if (i * 64 * WK + 64 * wave >= Q8_CH_UNIT) continue;  // wave-uniform
            const int co = coff[i] < valid ? coff[i] : 0;
            const uint32_t off = (uint32_t)min(crow[i], rmax) * (uint32_t)p.row_bytes + (uint32_t)co;
            reg[i] = ldg16(b0 + off);
        }
    };
    auto commit = [&]() {
#pragma unroll
        for (int i = 0; i < Q8_CH_THREAD; ++i) {
            if (i * 64 * WK + 64 * wave >= Q8_CH_UNIT) continue;
            *reinterpret_cast<uint4 *>(&stage[crow[i] * Q8_SEGP + coff[i]]) = reg[i];
        }
    };

    float acc = 0.f;
    int t = first_tile, k = (int)(ua - (int64_t)first_tile * un.upt);
    fetch(t, k);
    commit();
    __syncthreads();
    bool seg_first = k == 0;
    for (int64_t u = ua; u < ub; ++u) {
        const int j = k * Q8_UNIT_BLOCKS + 4 * wave;  // this wave's first block
        const bool active = j < p.nb;                // nb is a multiple of 8: all 4 or none
        const bool last_of_tile = k + 1 == un.upt;
        const int tn = last_of_tile ? t + 1 : t, kn = last_of_tile ? 0 : k + 1;
        const bool more = u + 1 < ub;
        if (more) fetch(tn, kn);
        if (active) {
            const uint8_t *lp = &stage[lane * Q8_SEGP + wave * 4 * Q8_BB];
            uint32_t D[34];
#pragma unroll
            for (int i = 0; i < 17; ++i) {
                const uint2 v = *reinterpret_cast<const uint2 *>(lp + 8 * i);
                D[2 * i] = v.x;
                D[2 * i + 1] = v.y;
            }
            cfloat *xb = as_const(p.x + 32 * (int64_t)j);
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                // block b starts at byte 34 b: d in its first two bytes, the
                // quants after them (2 bytes into a dword for even b)
                const int w0 = (34 * b) >> 2;
                const uint32_t dbits = (b & 1) ? (D[w0] >> 16) : (D[w0] & 0xFFFFu);
                uint32_t q8[8];
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    q8[i] = (b & 1) ? D[w0 + 1 + i]
                                    : __builtin_amdgcn_alignbyte(D[w0 + 1 + i], D[w0 + i], 2);
                const float d = __half2float(__ushort_as_half((unsigned short)dbits));
                acc = fmaf(d, q8_block_dot(q8, xb + 32 * b), acc);
            }
        }
        const bool seg_end = !more || last_of_tile;
        if (seg_end) {
            red[wave][0][lane] = acc;
            acc = 0.f;
        }
        __syncthreads();
        if (seg_end && wave == 0) {
            float tot[1] = {red[0][0][lane]};
#pragma unroll
            for (int w = 1; w < WK; ++w) tot[0] += red[w][0][lane];
            if (seg_first && last_of_tile)
                epilogue<1, 1, EPI_PLAIN>(p, t * 64, lane, tot, 1.f);
            else
                finish_split_tile<1, 1, EPI_PLAIN>(p, un, g, t, t == first_tile ? 0 : 1, lane, tot,
                                                   1.f);
        }
        if (seg_end) seg_first = true;
        t = tn;
        k = kn;
        if (more) commit();
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Q6_K GEMV (one vector).  Q6_K stores 256 weights in 210 bytes (public GGUF
// convention; the six-bit k-quant that q4_k_m files carry next to Q4_K):
// ql[128] (low four bits of the quants), qh[64] (high two bits), sixteen
// int8 scales (one per 16 weights), then a binary16 d.  Weight
// k = 128h + 32c + l takes the low (c < 2) or high (c >= 2) nibble of
// ql[64h + 32(c mod 2) + l] and bits 2c, 2c+1 of qh[32h + l]; with q in 0..63,
// w = d * sc[k/16] * (q - 32).  Per block the kernel forms
//    d * (sum_g sc_g * T_g  -  32 * sum_g sc_g * X_g)
// with T_g = sum(q x) and X_g = sum(x) over the 16 weights of group g.  As
// in the Q4_K kernel, a quant (at most 63) sitting in a 16-bit half is the
// binary16 subnormal q * 2^-24, so each weight costs one v_fma_mix_f32; the
// T_g carry that exact factor, removed once per block.
//
// Same skeleton as the Q4_K kernel: a unit is 64 rows x 4 blocks (one
// 840-byte run per row) and wave w takes block w of every row, one row per
// lane, activations through SGPRs.  A row of K/256 blocks is 8-byte aligned
// when K is a multiple of 1024 (the entry point requires it), so the unit is
// copied in 8-byte chunks; LDS rows are padded to 844 bytes (211 dwords, an
// odd count, so the row-strided dword reads below are conflict-free).  Odd
// blocks start 2 bytes into a dword: a wave reads the 54 aligned dwords
// covering its block and realigns them with one v_alignbit_b32 each.
constexpr int Q6_BB = 210;                       // bytes per block
constexpr int Q6_SEG = WK * Q6_BB;               // 840-byte row run
constexpr int Q6_SEGP = Q6_SEG + 4;              // LDS row stride (211 dwords)
constexpr int Q6_CH_ROW = Q6_SEG / 8;            // 105 eight-byte chunks per row
constexpr int Q6_CH_UNIT = 64 * Q6_CH_ROW;       // 6720 chunks per unit
constexpr int Q6_CH_THREAD = (Q6_CH_UNIT + 64 * WK - 1) / (64 * WK);  // 27 (the last for wave 0 only)
static_assert(Q6_SEG % 8 == 0 && Q6_SEGP % 4 == 0 && (Q6_SEGP / 4) % 2 == 1, "Q6_K staging");
static_assert(Q6_CH_UNIT - (Q6_CH_THREAD - 1) * 64 * WK == 64, "last copy slot = wave 0");

__global__ __launch_bounds__(64 * WK) void gemv_q6_kernel(const GemvParams p, const Units un) {
    __shared__ __attribute__((aligned(16))) uint8_t stage[64 * Q6_SEGP];
    __shared__ float red[WK][1][64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = blockIdx.x;
    const int64_t ua = un.begin(g), ub = un.begin(g + 1);
    if (ua >= ub) return;
    const int first_tile = un.small ? (int)((uint32_t)ua / (uint32_t)un.upt) : (int)(ua / un.upt);

    int crow[Q6_CH_THREAD], coff[Q6_CH_THREAD];
#pragma unroll
    for (int i = 0; i < Q6_CH_THREAD; ++i) {
        const int q = i * 64 * WK + tid;  // past Q6_CH_UNIT only in the last slot (waves 1..3)
        crow[i] = q / Q6_CH_ROW;
        coff[i] = 8 * (q - crow[i] * Q6_CH_ROW);
    }
    uint2 reg[Q6_CH_THREAD];
#pragma unroll
    for (int i = 0; i < Q6_CH_THREAD; ++i) reg[i] = make_uint2(0u, 0u);
    // every unit is whole: K/256 is a multiple of 4
    auto fetch = [&](int t, int k) {
        const int rmax = min(63, p.M - 1 - t * 64);
        const uint8_t *b0 = p.w0 + (int64_t)t * 64 * p.row_bytes + (int64_t)k * Q6_SEG;
#pragma unroll
        for (int i = 0; i < Q6_CH_THREAD; ++i) {
            if (i * 64 * WK + 64 * wave >= Q6_CH_UNIT) continue;  // wave-uniform
            const uint32_t off =
                (uint32_t)min(crow[i], rmax) * (uint32_t)p.row_bytes + (uint32_t)coff[i];
            reg[i] = *reinterpret_cast<const uint2 *>(b0 + off);
        }
    };
    auto commit = [&]() {
#pragma unroll
        for (int i = 0; i < Q6_CH_THREAD; ++i) {
            if (i * 64 * WK + 64 * wave >= Q6_CH_UNIT) continue;
            uint32_t *dst = reinterpret_cast<uint32_t *>(&stage[crow[i] * Q6_SEGP + coff[i]]);
            dst[0] = reg[i].x;  // 4-byte aligned only (odd rows): two dword stores
            dst[1] = reg[i].y;
        }
    };

    float acc = 0.f;
    int t = first_tile, k = (int)(ua - (int64_t)first_tile * un.upt);
    fetch(t, k);
    commit();
    __syncthreads();
    bool seg_first = k == 0;
    for (int64_t u = ua; u < ub; ++u) {
        const int j = k * WK + wave;  // this wave's block
        const bool last_of_tile = k + 1 == un.upt;
        const int tn = last_of_tile ? t + 1 : t, kn = last_of_tile ? 0 : k + 1;
        const bool more = u + 1 < ub;
        if (more) fetch(tn, kn);
        {
            const int off = wave * Q6_BB;  // block start inside the row run
            const uint32_t *lp =
                reinterpret_cast<const uint32_t *>(&stage[lane * Q6_SEGP + (off & ~3)]);
            const int sh = (off & 3) * 8;  // 0 or 16
            uint32_t B[53];
            {
                uint32_t D[54];
#pragma unroll
                for (int i = 0; i < 54; ++i) D[i] = lp[i];
#pragma unroll
                for (int i = 0; i < 53; ++i) B[i] = __builtin_amdgcn_alignbit(D[i + 1], D[i], sh);
            }
            cfloat *xb = as_const(p.x + 256 * (int64_t)j);
            const half2v bias = {(_Float16)-1056.0f, (_Float16)-1056.0f};
            float A = 0.f;
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int c = 0; c < 4; ++c)
#pragma unroll
                    for (int half = 0; half < 2; ++half) {  // group 8h + 2c + half
                        float t0 = 0.f, t1 = 0.f;
#pragma unroll
                        for (int i = 4 * half; i < 4 * half + 4; ++i) {
                            const uint32_t QL = B[16 * h + 8 * (c & 1) + i];
                            const uint32_t QH = B[32 + 8 * h + i];
                            const uint32_t lo = (c < 2 ? QL : QL >> 4) & 0x0F0F0F0Fu;
                            const uint32_t hi = (c < 1 ? QH << 4 : c < 2 ? QH << 2 : c < 3 ? QH : QH >> 2) &
                                                0x30303030u;
                            const uint32_t q4 = lo | hi;  // four six-bit quants, one per byte
                            // bytes 0, 2 and 1, 3 into binary16 halves as
                            // 0x6400 | q = 1024 + q; adding -1056 leaves
                            // q - 32 exactly
                            const half2v q02 =
                                __builtin_bit_cast(half2v, and_or(q4, 0x00FF00FFu, 0x64006400u)) + bias;
                            const half2v q13 =
                                __builtin_bit_cast(half2v, and_or(q4 >> 8, 0x00FF00FFu, 0x64006400u)) + bias;
                            const int kx = 128 * h + 32 * c + 4 * i;
                            t0 = fmaf((float)q02.x, xb[kx + 0], t0);
                            t1 = fmaf((float)q13.x, xb[kx + 1], t1);
                            t0 = fmaf((float)q02.y, xb[kx + 2], t0);
                            t1 = fmaf((float)q13.y, xb[kx + 3], t1);
                        }
                        const int grp = 8 * h + 2 * c + half;
                        const float scg =
                            (float)(int8_t)((B[48 + (grp >> 2)] >> (8 * (grp & 3))) & 0xFFu);
                        A = fmaf(scg, t0 + t1, A);
                    }
            const float d = __half2float(__ushort_as_half((unsigned short)(B[52] & 0xFFFFu)));
            acc = fmaf(d, A, acc);
        }
        const bool seg_end = !more || last_of_tile;
        if (seg_end) {
            red[wave][0][lane] = acc;
            acc = 0.f;
        }
        __syncthreads();
        if (seg_end && wave == 0) {
            float tot[1] = {red[0][0][lane]};
#pragma unroll
            for (int w = 1; w < WK; ++w) tot[0] += red[w][0][lane];
            if (seg_first && last_of_tile)
                epilogue<1, 1, EPI_PLAIN>(p, t * 64, lane, tot, 1.f);
            else
                finish_split_tile<1, 1, EPI_PLAIN>(p, un, g, t, t == first_tile ? 0 : 1, lane, tot,
                                                   1.f);
        }
        if (seg_end) seg_first = true;
        t = tn;
        k = kn;
        if (more) commit();
        __syncthreads();
    }
}

// xg[i] = x[i] * (1 + w[i]) (w null: xg not written) and the sums of squares
// of x per 32 elements, one element per thread.
__global__ __launch_bounds__(64) void norm_gain_kernel(const float *__restrict__ x,
                                                       const float *__restrict__ w, int64_t n,
                                                       float *__restrict__ xg,
                                                       float *__restrict__ sq) {
    const int64_t i = (int64_t)blockIdx.x * 64 + threadIdx.x;
    const float a = i < n ? x[i] : 0.f;
    if (w && i < n) xg[i] = a * (1.0f + w[i]);
    float s = a * a;
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 8);
    s += __shfl_xor(s, 4);
    s += __shfl_xor(s, 2);
    s += __shfl_xor(s, 1);
    const int64_t granule = (int64_t)blockIdx.x * 2 + (threadIdx.x >> 5);
    if ((threadIdx.x & 31) == 0 && granule * 32 < n) sq[granule] = s;
}

std::atomic<int> g_override_groups{0};

// Resident workgroups of each kernel instance on a device (occupancy queries
// are not free, so they are cached).
std::mutex g_occ_mutex;
std::map<std::pair<int, const void *>, std::pair<int, int>> g_occ;  // -> (resident groups, CUs)

int resident_groups(const void *fn, int *out, int *cus_out) {
    int dev = 0;
    Q4K_HIP(hipGetDevice(&dev));
    std::lock_guard<std::mutex> lock(g_occ_mutex);
    auto key = std::make_pair(dev, fn);
    auto it = g_occ.find(key);
    if (it == g_occ.end()) {
        int per_cu = 0, cus = 0;
        Q4K_HIP(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 64 * WK, 0));
        Q4K_HIP(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
        it = g_occ.emplace(key, std::make_pair(std::max(1, per_cu) * std::max(1, cus),
                                               std::max(1, cus))).first;
    }
    *out = it->second.first;
    *cus_out = it->second.second;
    return Q4K_OK;
}

int64_t units_of(int64_t M, int64_t K, int nmat) {
    const int64_t rows = 64 / nmat;
    return ((M + rows - 1) / rows) * ((K / 256 + WK - 1) / WK);
}

// Workgroup count: every resident slot, at most two workgroups per CU, each
// taking a contiguous range of units; tiles cut by a range boundary are
// finished in-kernel by their last contributor.  On the 50 MB MLP matrices
// two workgroups per CU measured 16.6-17.2 us against 17.8-19.1 us at three
// and 18.3-20.0 us at four, and every count from 384 to 640 workgroups was
// slower than 512; on the 715 MB lm_head two per CU took 134.6 us against
// 138.0 at three and 152.7 at four (interleaved runs).  One tile per
// workgroup (no cut tiles) was slower still.
// Four, eight and sixteen plain vectors run on the matrix cores: four and
// eight on the f32 4x4x1 form, sixteen on bf16 16x16x32 instructions with
// split operands (17408x5120: 42.8 us against 58.4-59.1 on the f32 16x16x4
// form and 68.0 on the 4x4x1 one).  For eight vectors the split kernel,
// whose instructions then idle half their columns, measured only 2-3%
// faster than the 4x4x1 one (37.2-38.1 against 38.5-39.5 us), so eight
// keep the f32 products.
template <int NV, int NMAT, int EPI>
constexpr bool kMfma = NMAT == 1 && EPI == EPI_PLAIN && (NV == 4 || NV == 8 || NV == 16);
template <int NV>
constexpr bool kSplit = NV == 16;

template <int NV, int NMAT, int EPI>
const void *gemv_fn() {
    if constexpr (kMfma<NV, NMAT, EPI>) {
        if constexpr (kSplit<NV>) return (const void *)gemv_split_kernel<NV>;
        else return (const void *)gemv_mfma_kernel<NV>;
    } else {
        return (const void *)gemv_kernel<NV, NMAT, EPI>;
    }
}

template <int NV, int NMAT, int EPI>
int groups_for(int64_t M, int64_t K, int *G) {
    int res = 0, cus = 0;
    const int o = g_override_groups.load();
    int64_t g = o;
    if (o <= 0) {
        int rc = resident_groups(gemv_fn<NV, NMAT, EPI>(), &res, &cus);
        if (rc) return rc;
        g = std::min(res, 2 * cus);
    }
    *G = (int)std::max<int64_t>(1, std::min<int64_t>(g, units_of(M, K, NMAT)));
    return Q4K_OK;
}

// The unit partition of a launch (what the kernels receive): tiles of
// 64 / nmat rows, units of bpu blocks of a tile's rows.
Units make_units(int64_t M, int64_t nb, int nmat, int64_t groups, int bpu = WK) {
    const int64_t rows = 64 / nmat;
    const int64_t tiles = (M + rows - 1) / rows;
    Units un;
    un.upt = (int)((nb + bpu - 1) / bpu);
    un.U = tiles * un.upt;
    un.G = (int)std::max<int64_t>(1, std::min<int64_t>(groups, un.U));
    un.small = (un.U + 1) * (int64_t)un.G + un.U < ((int64_t)1 << 32);
    return un;
}

template <int NV, int NMAT, int EPI>
int launch_t(const GemvParams &p, const GemvLaunch &L, hipStream_t stream) {
    constexpr int ROWS = 64 / NMAT;
    const int64_t tiles = (p.M + ROWS - 1) / ROWS;
    const Units un = make_units(p.M, p.nb, NMAT, L.ks);
    if (tiles > 0x7FFFFFFF) return fail(Q4K_EUNSUPPORTED, "gemv: too many rows");
    if constexpr (kMfma<NV, NMAT, EPI>) {
        if constexpr (kSplit<NV>)
            hipLaunchKernelGGL((gemv_split_kernel<NV>), dim3((unsigned)un.G), dim3(64 * WK), 0,
                               stream, p, un);
        else
            hipLaunchKernelGGL((gemv_mfma_kernel<NV>), dim3((unsigned)un.G), dim3(64 * WK), 0,
                               stream, p, un);
    } else
        hipLaunchKernelGGL((gemv_kernel<NV, NMAT, EPI>), dim3((unsigned)un.G), dim3(64 * WK), 0,
                           stream, p, un);
    Q4K_HIP(hipGetLastError());
    return Q4K_OK;
}

}  // namespace

void set_gemv_override(int groups) { g_override_groups = groups; }

GemvLaunch choose_gemv_launch(int64_t M, int64_t K, int nv, int nmat, int epi) {
    GemvLaunch L;
    L.wk = WK;
    int G = 0;
    int rc;
    if (nmat == 2) rc = groups_for<1, 2, EPI_SWIGLU>(M, K, &G);
    else if (epi == EPI_SCALE) rc = groups_for<1, 1, EPI_SCALE>(M, K, &G);
    else if (epi == EPI_RESID) rc = groups_for<1, 1, EPI_RESID>(M, K, &G);
    else if (nv >= 16) rc = groups_for<16, 1, EPI_PLAIN>(M, K, &G);
    else if (nv >= 8) rc = groups_for<8, 1, EPI_PLAIN>(M, K, &G);
    else if (nv >= 4) rc = groups_for<4, 1, EPI_PLAIN>(M, K, &G);
    else if (nv >= 2) rc = groups_for<2, 1, EPI_PLAIN>(M, K, &G);
    else rc = groups_for<1, 1, EPI_PLAIN>(M, K, &G);
    if (rc != Q4K_OK || G < 1) {
        // no device to query (e.g. host-only callers): assume 4 workgroups per CU, 256 CUs
        clear_error();
        const int o = g_override_groups.load();
        G = (int)std::max<int64_t>(1, std::min<int64_t>(o > 0 ? o : 1024, units_of(M, K, nmat)));
    }
    L.ks = G;
    return L;
}

size_t gemv_partial_floats(const GemvLaunch &L, int nv) {
    return (size_t)L.ks * 2 * (size_t)nv * 64;
}

size_t gemv_counters(const GemvLaunch &L) { return (size_t)L.ks; }

// Host-side check of a GEMV launch's partition, with the kernels' own range
// and owner arithmetic (Units): contiguous non-empty ranges covering every
// unit once; each tile cut between workgroups has consecutive contributors
// gf..gl that all hold some of its units, gf first-contributes to no other
// cut tile (its counter is the tile's), and every partial slot and counter
// index lies inside the workspace the launch reserves; the weight bytes the
// first and last unit of every range fetch (rows clamped to M - 1, blocks
// past the row end re-reading the unit's first block) stay inside the
// matrix, with 32-bit lane offsets that do not wrap.
namespace {
int check_units(int64_t M, int64_t nb, int64_t block_bytes, int bpu, int nmat, int nvk,
                int64_t groups) {
    const int64_t row_bytes = nb * block_bytes, rows = 64 / nmat;
    const Units un = make_units(M, nb, nmat, groups, bpu);
    const int G = un.G;
    const size_t partial_floats = gemv_partial_floats(GemvLaunch{WK, G}, nvk);
    if (gemv_counters(GemvLaunch{WK, G}) > kMaxCounters)
        return fail(Q4K_EINVAL, "check: %d workgroups exceed the counter region", G);
    if (un.small && (un.U + 1) * (int64_t)G + un.U >= ((int64_t)1 << 32))
        return fail(Q4K_EINVAL, "check: 32-bit range arithmetic would wrap");
    std::vector<int> first_of(G, 0);
    int64_t prev = 0;
    for (int g = 0; g < G; ++g) {
        const int64_t ua = un.begin(g), ub = un.begin(g + 1);
        if (ua != prev || ub <= ua)
            return fail(Q4K_EINVAL, "check: range of workgroup %d is [%lld, %lld)", g,
                        (long long)ua, (long long)ub);
        prev = ub;
        if (un.owner(ua) != g || un.owner(ub - 1) != g)
            return fail(Q4K_EINVAL, "check: owner() disagrees with begin() at workgroup %d", g);
        const int64_t ft = ua / un.upt, lt = (ub - 1) / un.upt;
        const int64_t tl[2] = {ft, lt};
        for (int slot = 0; slot < (ft == lt ? 1 : 2); ++slot) {
            const int64_t t = tl[slot];
            const int64_t t0u = t * un.upt, t1u = t0u + un.upt - 1;
            const bool cut = un.owner(t0u) != un.owner(t1u);
            if ((((int64_t)g * 2 + slot) * nvk + nvk) * 64 > (int64_t)partial_floats)
                return fail(Q4K_EINVAL, "check: partial slot of workgroup %d outside", g);
            if (!cut) continue;
            const int gf = un.owner(t0u), gl = un.owner(t1u);
            for (int w = gf; w <= gl; ++w)
                if (un.begin(w) > t1u || un.begin(w + 1) <= t0u)
                    return fail(Q4K_EINVAL, "check: workgroup %d holds none of cut tile %lld", w,
                                (long long)t);
            if (g == gf && ++first_of[gf] > 1)
                return fail(Q4K_EINVAL, "check: workgroup %d first-contributes to two cut tiles", gf);
        }
        for (int64_t u : {ua, ub - 1}) {
            const int64_t t = u / un.upt, k = u % un.upt, j0 = k * bpu;
            const int64_t rmax = std::min<int64_t>(rows - 1, M - 1 - t * rows);
            const int64_t valid = std::min<int64_t>(bpu, nb - j0) * block_bytes;
            const int64_t base = t * rows * row_bytes + j0 * block_bytes;
            const int64_t lane_max = rmax * row_bytes + valid;  // one past the last byte
            if (rmax < 0 || valid <= 0 || base + lane_max > M * row_bytes)
                return fail(Q4K_EINVAL, "check: unit %lld fetches outside the matrix",
                            (long long)u);
            if (lane_max > ((int64_t)1 << 32))
                return fail(Q4K_EINVAL, "check: 32-bit lane offset wraps at unit %lld",
                            (long long)u);
        }
    }
    if (prev != un.U) return fail(Q4K_EINVAL, "check: ranges end at %lld of %lld units",
                                  (long long)prev, (long long)un.U);
    return Q4K_OK;
}
}  // namespace

int check_gemv_partition(int64_t M, int64_t K, int nv, int nmat, int groups) {
    if (M <= 0 || K <= 0 || K % 256 != 0 || (nmat != 1 && nmat != 2) || nv < 1)
        return fail(Q4K_EINVAL, "check: bad arguments");
    GemvLaunch L = choose_gemv_launch(M, K, nv, nmat, nmat == 2 ? EPI_SWIGLU : EPI_PLAIN);
    if (groups > 0) L.ks = groups;
    const int nvk = nmat == 2 ? 1 : nv >= 16 ? 16 : nv >= 8 ? 8 : nv >= 4 ? 4 : nv >= 2 ? 2 : 1;
    return check_units(M, K / 256, kBlockBytes, WK, nmat, nvk, L.ks);
}

int check_gemv_q8_partition(int64_t M, int64_t K, int groups) {
    if (M <= 0 || K <= 0 || K % 32 != 0) return fail(Q4K_EINVAL, "check: bad arguments");
    GemvLaunch L = choose_gemv_q8_launch(M, K);
    if (groups > 0) L.ks = groups;
    return check_units(M, K / 32, Q8_BB, Q8_UNIT_BLOCKS, 1, 1, L.ks);
}

int check_gemv_q6_partition(int64_t M, int64_t K, int groups) {
    if (M <= 0 || K <= 0 || K % 1024 != 0) return fail(Q4K_EINVAL, "check: bad arguments");
    GemvLaunch L = choose_gemv_q6_launch(M, K);
    if (groups > 0) L.ks = groups;
    return check_units(M, K / 256, Q6_BB, WK, 1, 1, L.ks);
}

int launch_gemv(const GemvParams &p, int nv, int nmat, int epi, const GemvLaunch &L,
                hipStream_t stream) {
    if (nmat == 1 && epi == EPI_PLAIN) {
        switch (nv) {
            case 1: return launch_t<1, 1, EPI_PLAIN>(p, L, stream);
            case 2: return launch_t<2, 1, EPI_PLAIN>(p, L, stream);
            case 4: return launch_t<4, 1, EPI_PLAIN>(p, L, stream);
            case 8: return launch_t<8, 1, EPI_PLAIN>(p, L, stream);
            case 16: return launch_t<16, 1, EPI_PLAIN>(p, L, stream);
            default: return fail(Q4K_EINVAL, "unsupported vector count %d", nv);
        }
    }
    if (nv != 1) return fail(Q4K_EINVAL, "fused epilogues take one vector");
    if (nmat == 1 && epi == EPI_SCALE) return launch_t<1, 1, EPI_SCALE>(p, L, stream);
    if (nmat == 1 && epi == EPI_RESID) return launch_t<1, 1, EPI_RESID>(p, L, stream);
    if (nmat == 2 && epi == EPI_SWIGLU) return launch_t<1, 2, EPI_SWIGLU>(p, L, stream);
    return fail(Q4K_EINVAL, "unsupported GEMV variant");
}

GemvLaunch choose_gemv_q8_launch(int64_t M, int64_t K) {
    GemvLaunch L;
    L.wk = WK;
    const int64_t units = ((M + 63) / 64) * ((K / 32 + Q8_UNIT_BLOCKS - 1) / Q8_UNIT_BLOCKS);
    int G = g_override_groups.load(), res = 0, cus = 0;
    if (G <= 0) {
        // at most three workgroups per CU: on the 1.35 GB lm_head 241.6 us
        // against 256.2 at two, 249.3 at four and 278.5 at five (every
        // resident slot), interleaved runs
        if (resident_groups((const void *)gemv_q8_kernel, &res, &cus) == Q4K_OK)
            G = std::min(res, 3 * cus);
        else {
            clear_error();
            G = 1024;
        }
    }
    L.ks = (int)std::max<int64_t>(1, std::min<int64_t>(G, units));
    return L;
}

int launch_gemv_q8(const GemvParams &p, const GemvLaunch &L, hipStream_t stream) {
    const int64_t tiles = (p.M + 63) / 64;
    const Units un = make_units(p.M, p.nb, 1, L.ks, Q8_UNIT_BLOCKS);
    if (tiles > 0x7FFFFFFF) return fail(Q4K_EUNSUPPORTED, "gemv: too many rows");
    hipLaunchKernelGGL(gemv_q8_kernel, dim3((unsigned)un.G), dim3(64 * WK), 0, stream, p, un);
    Q4K_HIP(hipGetLastError());
    return Q4K_OK;
}

GemvLaunch choose_gemv_q6_launch(int64_t M, int64_t K) {
    GemvLaunch L;
    L.wk = WK;
    const int64_t units = ((M + 63) / 64) * (K / 256 / WK);
    int G = g_override_groups.load(), res = 0, cus = 0;
    if (G <= 0) {
        if (resident_groups((const void *)gemv_q6_kernel, &res, &cus) == Q4K_OK)
            G = std::min(res, 2 * cus);
        else {
            clear_error();
            G = 512;
        }
    }
    L.ks = (int)std::max<int64_t>(1, std::min<int64_t>(G, units));
    return L;
}

int launch_gemv_q6(const GemvParams &p, const GemvLaunch &L, hipStream_t stream) {
    const int64_t tiles = (p.M + 63) / 64;
    if (p.nb % WK != 0) return fail(Q4K_ESHAPE, "gemv_q6_k: K must be a multiple of 1024");
    const Units un = make_units(p.M, p.nb, 1, L.ks);  // nb is a multiple of WK
    if (tiles > 0x7FFFFFFF) return fail(Q4K_EUNSUPPORTED, "gemv: too many rows");
    hipLaunchKernelGGL(gemv_q6_kernel, dim3((unsigned)un.G), dim3(64 * WK), 0, stream, p, un);
    Q4K_HIP(hipGetLastError());
    return Q4K_OK;
}

int stack_groups(int *G) {
    int res = 0, cus = 0;
    int rc = resident_groups((const void *)stack_kernel, &res, &cus);
    if (rc) return rc;
    *G = std::max(1, std::min(res, 2 * cus));
    return Q4K_OK;
}

size_t stack_node_bytes() { return sizeof(StackNode); }

int fill_stack_node(void *dst, const GemvParams &p, int nmat, int epi, int G) {
    StackNode nd;
    nd.p = p;
    const int rows = 64 / nmat;
    const int64_t tiles = (p.M + rows - 1) / rows;
    if (tiles > 0x7FFFFFFF) return fail(Q4K_EUNSUPPORTED, "stack node: too many rows");
    nd.un.upt = (p.nb + WK - 1) / WK;
    nd.un.U = tiles * nd.un.upt;
    nd.un.G = (int)std::min<int64_t>(G, nd.un.U);
    nd.un.small = (nd.un.U + 1) * (int64_t)nd.un.G + nd.un.U < ((int64_t)1 << 32);
    nd.nmat = nmat;
    nd.epi = epi;
    memcpy(dst, &nd, sizeof nd);
    return Q4K_OK;
}

int launch_stack_kernel(const void *nodes, int n_nodes, unsigned *done, unsigned epoch,
                        unsigned *err, int spin_limit, int G, hipStream_t stream) {
    void *args[] = {(void *)&nodes, (void *)&n_nodes, (void *)&done, (void *)&epoch,
                    (void *)&err, (void *)&spin_limit};
    Q4K_HIP(hipLaunchCooperativeKernel((const void *)stack_kernel, dim3((unsigned)G),
                                       dim3(64 * WK), args, 0, stream));
    return Q4K_OK;
}

int launch_norm_gain(const float *x, const float *w, int64_t n, float *xg, float *sq,
                     hipStream_t stream) {
    const unsigned blocks = (unsigned)((n + 63) / 64);
    if (!blocks) return Q4K_OK;
    hipLaunchKernelGGL(norm_gain_kernel, dim3(blocks), dim3(64), 0, stream, x, w, n, xg, sq);
    Q4K_HIP(hipGetLastError());
    return Q4K_OK;
}

int launch_sumsq(const float *v, int64_t n, float *out, hipStream_t stream) {
    const unsigned blocks = (unsigned)((n + 63) / 64);
    if (!blocks) return Q4K_OK;
    hipLaunchKernelGGL(sumsq_kernel, dim3(blocks), dim3(64), 0, stream, v, n, out);
    Q4K_HIP(hipGetLastError());
    return Q4K_OK;
}

}  // namespace q4k
